"""GPU parity of the expert-balance telemetry (moe_bias_update_stats) against
the oracle.  The "Relay training" section of the article watches the
dead-expert fraction (top-2 paragraph) and shows expert balance on the
training dashboard (baton paragraph).

The bias is compared bit-exactly with the plain bias step; the four figures in
float32 against the oracle's float64 (dead fraction exactly, the others within
a relative 1e-5: one division, 64 logarithms and a 64-term sum in float32).
"""
import numpy as np
import pytest

import oracle.moe_oracle as om
from fine_grained_moe_amd import synth
from tests import _helpers as H

pytestmark = pytest.mark.gpu

GAMMA = 1e-3


def _check_stats(got, counts, total):
    want = om.load_stats(counts, total)
    assert got[0] == np.float32(want[0]), (got, want)
    np.testing.assert_allclose(got[1:], want[1:], rtol=1e-5, atol=1e-6)


def test_stats_after_the_layer_forward():
    """One forward of the 4096-token layer, then the bias step with telemetry:
    same bias bits as the plain step, figures as the oracle's."""
    import torch
    from fine_grained_moe_amd import moe
    inp = synth.make_workload("layer_t4096")
    H.remove_near_ties(inp)
    y, rn, dev = H.run_forward(inp)
    _, r_ref = H.oracle_forward(inp)
    H.check_routing_exact(rn, r_ref, inp.E)
    total = inp.T * inp.k
    b_plain = dev["b"].clone()
    moe.moe_bias_update(inp.E, total, dev["r"]["counts"], GAMMA, b_plain)
    stats = torch.full((4,), float("nan"), device="cuda")
    moe.moe_bias_update_stats(inp.E, total, dev["r"]["counts"], GAMMA, dev["b"], stats)
    torch.cuda.synchronize()
    assert dev["b"].cpu().numpy().view(np.uint32).tolist() == b_plain.cpu().numpy().view(np.uint32).tolist()
    got = stats.cpu().numpy()
    print(f"balance after the layer forward: {got.tolist()}", flush=True)
    _check_stats(got, rn["counts"], total)


@pytest.mark.parametrize("case", ["uniform", "one_hot", "two_of_eight", "empty", "one_expert", "ragged_E"])
def test_stats_closed_forms(case):
    """Loads with closed-form figures, written straight into the counts."""
    import torch
    from fine_grained_moe_amd import moe
    if case == "uniform":
        c = np.full(64, 128)
    elif case == "one_hot":
        c = np.zeros(64, np.int64)
        c[40] = 8192
    elif case == "two_of_eight":
        c = np.array([0, 50, 0, 0, 50, 0, 0, 0])
    elif case == "empty":
        c = np.zeros(16, np.int64)
    elif case == "one_expert":
        c = np.array([77])
    else:
        c = np.random.default_rng(3).integers(0, 40, size=37)
    total = int(c.sum())
    counts = torch.from_numpy(c.astype(np.int32)).cuda()
    bias = torch.zeros(c.size, device="cuda")
    stats = torch.full((4,), float("nan"), device="cuda")
    moe.moe_bias_update_stats(c.size, total, counts, GAMMA, bias, stats)
    torch.cuda.synchronize()
    _check_stats(stats.cpu().numpy(), c, total)
    want_b = om.bias_update(np.zeros(c.size, np.float32), c, total, GAMMA)
    assert bias.cpu().numpy().view(np.uint32).tolist() == want_b.view(np.uint32).tolist()


@pytest.mark.slow
def test_ten_step_balancing_loop_without_host_sync():
    """Skewed routing (Zipf(1) expected loads), 10 route + bias-step-with-
    telemetry steps on the same batch, each writing its row of a [10, 4]
    buffer with no host synchronisation in between; afterwards every row and
    the final bias against the oracle's sequence."""
    import torch
    from fine_grained_moe_amd import moe
    inp = synth.make_workload("zipf_t16384")
    for _ in range(3):   # the preset depends on x; redraw until stable
        b0 = H.zipf_bias(inp)
        if H.remove_near_ties(inp, bias_states=[b0], steps_after=10) == 0:
            break
    states = H.bias_sequence(inp, b0, 10)
    x, w = H.to_gpu(inp)
    dims = moe.make_dims(inp.T, inp.d, inp.E, inp.F, inp.Fs, inp.k, inp.act)
    b = torch.from_numpy(b0.copy()).cuda()
    r = moe.alloc_routing(dims)
    ws = moe.alloc_workspace(dims)
    stats = torch.full((10, 4), float("nan"), device="cuda")
    total = inp.T * inp.k
    for step in range(10):
        moe.moe_route(dims, x, w["w_router"], b, r, ws)
        moe.moe_bias_update_stats(inp.E, total, r["counts"], GAMMA, b, stats[step])
    torch.cuda.synchronize()
    assert b.cpu().numpy().view(np.uint32).tolist() == states[10].view(np.uint32).tolist()
    got = stats.cpu().numpy()
    for step in range(10):
        counts = om.expert_counts(om.route(inp.x, inp.w_router, states[step], inp.k).idx, inp.E)
        _check_stats(got[step], counts, total)
    print(f"zipf balance, step 0: {got[0].tolist()}, step 9: {got[9].tolist()}", flush=True)
    assert got[0][1] > 10.0            # the hottest expert holds ~20% of assignments: ~13x the mean


def _fused_vs_separate(dims, x, w, b0, with_stats=True):
    """moe_forward + moe_bias_update_stats against moe_forward_bias_step from
    the same bias: y, routing, the new bias and the figures bit for bit."""
    import torch
    from fine_grained_moe_amd import moe
    T, E, k = dims.T, dims.E, dims.k
    outs = []
    for fused in (False, True):
        bias = b0.clone()
        y = torch.empty_like(x)
        r = moe.alloc_routing(dims)
        ws = moe.alloc_workspace(dims)
        st = torch.full((4,), -7.0, device="cuda") if with_stats else None
        if fused:
            moe.moe_forward_bias_step(dims, x, w, bias, GAMMA, st, y, r, ws)
        else:
            moe.moe_forward(dims, x, w, bias, y, r, ws)
            if with_stats:
                moe.moe_bias_update_stats(E, T * k, r["counts"], GAMMA, bias, st)
            else:
                moe.moe_bias_update(E, T * k, r["counts"], GAMMA, bias)
        torch.cuda.synchronize()
        outs.append((y, r, bias, st))
    (y0, r0, b_0, s0), (y1, r1, b_1, s1) = outs
    assert torch.equal(y0, y1)
    for n in r0:
        assert torch.equal(r0[n], r1[n]), n
    assert torch.equal(b_0.view(torch.int32), b_1.view(torch.int32))
    assert not torch.equal(b_1, b0) or T == 0
    if with_stats:
        assert torch.equal(s0.view(torch.int32), s1.view(torch.int32))
        _check_stats(s1.cpu().numpy(), r1["counts"].cpu().numpy(), T * k)
    return r1


@pytest.mark.parametrize("case", ["layer_t4096", "tiny_f32", "empty", "no_stats"])
def test_fused_bias_step_bitwise(case):
    import torch
    from fine_grained_moe_amd import moe
    name = "tiny_f32" if case == "tiny_f32" else "layer_t4096"
    T = 0 if case == "empty" else (1500 if case == "no_stats" else None)
    inp = synth.make_workload(name, T=T) if T is not None else synth.make_workload(name)
    x, w = H.to_gpu(inp)
    dims = moe.make_dims(inp.T, inp.d, inp.E, inp.F, inp.Fs, inp.k, inp.act)
    b0 = torch.from_numpy(np.linspace(-0.01, 0.01, inp.E).astype(np.float32)).cuda()
    _fused_vs_separate(dims, x, w, b0, with_stats=case != "no_stats")


@pytest.mark.parametrize("T", [8, 300])
def test_fused_bias_step_int4(T):
    """The int4 top-1 layer: the decode (T <= 64: the bias step stays a launch
    of its own) and the prefill (the dispatch launch takes it)."""
    import torch
    from fine_grained_moe_amd import moe
    base = synth.make_layer(T=T, d=1024, E=64, F=512, Fs=2048, k=1, act="bf16", seed=77)
    qg, sg = om.quantize_int4(base.w_gate_up)
    qd, sd = om.quantize_int4(base.w_down)

    def bf(a):
        return torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(device="cuda", dtype=torch.bfloat16)

    w = dict(w_router=bf(base.w_router), w_gate_up=torch.from_numpy(qg).cuda(), s_gate_up=bf(sg),
             w_down=torch.from_numpy(qd).cuda(), s_down=bf(sd), w_sh_gate_up=bf(base.w_sh_gate_up),
             w_sh_down=bf(base.w_sh_down))
    dims = moe.make_dims(T, 1024, 64, 512, 2048, 1, "bf16", w_routed="int4")
    _fused_vs_separate(dims, bf(base.x), w, torch.zeros(64, device="cuda"))
