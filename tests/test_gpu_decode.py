"""GPU parity of the top-1 serving path with int4 routed experts.

The routed experts are N(0, 0.02) weights quantised by the oracle's int4
encoder (symmetric, groups of 128, bf16 scales); both sides read the same
packed bytes and scales.  Routing is compared bit-exactly (gate exactly 1),
y within relative Frobenius error 1e-2.
"""
import numpy as np
import pytest

import oracle.moe_oracle as om
from fine_grained_moe_amd import synth
from tests import _helpers as H

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def weights():
    import torch
    base = synth.make_layer(T=1, d=1024, E=64, F=512, Fs=2048, k=1, act="bf16", seed=7)
    qg, sg = om.quantize_int4(base.w_gate_up)
    qd, sd = om.quantize_int4(base.w_down)

    def bf(a):
        return torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(device="cuda", dtype=torch.bfloat16)

    dev = dict(w_router=bf(base.w_router), w_gate_up=torch.from_numpy(qg).cuda(), s_gate_up=bf(sg),
               w_down=torch.from_numpy(qd).cuda(), s_down=bf(sd),
               w_sh_gate_up=bf(base.w_sh_gate_up), w_sh_down=bf(base.w_sh_down))
    host = dict(base=base, qg=qg, sg=sg, qd=qd, sd=sd)
    return dev, host


def _run(weights, T, seed, bias=None):
    import torch
    from fine_grained_moe_amd import moe
    dev, host = weights
    base = host["base"]
    inp = synth.make_layer(T=T, d=1024, E=64, F=512, Fs=2048, k=1, act="bf16", seed=seed)
    inp.w_router = base.w_router
    b = np.zeros(64, np.float32) if bias is None else np.asarray(bias, np.float32)
    if T:
        H.remove_near_ties(inp, bias_states=[b])
    dims = moe.make_dims(T, 1024, 64, 512, 2048, 1, "bf16", w_routed="int4")
    x = torch.from_numpy(inp.x).to(device="cuda", dtype=torch.bfloat16)
    y = torch.empty_like(x)
    r = moe.alloc_routing(dims)
    ws = moe.alloc_workspace(dims)
    bt = torch.from_numpy(b).cuda()
    moe.moe_forward(dims, x, dev, bt, y, r, ws)
    torch.cuda.synchronize()
    rn = {k: v.cpu().numpy() for k, v in r.items()}
    y_ref, ref = om.forward_int4_top1(inp.x, base.w_router, host["qg"], host["sg"], host["qd"], host["sd"],
                                      base.w_sh_gate_up, base.w_sh_down, b)
    return y.float().cpu().numpy(), rn, y_ref, ref


@pytest.mark.parametrize("T", [1, 8, 13, 16, 17, 33, 48, 63, 64])
def test_int4_top1_decode(weights, T):
    y, rn, y_ref, ref = _run(weights, T, seed=100 + T)
    H.check_routing_exact(rn, ref, 64)
    assert np.all(rn["gate"] == 1.0)
    H.check_close(y, y_ref, "bf16", f"decode T={T} ({np.count_nonzero(rn['counts'])} active experts) y:")


def test_int4_decode_all_tokens_one_expert(weights):
    bias = np.zeros(64, np.float32)
    bias[37] = 5.0
    y, rn, y_ref, ref = _run(weights, 64, seed=3, bias=bias)
    assert np.all(rn["idx"] == 37) and rn["counts"][37] == 64
    H.check_routing_exact(rn, ref, 64)
    assert H.rel_fro(y, y_ref) <= 1e-2


def test_int4_decode_empty_batch(weights):
    import torch
    from fine_grained_moe_amd import moe
    dev, _ = weights
    dims = moe.make_dims(0, 1024, 64, 512, 2048, 1, "bf16", w_routed="int4")
    x = torch.empty(0, 1024, dtype=torch.bfloat16, device="cuda")
    r = moe.alloc_routing(dims)
    r["counts"].fill_(3)
    moe.moe_forward(dims, x, dev, torch.zeros(64, device="cuda"), torch.empty_like(x), r, moe.alloc_workspace(dims))
    torch.cuda.synchronize()
    assert torch.all(r["counts"] == 0) and torch.all(r["offsets"] == 0)


def test_int4_rejects_unsupported_shapes():
    from fine_grained_moe_amd import moe
    assert moe.moe_workspace_bytes(moe.make_dims(8, 1024, 64, 512, 2048, 2, "bf16", w_routed="int4")) == 0
    assert moe.moe_workspace_bytes(moe.make_dims(8, 1024, 64, 512, 2048, 1, "bf16", w_routed="int4")) > 0


def test_int4_decode_graph_replay_matches_eager(weights):
    """The serving forward captured in a HIP graph gives, on every replay,
    exactly the eager result (bitwise), with other eager work and host
    synchronisations between the replays."""
    import torch
    from fine_grained_moe_amd import moe
    dev, _ = weights
    T = 8
    inp = synth.make_layer(T=T, d=1024, E=64, F=512, Fs=2048, k=1, act="bf16", seed=55)
    dims = moe.make_dims(T, 1024, 64, 512, 2048, 1, "bf16", w_routed="int4")
    x = torch.from_numpy(inp.x).to(device="cuda", dtype=torch.bfloat16)
    bias = torch.zeros(64, device="cuda")
    y_eager, r_eager, ws_eager = torch.empty_like(x), moe.alloc_routing(dims), moe.alloc_workspace(dims)
    moe.moe_forward(dims, x, dev, bias, y_eager, r_eager, ws_eager)
    torch.cuda.synchronize()
    y, r, ws = torch.empty_like(x), moe.alloc_routing(dims), moe.alloc_workspace(dims)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        moe.moe_forward(dims, x, dev, bias, y, r, ws)
    other = torch.roll(x, 1, 0).contiguous()
    y_other = torch.empty_like(x)
    for rep in range(3):
        y.fill_(0)
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y, y_eager), rep
        for n in ("idx", "gate", "counts", "offsets", "perm", "pos"):
            assert torch.equal(r[n], r_eager[n]), (rep, n)
        # eager work between replays, on the same weights and its own buffers
        moe.moe_forward(dims, other, dev, bias, y_other, moe.alloc_routing(dims), moe.alloc_workspace(dims))
        torch.cuda.synchronize()


@pytest.mark.parametrize("T", [1, 8, 16, 17, 64])
def test_next_layer_hint_changes_no_bits(weights, T):
    """The next-layer prefetch hint (moe_weights.next) only moves the next
    layer's router and shared gate/up rows into the caches: y and the routing
    are bitwise those of the call without it, for the layer forward and the
    MoE block, and the hinted layer's own call is unchanged too."""
    import torch
    from fine_grained_moe_amd import moe
    dev, _ = weights
    other = {n: (t.flip(0).contiguous() if n in ("w_router", "w_sh_gate_up") else t) for n, t in dev.items()}
    inp = synth.make_layer(T=T, d=1024, E=64, F=512, Fs=2048, k=1, act="bf16", seed=300 + T)
    dims = moe.make_dims(T, 1024, 64, 512, 2048, 1, "bf16", w_routed="int4")
    x = torch.from_numpy(inp.x).to(device="cuda", dtype=torch.bfloat16)
    bias = torch.zeros(64, device="cuda")
    ws = moe.alloc_workspace(dims)
    gw = torch.ones(1024, device="cuda")
    outs = []
    for w in (dev, dict(dev, next=other), dict(dev, next=dev)):
        y = torch.empty_like(x)
        r = moe.alloc_routing(dims)
        moe.moe_forward(dims, x, w, bias, y, r, ws)
        hb = torch.empty_like(x)
        rb = moe.alloc_routing(dims)
        moe.moe_forward_block(dims, x, gw, 1e-6, w, bias, hb, rb, ws)
        # the layer run next, after a call that hinted it
        y2 = torch.empty_like(x)
        moe.moe_forward(dims, x, other, bias, y2, moe.alloc_routing(dims), ws)
        torch.cuda.synchronize()
        outs.append((y.view(torch.int16).cpu(), {k: v.cpu() for k, v in r.items()}, hb.view(torch.int16).cpu(),
                     y2.view(torch.int16).cpu()))
    for o in outs[1:]:
        assert torch.equal(o[0], outs[0][0])
        for k in outs[0][1]:
            assert torch.equal(o[1][k], outs[0][1][k]), k
        assert torch.equal(o[2], outs[0][2])
        assert torch.equal(o[3], outs[0][3])


@pytest.mark.parametrize("T", [17, 33, 64])
def test_decode_rows_do_not_depend_on_the_batch(weights, T):
    """Each token's output is computed from its own row only, in an order that
    does not depend on the batch: at 17 .. 64 tokens (several token tiles,
    the multi-tile stage-1 kernel) the first 16 outputs are the same bits as
    those of the 16-token batch (one tile) of the same rows."""
    import torch
    from fine_grained_moe_amd import moe
    dev, host = weights
    inp = synth.make_layer(T=T, d=1024, E=64, F=512, Fs=2048, k=1, act="bf16", seed=900 + T)
    x = torch.from_numpy(inp.x).to(device="cuda", dtype=torch.bfloat16)
    bt = torch.zeros(64, device="cuda")

    def fwd(n):
        dims = moe.make_dims(n, 1024, 64, 512, 2048, 1, "bf16", w_routed="int4")
        y = torch.empty_like(x[:n])
        r = moe.alloc_routing(dims)
        moe.moe_forward(dims, x[:n].contiguous(), dev, bt, y, r, moe.alloc_workspace(dims))
        torch.cuda.synchronize()
        return y, r["idx"].clone()

    y_all, idx_all = fwd(T)
    y_16, idx_16 = fwd(16)
    assert torch.equal(idx_all[:16], idx_16)
    assert torch.equal(y_all[:16], y_16)
