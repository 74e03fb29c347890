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
