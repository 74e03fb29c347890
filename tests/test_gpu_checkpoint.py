"""Checkpoint and resume of the balancing state.

The expert bias is the layer's only state that changes from batch to batch
(architecture paragraph of the seventnews article's opening section: the
per-layer bias is nudged after every batch; its "Relay training" section
hands the run from one rented machine to the next, so the state must survive
a save and a reload).  On the skewed-routing workload (T = 16384, Zipf(1)
preset): 5 fused forward + bias steps, the bias saved to .npy and reloaded
into a fresh device tensor, 5 more steps; the result must be bit-identical to
10 steps without the break, and to the oracle's sequence at every step."""
import numpy as np
import pytest

from fine_grained_moe_amd import synth
from tests import _helpers as H

pytestmark = pytest.mark.gpu

GAMMA = 1e-3


@pytest.mark.slow
def test_bias_save_reload_resume_is_bit_identical(tmp_path):
    import torch
    from fine_grained_moe_amd import moe
    inp = synth.make_workload("zipf_t16384")
    for _ in range(3):
        b0 = H.zipf_bias(inp)
        if H.remove_near_ties(inp, bias_states=[b0], steps_after=10) == 0:
            break
    states = H.bias_sequence(inp, b0, 10)
    x, w = H.to_gpu(inp)
    dims = moe.make_dims(inp.T, inp.d, inp.E, inp.F, inp.Fs, inp.k, inp.act)
    r = moe.alloc_routing(dims)
    ws = moe.alloc_workspace(dims)
    y = torch.empty_like(x)

    def steps(bias, n, first):
        bits = []
        for i in range(n):
            moe.moe_forward_bias_step(dims, x, w, bias, GAMMA, None, y, r, ws)
            torch.cuda.synchronize()
            got = bias.cpu().numpy()
            assert got.view(np.uint32).tolist() == states[first + i + 1].view(np.uint32).tolist(), first + i
            bits.append(got.view(np.uint32).copy())
        return bits

    straight = steps(torch.from_numpy(b0.copy()).cuda(), 10, 0)

    b = torch.from_numpy(b0.copy()).cuda()
    first = steps(b, 5, 0)
    path = tmp_path / "bias_step5.npy"
    np.save(path, b.cpu().numpy())
    del b
    torch.cuda.synchronize()
    loaded = np.load(path)
    assert loaded.dtype == np.float32 and loaded.shape == (inp.E,)
    b2 = torch.from_numpy(loaded).cuda()
    second = steps(b2, 5, 5)
    for i, (a, c) in enumerate(zip(straight, first + second)):
        assert a.tolist() == c.tolist(), i
    print(f"resume after step 5: bias bit-identical to 10 straight steps; hottest expert bias "
          f"{float(loaded.max()):.4f}", flush=True)
