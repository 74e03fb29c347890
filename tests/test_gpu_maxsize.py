"""The layer at the largest batch the library accepts for the NanoColibri
shape (d = 1024, 64 experts of width 512, top-2, shared width 2048, bf16):
the host check admits T * max(d, 2 Fs) < 2^31, so T = 524,287 tokens (2,047
tiles of 256 rows and a ragged tail of 255).  One moe_forward_bias_step call,
then what holds at any size, checked on the whole batch: loads that sum to
2T and equal the histogram of the selected experts, offsets their exclusive
prefix, a dispatch order sorted by (expert, slot), pos its inverse, and the
bias step bit-exact from those loads; and against the oracle on 48 sampled
tokens (the first and last, tile edges, random ones): selections exactly,
gates within 1e-6, y within relative Frobenius error 1e-2.  A token whose
top-2 margin is under 1e-3 may break the tie either way; there only the
chosen experts' keys are checked to lie within that margin of the best.

x is drawn with torch's CPU generator (seed 2027): unit normal rows scaled to
unit RMS, rounded to bf16; the weights come from the seeded layer generator.
"""
import numpy as np
import pytest

import oracle.moe_oracle as om
from fine_grained_moe_amd import synth
from tests import _helpers as H

pytestmark = pytest.mark.gpu

D, E, F, FS, K = 1024, 64, 512, 2048, 2
T_MAX = ((1 << 31) - 1) // max(D, 2 * FS)          # 524,287
GAMMA = 1e-3


def _x_host(T, seed):
    import torch
    g = torch.Generator().manual_seed(seed)
    x = torch.empty((T, D), dtype=torch.bfloat16)
    step = 1 << 16
    for t0 in range(0, T, step):
        blk = torch.randn((min(step, T - t0), D), generator=g, dtype=torch.float32)
        blk = blk / torch.sqrt((blk.double() ** 2).mean(dim=1, keepdim=True) + 1e-6).float()
        x[t0:t0 + blk.shape[0]] = blk.to(torch.bfloat16)
    return x


def test_largest_accepted_batch():
    import torch
    from fine_grained_moe_amd import moe
    T = T_MAX
    assert moe.moe_workspace_bytes(moe.make_dims(T + 1, D, E, F, FS, K, "bf16")) == 0   # one more is refused
    dims = moe.make_dims(T, D, E, F, FS, K, "bf16")
    lay = synth.make_layer(T=1, d=D, E=E, F=F, Fs=FS, k=K, act="bf16", seed=29)

    def up(a):
        return torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(device="cuda", dtype=torch.bfloat16)

    w = dict(w_router=up(lay.w_router), w_gate_up=up(lay.w_gate_up), w_down=up(lay.w_down),
             w_sh_gate_up=up(lay.w_sh_gate_up), w_sh_down=up(lay.w_sh_down))
    xh = _x_host(T, 2027)
    x = xh.cuda()
    bias0 = (np.random.default_rng(5).standard_normal(E) * 1e-3).astype(np.float32)
    bias = torch.from_numpy(bias0).cuda()
    y = torch.empty_like(x)
    r = moe.alloc_routing(dims)
    stats = torch.zeros(4, dtype=torch.float32, device="cuda")
    print(f"max batch: T={T}, workspace {moe.moe_workspace_bytes(dims) / 2**30:.2f} GiB", flush=True)
    moe.moe_forward_bias_step(dims, x, w, bias, GAMMA, stats, y, r, moe.alloc_workspace(dims))
    torch.cuda.synchronize()

    # properties over the whole batch
    slots = T * K
    idx = r["idx"].long().reshape(-1)
    counts = r["counts"].long()
    assert int(counts.sum()) == slots
    assert torch.equal(torch.bincount(idx, minlength=E), counts)
    offs = r["offsets"].long()
    assert torch.equal(offs, torch.cat([torch.zeros(1, dtype=torch.long, device="cuda"), torch.cumsum(counts, 0)]))
    perm = r["perm"].long()
    key = idx[perm] * slots + perm
    assert bool((key[1:] > key[:-1]).all())                 # sorted by (expert, slot), every slot once
    pos = r["pos"].long().reshape(-1)
    assert torch.equal(perm[pos], torch.arange(slots, device="cuda"))
    got_bias = bias.cpu().numpy()
    want_bias = om.bias_update(bias0, counts.cpu().numpy(), slots, GAMMA)
    assert got_bias.view(np.uint32).tolist() == want_bias.view(np.uint32).tolist()

    # sampled tokens against the oracle
    rng = np.random.default_rng(11)
    fixed = [0, 1, 255, 256, 4095, 4096, T // 2, T - 257, T - 256, T - 255, T - 2, T - 1]
    sample = np.unique(np.concatenate([fixed, rng.choice(T, 48 - len(fixed), replace=False)]))
    st = torch.from_numpy(sample).cuda()
    xs = xh[torch.from_numpy(sample)].float().numpy().astype(np.float64)
    ys = y[st].float().cpu().numpy().astype(np.float64)
    idx_s = r["idx"][st].cpu().numpy()
    gate_s = r["gate"][st].cpu().numpy()
    y_ref, ref = om.forward(xs, lay.w_router, lay.w_gate_up, lay.w_down, lay.w_sh_gate_up, lay.w_sh_down,
                            bias0, K)
    margin = om.topk_margin(ref.v, K)
    clear = margin >= 1e-3
    assert clear.sum() >= len(sample) - 4
    np.testing.assert_array_equal(idx_s[clear], ref.idx[clear])
    np.testing.assert_allclose(gate_s[clear], ref.gate[clear], rtol=0, atol=1e-6)
    for i in np.nonzero(~clear)[0]:                          # near ties: any of the near-best experts
        kth = np.sort(ref.v[i])[::-1][K - 1]
        assert np.all(ref.v[i][idx_s[i]] >= kth - 1e-3)
    err = float(np.linalg.norm(ys[clear] - y_ref[clear]) / np.linalg.norm(y_ref[clear]))
    print(f"max batch: {clear.sum()} of {len(sample)} sampled tokens clear of ties, rel_fro(y) = {err:.3e}",
          flush=True)
    assert err <= 1e-2
    row = H.row_rel_max(ys[clear], y_ref[clear])
    print(f"  worst sampled row {row:.3e}", flush=True)
    assert row <= 3e-2
