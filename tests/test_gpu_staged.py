"""Stage-major routed weights (w_routed = bf16_staged, moe_pack_routed_bf16).

The pack is a storage order of the same bf16 matrices: its output is checked
element by element against the order restated here (per expert, per 256-row
tile, per 32-element contraction chunk, the tile's rows in the GEMM's LDS
order).  The forward that reads it performs the same products in the same
order as the row-major forward, so its outputs are compared bitwise with
moe_forward on the row-major weights (itself checked against the oracle in
test_gpu_forward.py), and once more against the oracle directly.
"""
import numpy as np
import pytest

from fine_grained_moe_amd import synth
from tests import _helpers as H

pytestmark = pytest.mark.gpu


def _lds_row(swiglu, R, nt, up_off):
    if swiglu:
        half, h = R >> 7, R & 127
        w, ni, f = h >> 6, (h >> 4) & 3, h & 15
        return (up_off if half else 0) + nt * 128 + w * 64 + 4 * f + ni
    w, ni, f = R >> 7, (R >> 4) & 7, R & 15
    return nt * 256 + w * 128 + 8 * f + ni


def _expected_pack(W, swiglu, up_off):
    """W: [E, rows, K] (uint16 bf16 bits) -> [E, tiles, K/32, 256, 32]."""
    E, rows, K = W.shape
    tiles = rows // 256
    out = np.empty((E, tiles, K // 32, 256, 32), W.dtype)
    for nt in range(tiles):
        src = np.array([_lds_row(swiglu, R, nt, up_off) for R in range(256)])
        blk = W[:, src, :].reshape(E, 256, K // 32, 32)
        out[:, nt] = blk.transpose(0, 2, 1, 3)
    return out


def _bits(t):
    import torch
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def _staged(w, dims_staged):
    import torch
    from fine_grained_moe_amd import moe
    ws = dict(w)
    ws["w_gate_up"] = torch.empty_like(w["w_gate_up"])
    ws["w_down"] = torch.empty_like(w["w_down"])
    moe.moe_pack_routed_bf16(dims_staged, w["w_gate_up"], w["w_down"], ws["w_gate_up"], ws["w_down"])
    return ws


def test_pack_layout():
    import torch
    from fine_grained_moe_amd import moe
    E, d, F = 3, 512, 256
    g = torch.Generator().manual_seed(3)
    wgu = torch.randn((E, 2 * F, d), generator=g).to(torch.bfloat16).cuda()
    wd = torch.randn((E, d, F), generator=g).to(torch.bfloat16).cuda()
    ogu, od = torch.empty_like(wgu), torch.empty_like(wd)
    moe.moe_pack_routed_bf16(moe.make_dims(0, d, E, F, 256, 2, "bf16"), wgu, wd, ogu, od)
    torch.cuda.synchronize()
    want_gu = _expected_pack(_bits(wgu), True, F)
    want_d = _expected_pack(_bits(wd), False, 0)
    assert np.array_equal(_bits(ogu).reshape(want_gu.shape), want_gu)
    assert np.array_equal(_bits(od).reshape(want_d.shape), want_d)


def _compare(inp, bias_step=False):
    import torch
    from fine_grained_moe_amd import moe
    x, w = H.to_gpu(inp)
    dims = moe.make_dims(inp.T, inp.d, inp.E, inp.F, inp.Fs, inp.k, "bf16")
    dims_s = moe.make_dims(inp.T, inp.d, inp.E, inp.F, inp.Fs, inp.k, "bf16", w_routed="bf16_staged")
    wst = _staged(w, dims_s)
    outs = []
    for dm, ww in ((dims, w), (dims_s, wst)):
        b = torch.from_numpy(np.asarray(inp.bias, np.float32)).cuda()
        y = torch.empty_like(x)
        r = moe.alloc_routing(dm)
        stats = torch.zeros(4, dtype=torch.float32, device="cuda")
        if bias_step:
            moe.moe_forward_bias_step(dm, x, ww, b, 1e-3, stats, y, r, moe.alloc_workspace(dm))
        else:
            moe.moe_forward(dm, x, ww, b, y, r, moe.alloc_workspace(dm))
        torch.cuda.synchronize()
        outs.append((y, r, b, stats))
    (y0, r0, b0, s0), (y1, r1, b1, s1) = outs
    assert torch.equal(y0.view(torch.int16), y1.view(torch.int16))
    for n in r0:
        assert torch.equal(r0[n], r1[n]), n
    assert torch.equal(b0, b1) and torch.equal(s0, s1)
    return y1


@pytest.mark.parametrize("T", [1, 65, 1027, 4096])
def test_staged_forward_bitwise(T):
    inp = synth.make_layer(T=T, d=1024, E=64, F=512, Fs=2048, k=2, act="bf16", seed=400 + T)
    _compare(inp)


def test_staged_forward_bias_step_bitwise():
    inp = synth.make_layer(T=4096, d=1024, E=64, F=512, Fs=2048, k=2, act="bf16", seed=9)
    _compare(inp, bias_step=True)


def test_staged_other_shape_against_oracle():
    """d = 256, 8 experts of width 128, top-3: bitwise against the row-major
    forward, and within the bf16 tolerance of the oracle."""
    inp = synth.make_layer(T=300, d=256, E=8, F=128, Fs=256, k=3, act="bf16", seed=21)
    H.remove_near_ties(inp)
    y = _compare(inp).float().cpu().numpy().astype(np.float64)
    y_ref, _ = H.oracle_forward(inp)
    H.check_close(y, y_ref, "bf16", "staged d=256 E=8 k=3 y:")


def test_staged_block_bitwise_equal_row_major():
    """The MoE block (RMSNorm in, residual out) on stage-major routed weights,
    as the 23-layer stack leg runs it, gives the bits of the block on the
    row-major weights (itself checked against the oracle in
    test_gpu_block.py)."""
    import torch
    from fine_grained_moe_amd import moe
    T, d, E, F, Fs = 600, 1024, 64, 512, 2048
    inp = synth.make_layer(T=T, d=d, E=E, F=F, Fs=Fs, k=2, act="bf16", seed=33)
    x, w = H.to_gpu(inp)
    rng = np.random.default_rng(33)
    h = torch.from_numpy(synth.round_to_bf16((rng.standard_normal((T, d)) * 2.0).astype(np.float32))).to(
        device="cuda", dtype=torch.bfloat16)
    gamma = torch.from_numpy((1.0 + 0.1 * rng.standard_normal(d)).astype(np.float32)).cuda()
    bias = torch.zeros(E, device="cuda")
    dims = moe.make_dims(T, d, E, F, Fs, 2, "bf16")
    dims_s = moe.make_dims(T, d, E, F, Fs, 2, "bf16", w_routed="bf16_staged")
    outs = []
    for dm, ww in ((dims, w), (dims_s, _staged(w, dims_s))):
        out = torch.empty_like(h)
        r = moe.alloc_routing(dm)
        moe.moe_forward_block(dm, h, gamma, 1e-6, ww, bias, out, r, moe.alloc_workspace(dm))
        torch.cuda.synchronize()
        outs.append((out, r))
    assert torch.equal(outs[0][0], outs[1][0])
    for n in outs[0][1]:
        assert torch.equal(outs[0][1][n], outs[1][1][n]), n
