"""GPU parity of the int4 export (moe_quantize_int4) against the oracle's
encoder (reading R10): packed bytes and bf16 scale bits compared exactly, on
the layer's full weight tensors and on hand-built groups (zeros, exact
half-way quotients, a lone nonzero, fp32 inputs), then the exported weights
served by the int4 top-1 path against the oracle's dequantised layer."""
import numpy as np
import pytest

import oracle.moe_oracle as om
from fine_grained_moe_amd import synth
from tests import _helpers as H

pytestmark = pytest.mark.gpu


def _gpu_quant(w_np, dtype_name="bf16"):
    import torch
    from fine_grained_moe_amd import moe
    dt = torch.bfloat16 if dtype_name == "bf16" else torch.float32
    w = torch.from_numpy(np.ascontiguousarray(w_np, np.float32)).to(device="cuda", dtype=dt)
    K = w.shape[-1]
    packed = torch.empty(*w.shape[:-1], K // 2, dtype=torch.uint8, device="cuda")
    scales = torch.empty(*w.shape[:-1], K // 128, dtype=torch.bfloat16, device="cuda")
    moe.moe_quantize_int4(w, packed, scales)
    torch.cuda.synchronize()
    return packed.cpu().numpy(), scales.view(torch.int16).cpu().numpy().view(np.uint16), (w, packed, scales)


def _oracle_quant(w_np):
    packed, scale = om.quantize_int4(np.asarray(w_np, np.float64))
    f = scale.astype(np.float32)
    assert np.all(f.astype(np.float64) == scale)           # 8 significant bits: exact in float32
    bits = f.view(np.uint32)
    assert np.all(bits & 0xFFFF == 0)                        # ... and in bfloat16
    return packed, (bits >> 16).astype(np.uint16)


def _check_exact(w_np, dtype_name="bf16"):
    if dtype_name == "bf16":                                 # the values the bf16 tensor holds
        w_np = synth.round_to_bf16(np.asarray(w_np, np.float32))
    gp, gs, _ = _gpu_quant(w_np, dtype_name)
    op, os_ = _oracle_quant(w_np)
    bad_s = np.count_nonzero(gs != os_)
    bad_p = np.count_nonzero(gp != op)
    print(f"int4 export {dtype_name} {tuple(np.shape(w_np))}: {bad_p} packed bytes and {bad_s} scales differ",
          flush=True)
    assert bad_s == 0 and bad_p == 0


def test_layer_weights_bit_exact():
    """The full routed weights of a 64-expert layer (N(0, 0.02), bf16)."""
    inp = synth.make_layer(T=1, d=1024, E=64, F=512, Fs=2048, k=1, act="bf16", seed=21)
    _check_exact(inp.w_gate_up)      # [64, 1024, 1024]: 524,288 groups
    _check_exact(inp.w_down)         # [64, 1024, 512]


def test_fp32_inputs_bit_exact():
    rng = np.random.default_rng(5)
    w = (rng.standard_normal((300, 1024)) * 0.02).astype(np.float32)
    w[7, 128:256] *= 1e3                                     # one group of large values
    _check_exact(w, "f32")


def _edge_groups():
    rows = []
    z = np.zeros(128, np.float32)
    rows.append(z.copy())                                   # all zero: scale 0, q 0
    g = z.copy()
    g[0] = 7.0                                              # scale = 1 exactly
    g[1:9] = [2.5, 3.5, -2.5, -0.5, 0.5, 1.5, -1.5, 6.5]   # exact half-way quotients: ties to even
    rows.append(g)
    g = z.copy()
    g[77] = -3.0e-3                                         # a lone negative absmax
    rows.append(g)
    g = np.full(128, -0.125, np.float32)
    g[5] = 0.875                                            # absmax 0.875: scale 0.125, q = 7 and -1
    rows.append(g)
    g = np.linspace(-1.0, 1.0, 128, dtype=np.float32)
    rows.append(synth.round_to_bf16(g))                     # a ramp: every code
    g = synth.round_to_bf16(np.geomspace(1e-4, 50.0, 128).astype(np.float32))
    g[::3] *= -1
    rows.append(g)                                          # six decades in one group
    g = z.copy()
    g[5] = 7 * (1 + 2 ** -8)                                # absmax / 7 = 1 + 2^-8, a bf16 tie: scale 1 (even)
    g[9] = -3.5                                             # q tie: to even, -4
    rows.append(g)
    g = z.copy()
    g[40] = -7 * (1 + 3 * 2 ** -8)                          # absmax / 7 = 1 + 3 * 2^-8: scale rounds up to 1 + 2^-6
    rows.append(g)
    return np.stack(rows)


def test_edge_groups_bit_exact():
    w = _edge_groups()
    _check_exact(w, "bf16")
    _check_exact(w, "f32")
    # the tie group decodes to the even neighbours
    gp, _, _ = _gpu_quant(w)
    q = om.unpack_int4(gp[1])
    assert q[:9].tolist() == [7, 2, 4, -2, 0, 0, 2, -2, 6]


def test_ragged_row_counts():
    rng = np.random.default_rng(9)
    for rows in (1, 3, 5, 129):
        w = synth.round_to_bf16((rng.standard_normal((rows, 256)) * 0.05).astype(np.float32))
        _check_exact(w)


def test_exported_weights_serve_the_int4_path():
    """bf16 training weights -> GPU int4 export -> int4 top-1 forward, against
    the oracle's layer on the oracle's own encoding of the same weights."""
    import torch
    from fine_grained_moe_amd import moe
    T = 8
    inp = synth.make_layer(T=T, d=1024, E=64, F=512, Fs=2048, k=1, act="bf16", seed=31)
    H.remove_near_ties(inp, bias_states=[np.zeros(64, np.float32)])
    _, _, (_, pg, sg) = _gpu_quant(inp.w_gate_up)
    _, _, (_, pd, sd) = _gpu_quant(inp.w_down)

    def bf(a):
        return torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(device="cuda", dtype=torch.bfloat16)

    w = dict(w_router=bf(inp.w_router), w_gate_up=pg, s_gate_up=sg, w_down=pd, s_down=sd,
             w_sh_gate_up=bf(inp.w_sh_gate_up), w_sh_down=bf(inp.w_sh_down))
    dims = moe.make_dims(T, 1024, 64, 512, 2048, 1, "bf16", w_routed="int4")
    x = bf(inp.x)
    y = torch.empty_like(x)
    r = moe.alloc_routing(dims)
    moe.moe_forward(dims, x, w, torch.zeros(64, device="cuda"), y, r, moe.alloc_workspace(dims))
    torch.cuda.synchronize()
    qg, s_g = om.quantize_int4(inp.w_gate_up)
    qd, s_d = om.quantize_int4(inp.w_down)
    y_ref, ref = om.forward_int4_top1(inp.x, inp.w_router, qg, s_g, qd, s_d, inp.w_sh_gate_up, inp.w_sh_down,
                                      np.zeros(64, np.float32))
    rn = {k: v.cpu().numpy() for k, v in r.items()}
    H.check_routing_exact(rn, ref, 64)
    H.check_close(y.float().cpu().numpy(), y_ref, "bf16", f"export -> serve T={T} y:")
