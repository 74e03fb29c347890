"""GPU parity of the int4 top-1 prefill (w_routed = int4, more than 64 tokens):
routing and the grouped GEMMs reading the packed experts (each operand
fragment expanded to bf16(q * scale) in registers; for contractions longer
than 3072, dequantised bf16 copies of the loaded experts), against the
oracle's layer on the exactly dequantised weights (forward_int4_top1).

The routed weights are N(0, 0.02) draws encoded by the oracle's int4 encoder;
both sides read the same bytes and scales.  Routing is compared bit-exactly
(gate exactly 1); y within relative Frobenius error 1e-2.  The prefill rounds
each dequantised weight q * scale once to bf16 before its products (at most
2^-9 of the weight), inside that bound.
"""
import numpy as np
import pytest

import oracle.moe_oracle as om
from fine_grained_moe_amd import synth
from tests import _helpers as H

pytestmark = pytest.mark.gpu

SHAPE = dict(d=1024, E=64, F=512, Fs=2048)


def _bf(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(device="cuda", dtype=torch.bfloat16)


def _int4_layer(T, seed, bias=None, **shape):
    shp = dict(SHAPE)
    shp.update(shape)
    inp = synth.make_layer(T=T, k=1, act="bf16", seed=seed, **shp)
    b = np.zeros(inp.E, np.float32) if bias is None else np.asarray(bias, np.float32)
    H.remove_near_ties(inp, bias_states=[b])
    qg, sg = om.quantize_int4(inp.w_gate_up)
    qd, sd = om.quantize_int4(inp.w_down)
    return inp, b, (qg, sg, qd, sd)


def _dev_weights(inp, q):
    import torch
    qg, sg, qd, sd = q
    return dict(w_router=_bf(inp.w_router), w_gate_up=torch.from_numpy(qg).cuda(), s_gate_up=_bf(sg),
                w_down=torch.from_numpy(qd).cuda(), s_down=_bf(sd), w_sh_gate_up=_bf(inp.w_sh_gate_up),
                w_sh_down=_bf(inp.w_sh_down))


def _run(inp, b, q, fill_ws=None):
    import torch
    from fine_grained_moe_amd import moe
    dims = moe.make_dims(inp.T, inp.d, inp.E, inp.F, inp.Fs, 1, "bf16", w_routed="int4")
    x = _bf(inp.x)
    y = torch.empty_like(x)
    r = moe.alloc_routing(dims)
    ws = moe.alloc_workspace(dims)
    if fill_ws is not None:
        ws.fill_(fill_ws)
    moe.moe_forward(dims, x, _dev_weights(inp, q), torch.from_numpy(b).cuda(), y, r, ws)
    torch.cuda.synchronize()
    return y.float().cpu().numpy(), {k: v.cpu().numpy() for k, v in r.items()}


def _check(inp, b, q, y, rn, what):
    qg, sg, qd, sd = q
    y_ref, ref = om.forward_int4_top1(inp.x, inp.w_router, qg, sg, qd, sd, inp.w_sh_gate_up, inp.w_sh_down, b)
    H.check_routing_exact(rn, ref, inp.E)
    assert np.all(rn["gate"] == 1.0)
    err = H.check_close(y, y_ref, "bf16",
                        f"[{what}] prefill T={inp.T} ({np.count_nonzero(rn['counts'])} active experts) y:")
    return err


@pytest.mark.parametrize("T", [65, 300, 1027, 4096])
def test_int4_prefill(T):
    inp, b, q = _int4_layer(T, seed=200 + T)
    y, rn = _run(inp, b, q)
    _check(inp, b, q, y, rn, "nanocolibri")


def _tiered_bias(E=64, hot=0.12):
    """Biases that give, at 4096 tokens, experts of every tile class: most
    with at most 64 rows, some with 65-128, some with 129-256, and two with
    more than 256 (whole 256-row tiles plus a ragged one)."""
    b = np.zeros(E, np.float32)
    b[:2] = hot
    b[2:6] = hot / 2
    b[6:12] = hot / 4
    return b


def _tile_classes(counts):
    c = np.asarray(counts)
    return [int((c[c > 0] <= 64).sum()), int(((c > 64) & (c <= 128)).sum()), int(((c > 128) & (c <= 256)).sum()),
            int((c > 256).sum())]


def test_int4_prefill_every_tile_layout():
    """Skewed loads at 4096 tokens: the routed tiles of one forward run in the
    1 x 8 (at most 64 rows), 2 x 4 (at most 128) and 4 x 2 wave layouts, and
    an expert spans several 256-row tiles."""
    inp, b, q = _int4_layer(4096, seed=31, bias=_tiered_bias())
    y, rn = _run(inp, b, q)
    classes = _tile_classes(rn["counts"])
    assert all(n > 0 for n in classes), classes
    _check(inp, b, q, y, rn, f"tiered loads {classes}")


def test_int4_prefill_other_shape():
    """Not the decode shape: d = 256, 8 experts of width 128, shared 256."""
    inp, b, q = _int4_layer(200, seed=7, d=256, E=8, F=128, Fs=256)
    y, rn = _run(inp, b, q)
    _check(inp, b, q, y, rn, "d256")


def test_int4_prefill_idle_experts_are_not_read():
    """Half the experts get no tokens (bias -4); the workspace starts as NaN
    bytes, so a read of an idle expert's (not dequantised) weights would show."""
    bias = np.zeros(64, np.float32)
    bias[::2] = -4.0
    inp, b, q = _int4_layer(500, seed=11, bias=bias)
    y, rn = _run(inp, b, q, fill_ws=255)
    assert np.all(rn["counts"][::2] == 0)
    assert np.all(np.isfinite(y))
    _check(inp, b, q, y, rn, "idle experts")


def test_int4_prefill_run_to_run_bitwise():
    import torch
    from fine_grained_moe_amd import moe
    inp, b, q = _int4_layer(700, seed=3)
    dims = moe.make_dims(inp.T, inp.d, inp.E, inp.F, inp.Fs, 1, "bf16", w_routed="int4")
    x = _bf(inp.x)
    w = _dev_weights(inp, q)
    bt = torch.from_numpy(b).cuda()
    outs = []
    for _ in range(2):
        y = torch.empty_like(x)
        moe.moe_forward(dims, x, w, bt, y, moe.alloc_routing(dims), moe.alloc_workspace(dims))
        torch.cuda.synchronize()
        outs.append(y)
    assert torch.equal(outs[0], outs[1])


@pytest.mark.parametrize("T", [1, 8, 64])
def test_int4_small_batch_other_shape(T):
    """Up to 64 tokens at a shape the decode kernels are not built for, the
    int4 top-1 forward runs the prefill path (route, grouped GEMMs on the
    packed experts, combine) and matches the oracle."""
    inp, b, q = _int4_layer(T, seed=400 + T, d=256, E=8, F=128, Fs=256)
    y, rn = _run(inp, b, q)
    _check(inp, b, q, y, rn, "small batch, other shape")


@pytest.mark.parametrize("T,shape", [(130, {}), (8, dict(d=256, E=8, F=128, Fs=256))])
def test_int4_prefill_block(T, shape):
    """The MoE block (RMSNorm in, residual out) on the prefill path: above
    64 tokens, and at 8 tokens of a shape the decode kernels are not built
    for (the norm then runs as its own launch)."""
    import torch
    from fine_grained_moe_amd import moe
    inp, b, q = _int4_layer(1, seed=17, **shape)
    d, E = inp.d, inp.E
    rng = np.random.default_rng(17)
    gamma = (1.0 + 0.1 * rng.standard_normal(d)).astype(np.float32)
    h = synth.round_to_bf16((rng.standard_normal((T, d)) * rng.uniform(0.5, 4.0, (T, 1))).astype(np.float32))
    for _ in range(20):                                    # no near-tie rows in the routing of RMSNorm(h)
        x = om.rms_norm(h, gamma)
        v = om.route(x, inp.w_router, b, 1).v
        bad = np.nonzero(om.topk_margin(v, 1) < 1e-3)[0]
        if bad.size == 0:
            break
        h[bad] = synth.round_to_bf16(rng.standard_normal((bad.size, d)).astype(np.float32))
    dims = moe.make_dims(T, d, E, inp.F, inp.Fs, 1, "bf16", w_routed="int4")
    ht = _bf(h)
    out = torch.empty_like(ht)
    r = moe.alloc_routing(dims)
    moe.moe_forward_block(dims, ht, torch.from_numpy(gamma).cuda(), 1e-6, _dev_weights(inp, q),
                          torch.from_numpy(b).cuda(), out, r, moe.alloc_workspace(dims))
    torch.cuda.synchronize()
    qg, sg, qd, sd = q
    h_ref, _, ref = om.block_forward(h, gamma, inp.w_router, om.dequantize_int4(qg, sg), om.dequantize_int4(qd, sd),
                                     inp.w_sh_gate_up, inp.w_sh_down, b, 1)
    H.check_routing_exact({k: v.cpu().numpy() for k, v in r.items()}, ref, E)
    h_out = out.float().cpu().numpy().astype(np.float64)
    y_ref = h_ref - h.astype(np.float64)
    err = float(np.linalg.norm(h_out - h_ref))
    bound = 1e-2 * float(np.linalg.norm(y_ref)) + 2.0 ** -8 * float(np.linalg.norm(h_ref))
    print(f"[block] prefill T={T}: ||h_out - h_ref|| / ||y_ref|| = {err / np.linalg.norm(y_ref):.2e}", flush=True)
    assert H.rel_fro(h_out, h_ref) <= 1e-2 and err <= bound
    rerr = np.linalg.norm(h_out - h_ref, axis=-1)
    rbound = 3e-2 * np.linalg.norm(y_ref, axis=-1) + 2.0 ** -8 * np.linalg.norm(h_ref, axis=-1)
    assert np.all(rerr <= rbound), ("worst row", float((rerr / rbound).max()))


@pytest.mark.parametrize("T,tiered", [(300, False), (4096, True)])
def test_int4_prefill_fused_equals_bf16_path_bitwise(T, tiered):
    """The prefill's GEMMs expand each int4 operand fragment to bf16(q *
    scale) in registers, in the small-tile wave layouts where a tile has few
    rows.  Fed the same values as bf16 weights (the host's exact q * scale,
    rounded once to bf16), the bf16 layer (k = 1, every tile in the 4 x 2
    layout) runs the same products in the same order for every output
    element: the outputs must be the same bits."""
    import torch
    from fine_grained_moe_amd import moe
    inp, b, q = _int4_layer(T, seed=23 if not tiered else 31, bias=_tiered_bias() if tiered else None)
    qg, sg, qd, sd = q
    y4, rn4 = _run(inp, b, q)
    dims = moe.make_dims(inp.T, inp.d, inp.E, inp.F, inp.Fs, 1, "bf16")
    w = dict(w_router=_bf(inp.w_router), w_gate_up=_bf(synth.round_to_bf16(om.dequantize_int4(qg, sg).astype(np.float32))),
             w_down=_bf(synth.round_to_bf16(om.dequantize_int4(qd, sd).astype(np.float32))),
             w_sh_gate_up=_bf(inp.w_sh_gate_up), w_sh_down=_bf(inp.w_sh_down))
    x = _bf(inp.x)
    y = torch.empty_like(x)
    r = moe.alloc_routing(dims)
    moe.moe_forward(dims, x, w, torch.from_numpy(b).cuda(), y, r, moe.alloc_workspace(dims))
    torch.cuda.synchronize()
    for n in ("idx", "counts", "perm", "pos"):
        np.testing.assert_array_equal(r[n].cpu().numpy(), rn4[n], err_msg=n)
    np.testing.assert_array_equal(y.float().cpu().numpy(), y4)


def test_int4_prefill_long_contraction():
    """d = 3200 (25 scale groups per row, more than a GEMM tile keeps in LDS):
    the prefill dequantises the loaded experts to bf16 copies first."""
    inp, b, q = _int4_layer(100, seed=29, d=3200, E=8, F=128, Fs=256)
    y, rn = _run(inp, b, q)
    _check(inp, b, q, y, rn, "d3200")
