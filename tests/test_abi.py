"""The C ABI library: it loads, exports every function include/moe.h declares,
and rejects bad arguments on the host before anything reaches a GPU."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe.h")
LIBPATH = os.path.join(ROOT, "fine_grained_moe_amd", "libfgmoe.so")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIBPATH):
        pytest.fail("libfgmoe.so is not built; run python -m fine_grained_moe_amd.build")
    import torch  # noqa: F401  (same load order as the binding)
    from fine_grained_moe_amd import moe
    return moe


def test_header_declares_the_entry_points():
    assert declared_functions() == sorted(["moe_workspace_bytes", "moe_route", "moe_forward", "moe_forward_block",
                                           "moe_bias_update", "moe_bias_update_stats", "moe_backward",
                                           "moe_quantize_int4", "moe_pack_routed_bf16", "moe_forward_bias_step", "moe_status_str",
                                           "moe_forward_events", "moe_forward_noalloc", "moe_forward_cached", "moe_cache_create",
                                           "moe_cache_prepare", "moe_cache_state", "moe_cache_destroy"])


def test_library_exports_every_declared_symbol(lib):
    raw = ctypes.CDLL(LIBPATH)
    for name in declared_functions():
        assert hasattr(raw, name), name


def test_status_strings(lib):
    for code in range(6):
        assert lib.moe_status_str(code)
    assert lib.moe_status_str(0) == "ok"
    assert "unknown" in lib.moe_status_str(99)


def test_workspace_bytes(lib):
    d = lib.make_dims(4096, 1024, 64, 512, 2048, 2, "bf16")
    n = lib.moe_workspace_bytes(d)
    slots = 4096 * 2
    assert n >= slots * 512 * 2 + slots * 1024 * 2 + 4096 * 2048 * 2
    assert lib.moe_workspace_bytes(d, training=True) > n
    for bad in (dict(E=65), dict(k=9), dict(k=3, E=2), dict(d=100), dict(F=96), dict(Fs=32)):
        args = dict(T=16, d=1024, E=64, F=512, Fs=2048, k=2)
        args.update(bad)
        assert lib.moe_workspace_bytes(lib.make_dims(act="bf16", **args)) == 0, bad
    assert lib.moe_workspace_bytes(lib.make_dims(-1, 1024, 64, 512, 2048, 2)) == 0


def _call_forward(lib, dims, x, y, ws, ws_bytes, weights=None, routing=None):
    W = lib.MoeWeights(*(weights or [0x10000000 + i * 0x1000000 for i in range(7)]))
    R = lib.MoeRouting(*(routing or [0x40000000 + i * 0x1000000 for i in range(6)]))
    return lib.LIB.moe_forward(ctypes.byref(dims), x, ctypes.byref(W), 0x50000000, y, ctypes.byref(R), 0, ws,
                               ws_bytes, None)


def test_host_checks_reject_before_launch(lib):
    """Fake addresses: every one of these calls must fail its host checks, so
    nothing is ever enqueued (there is no GPU here)."""
    dims = lib.make_dims(16, 128, 8, 64, 256, 2, "f32")
    need = lib.moe_workspace_bytes(dims)
    x, y, ws = 0x60000000, 0x70000000, 0x80000000
    assert _call_forward(lib, dims, x, y, ws, need - 1) == lib.MOE_E_WORKSPACE
    assert _call_forward(lib, dims, x, y, None, need) == lib.MOE_E_WORKSPACE
    assert _call_forward(lib, dims, None, y, ws, need) == lib.MOE_E_ARG
    assert _call_forward(lib, dims, x, x + 64, ws, need) == lib.MOE_E_ALIAS        # y overlaps x
    assert _call_forward(lib, dims, x, y, y + 16, need) == lib.MOE_E_ALIAS          # ws overlaps y
    bad_w = [0x10000000 + i * 0x1000000 for i in range(7)]
    bad_w[2] = None
    assert _call_forward(lib, dims, x, y, ws, need, weights=bad_w) == lib.MOE_E_ARG
    bad_r = [0x40000000 + i * 0x1000000 for i in range(6)]
    bad_r[1] = bad_r[0] + 8                                                         # gate overlaps idx
    assert _call_forward(lib, dims, x, y, ws, need, routing=bad_r) == lib.MOE_E_ALIAS
    big = lib.make_dims(16, 128, 65, 64, 256, 2, "f32")
    assert _call_forward(lib, big, x, y, ws, need) == lib.MOE_E_UNSUPPORTED
    neg = lib.make_dims(-5, 128, 8, 64, 256, 2, "f32")
    assert _call_forward(lib, neg, x, y, ws, need) == lib.MOE_E_ARG
    assert lib.LIB.moe_forward(None, x, None, None, y, None, 0, ws, need, None) == lib.MOE_E_ARG
    # bias step: null pointers, bad E, counts overlapping bias
    assert lib.LIB.moe_bias_update(8, 16, None, 1e-3, 0x1000, None) == lib.MOE_E_ARG
    assert lib.LIB.moe_bias_update(0, 16, 0x2000, 1e-3, 0x1000, None) == lib.MOE_E_ARG
    assert lib.LIB.moe_bias_update(65, 16, 0x2000, 1e-3, 0x1000, None) == lib.MOE_E_UNSUPPORTED
    assert lib.LIB.moe_bias_update(8, 16, 0x1000, 1e-3, 0x1010, None) == lib.MOE_E_ALIAS
    # bias step with telemetry: stats must be present and overlap neither input
    st = lib.LIB.moe_bias_update_stats
    assert st(8, 16, 0x2000, 1e-3, 0x1000, None, None) == lib.MOE_E_ARG
    assert st(8, 16, 0x2000, 1e-3, 0x1000, 0x1010, None) == lib.MOE_E_ALIAS
    assert st(8, 16, 0x2000, 1e-3, 0x1000, 0x2008, None) == lib.MOE_E_ALIAS
    assert st(65, 16, 0x2000, 1e-3, 0x1000, 0x3000, None) == lib.MOE_E_UNSUPPORTED
    assert st(8, -1, 0x2000, 1e-3, 0x1000, 0x3000, None) == lib.MOE_E_ARG


def test_route_host_checks(lib):
    dims = lib.make_dims(16, 128, 8, 64, 256, 2, "bf16")
    need = lib.moe_workspace_bytes(dims)
    R = lib.MoeRouting(*[0x40000000 + i * 0x1000000 for i in range(6)])
    assert lib.LIB.moe_route(ctypes.byref(dims), 0x1000, 0x20000, 0x30000, ctypes.byref(R), 0x90000000,
                             need - 1, None) == lib.MOE_E_WORKSPACE
    assert lib.LIB.moe_route(ctypes.byref(dims), 0x1000, 0x20000, 0x30000, None, 0x90000000, need,
                             None) == lib.MOE_E_ARG


def test_forward_bias_step_host_checks(lib):
    """moe_forward_bias_step rejects a null bias, and a bias or stats that
    overlaps another argument, before any launch."""
    dims = lib.make_dims(16, 128, 8, 64, 256, 2, "bf16")
    need = lib.moe_workspace_bytes(dims)
    W = lib.MoeWeights(0x100000, 0x200000, 0x300000, None, None, 0x400000, 0x500000)
    R = lib.MoeRouting(*[0x40000000 + i * 0x1000000 for i in range(6)])
    f = lib.LIB.moe_forward_bias_step
    x, y, ws = 0x1000, 0x8000, 0x90000000
    ok = (ctypes.byref(dims), x, ctypes.byref(W))
    assert f(*ok, None, 1e-3, None, y, ctypes.byref(R), 0, ws, need, None) == lib.MOE_E_ARG
    # the bias inside x (x is 16 x 128 bf16 = 4 KiB from 0x1000)
    assert f(*ok, 0x1100, 1e-3, None, y, ctypes.byref(R), 0, ws, need, None) == lib.MOE_E_ALIAS
    # stats inside the bias
    assert f(*ok, 0x20000, 1e-3, 0x20004, y, ctypes.byref(R), 0, ws, need, None) == lib.MOE_E_ALIAS
    # stats inside the workspace
    assert f(*ok, 0x20000, 1e-3, ws + 64, y, ctypes.byref(R), 0, ws, need, None) == lib.MOE_E_ALIAS
    assert f(*ok, 0x20000, 1e-3, None, y, ctypes.byref(R), 0, ws, need - 1, None) == lib.MOE_E_WORKSPACE


def test_forward_events_host_checks(lib):
    """The instrumented forward checks its own arguments (event count 0..8,
    no null event among them, bias_step 0 or 1) and otherwise reports the
    statuses of the call it instruments, before any launch."""
    dims = lib.make_dims(16, 128, 8, 64, 256, 2, "bf16")
    need = lib.moe_workspace_bytes(dims)
    W = lib.MoeWeights(0x100000, 0x200000, 0x300000, None, None, 0x400000, 0x500000)
    R = lib.MoeRouting(*[0x40000000 + i * 0x1000000 for i in range(6)])
    f = lib.LIB.moe_forward_events
    x, y, ws, b = 0x1000, 0x8000, 0x90000000, 0x20000
    ev9 = (ctypes.c_void_p * 9)(*([0x123] * 9))
    ev_null = (ctypes.c_void_p * 2)(0x123, None)
    head = (ctypes.byref(dims), x, ctypes.byref(W), b)
    tail = (y, ctypes.byref(R), 0, ws, need, None)
    assert f(*head, 0, 0.0, None, *tail, ev9, 9) == lib.MOE_E_ARG
    assert f(*head, 0, 0.0, None, *tail, ev9, -1) == lib.MOE_E_ARG
    assert f(*head, 0, 0.0, None, *tail, None, 2) == lib.MOE_E_ARG
    assert f(*head, 0, 0.0, None, *tail, ev_null, 2) == lib.MOE_E_ARG
    assert f(*head, 2, 0.0, None, *tail, ev9, 0) == lib.MOE_E_ARG
    assert f(ctypes.byref(dims), x, ctypes.byref(W), None, 1, 1e-3, None, *tail, ev9, 0) == lib.MOE_E_ARG
    # the instrumented call's own checks: workspace, aliasing
    assert f(*head, 0, 0.0, None, y, ctypes.byref(R), 0, ws, need - 1, None, ev9, 0) == lib.MOE_E_WORKSPACE
    assert f(*head, 1, 1e-3, 0x20004, *tail, ev9, 0) == lib.MOE_E_ALIAS


def test_quantize_int4_host_checks(lib):
    """moe_quantize_int4 rejects, before any launch: bad sizes, other dtypes, K
    not a multiple of 128, null pointers and overlapping outputs."""
    q = lib.LIB.moe_quantize_int4
    bf, f32 = lib.MOE_BF16, lib.MOE_F32
    assert q(bf, 0x1000, -1, 128, 0x100000, 0x200000, None) == lib.MOE_E_ARG
    assert q(bf, 0x1000, 4, 0, 0x100000, 0x200000, None) == lib.MOE_E_ARG
    assert q(lib.MOE_INT4_G128, 0x1000, 4, 128, 0x100000, 0x200000, None) == lib.MOE_E_UNSUPPORTED
    assert q(bf, 0x1000, 4, 192, 0x100000, 0x200000, None) == lib.MOE_E_UNSUPPORTED
    assert q(bf, 0x1000, 0, 128, None, None, None) == lib.MOE_OK          # nothing to do
    assert q(bf, None, 4, 128, 0x100000, 0x200000, None) == lib.MOE_E_ARG
    assert q(f32, 0x1000, 4, 128, None, 0x200000, None) == lib.MOE_E_ARG
    # w is 4 x 128 bf16 = 1 KiB at 0x1000: packed inside it overlaps
    assert q(bf, 0x1000, 4, 128, 0x1200, 0x200000, None) == lib.MOE_E_ALIAS
    # packed (256 B) and scales (8 B) overlapping each other
    assert q(bf, 0x1000, 4, 128, 0x100000, 0x100080, None) == lib.MOE_E_ALIAS


def test_int4_requires_top1_bf16(lib):
    for act, k in (("f32", 1), ("bf16", 2)):
        d = lib.make_dims(8, 1024, 64, 512, 2048, k, act, w_routed="int4")
        assert lib.moe_workspace_bytes(d) == 0


def test_int4_shapes_decode_and_prefill(lib):
    """Up to 64 tokens at the NanoColibri shape the int4 path is the decode
    kernels; every other batch (above 64 tokens, or another shape) runs the
    prefill's grouped GEMMs, for any shape whose F is a multiple of 128.
    Its GEMMs read the packed experts directly while a tile's scales fit in
    LDS (d / 128 and F / 128 at most 24): then it needs no more workspace than
    the bf16 layer; beyond that it keeps dequantised copies of the experts."""
    ws = lambda T, d=1024, E=64, F=512, Fs=2048: lib.moe_workspace_bytes(
        lib.make_dims(T, d, E, F, Fs, 1, "bf16", w_routed="int4"))
    assert ws(64) > 0 and ws(65) > 0 and ws(4096) > 0
    other = dict(d=256, E=8, F=128, Fs=256)                         # not the decode shape: the prefill path
    assert ws(64, **other) == lib.moe_workspace_bytes(lib.make_dims(64, 256, 8, 128, 256, 1, "bf16"))
    assert ws(1, **other) > 0 and ws(65, **other) > 0
    assert ws(65, F=192) == 0 and ws(8, F=192) == 0                 # groups of 128 along F
    bf16_layer = lib.moe_workspace_bytes(lib.make_dims(4096, 1024, 64, 512, 2048, 1, "bf16"))
    assert ws(4096) == bf16_layer
    long_d = lambda T: lib.moe_workspace_bytes(lib.make_dims(T, 3200, 8, 128, 256, 1, "bf16", w_routed="int4"))
    bf16_long = lib.moe_workspace_bytes(lib.make_dims(100, 3200, 8, 128, 256, 1, "bf16"))
    assert long_d(100) >= bf16_long + 8 * 3 * 3200 * 128 * 2     # 25 scale groups along d: copies


def test_library_has_no_undefined_kernel_stubs():
    """Every kernel the library launches is defined in it (a host-side launch
    stub left undefined only fails when the library is loaded on a GPU machine)."""
    import subprocess
    out = subprocess.run(["nm", "-D", LIBPATH], stdout=subprocess.PIPE, text=True).stdout
    undefined = [l for l in out.splitlines() if " U " in l and "fgmoe" in l]
    assert not undefined, undefined


def test_block_host_checks(lib):
    """moe_forward_block rejects, before any launch: fp32 activations, a null
    norm scale, a negative eps, a short workspace, h_out overlapping h."""
    W = lib.MoeWeights(*[0x10000000 + i * 0x1000000 for i in range(7)])
    R = lib.MoeRouting(*[0x40000000 + i * 0x1000000 for i in range(6)])
    h, h_out, g, ws = 0x60000000, 0x70000000, 0x5f000000, 0x80000000

    def call(dims, h_, g_, eps, out, ws_bytes):
        return lib.LIB.moe_forward_block(ctypes.byref(dims), h_, g_, eps, ctypes.byref(W), 0x50000000, out,
                                         ctypes.byref(R), ws, ws_bytes, None)

    f32 = lib.make_dims(16, 128, 8, 64, 256, 2, "f32")
    assert call(f32, h, g, 1e-6, h_out, 1 << 30) == lib.MOE_E_UNSUPPORTED
    dims = lib.make_dims(16, 128, 8, 64, 256, 2, "bf16")
    need = lib.moe_workspace_bytes(dims)
    assert call(dims, h, None, 1e-6, h_out, need) == lib.MOE_E_ARG
    assert call(dims, h, g, -1.0, h_out, need) == lib.MOE_E_ARG
    assert call(dims, h, g, 1e-6, h_out, need - 1) == lib.MOE_E_WORKSPACE
    assert call(dims, h, g, 1e-6, h + 64, need) == lib.MOE_E_ALIAS


def test_pack_routed_host_checks(lib):
    moe = lib
    import ctypes
    f = moe.LIB.moe_pack_routed_bf16
    d = moe.make_dims(0, 1024, 64, 512, 2048, 2, "bf16")
    gu, dn = 0x10000000, 0x20000000
    assert f(ctypes.byref(d), None, dn, 0x30000000, 0x40000000, None) == moe.MOE_E_ARG
    assert f(ctypes.byref(d), gu, dn, gu, 0x40000000, None) == moe.MOE_E_ALIAS          # output over its input
    assert f(ctypes.byref(moe.make_dims(0, 1024, 64, 512, 2048, 2, "f32")), gu, dn, 0x30000000, 0x40000000,
             None) == moe.MOE_E_UNSUPPORTED
    assert f(ctypes.byref(moe.make_dims(0, 384, 64, 512, 2048, 2, "bf16")), gu, dn, 0x30000000, 0x40000000,
             None) == moe.MOE_E_UNSUPPORTED                                               # d % 256
    assert f(ctypes.byref(moe.make_dims(0, 1024, 64, 192, 2048, 2, "bf16")), gu, dn, 0x30000000, 0x40000000,
             None) == moe.MOE_E_UNSUPPORTED                                               # F % 128
    staged = moe.make_dims(4096, 1024, 64, 512, 2048, 2, "bf16", w_routed="bf16_staged")
    assert moe.moe_workspace_bytes(staged) > 0
    assert moe.moe_workspace_bytes(staged, training=True) == 0                           # inference only
    assert moe.moe_workspace_bytes(moe.make_dims(4096, 1024, 64, 512, 2048, 2, "f32", w_routed="bf16_staged")) == 0


def test_noalloc_refuses_what_does_not_fit(lib):
    """moe_forward_noalloc checks the dims and the size of their workspace
    against its static array before it touches any device state, so these
    refusals need no GPU."""
    f = lib.LIB.moe_forward_noalloc
    W = lib.MoeWeights(0x100000, 0x200000, 0x300000, None, None, 0x400000, 0x500000)
    R = lib.MoeRouting(*[0x40000000 + i * 0x1000000 for i in range(6)])
    big = lib.make_dims(4096, 1024, 64, 512, 2048, 2, "bf16")
    assert lib.moe_workspace_bytes(big) > lib.MOE_NOALLOC_SCRATCH_BYTES
    assert f(ctypes.byref(big), 0x1000, ctypes.byref(W), 0x2000, 0x3000, ctypes.byref(R), None) == lib.MOE_E_WORKSPACE
    bad = lib.make_dims(16, 1024, 65, 512, 2048, 2, "bf16")
    assert f(ctypes.byref(bad), 0x1000, ctypes.byref(W), 0x2000, 0x3000, ctypes.byref(R), None) == lib.MOE_E_UNSUPPORTED
    fits = lib.make_dims(500, 1024, 64, 512, 2048, 2, "bf16")
    assert lib.moe_workspace_bytes(fits) <= lib.MOE_NOALLOC_SCRATCH_BYTES


def test_weights_struct_carries_the_next_layer(lib, monkeypatch):
    """moe_weights ends with `next`, a pointer to another moe_weights (the
    next-layer hint): the binding lays it out as eight pointers and fills
    `next` from a nested weights dict, keeping that struct alive with it.
    (Stand-in device addresses: the binding's pointer helper accepts only GPU
    tensors.)"""
    assert [f[0] for f in lib.MoeWeights._fields_] == list(lib.WEIGHT_FIELDS) + ["next"]
    assert ctypes.sizeof(lib.MoeWeights) == 8 * ctypes.sizeof(ctypes.c_void_p)
    monkeypatch.setattr(lib, "_ptr", lambda a: a)
    cur = {f: 0x10000 * (i + 1) for i, f in enumerate(lib.WEIGHT_FIELDS)}
    nxt = {f: 0x1000000 * (i + 1) for i, f in enumerate(lib.WEIGHT_FIELDS)}
    w = lib._struct(lib.MoeWeights, lib.WEIGHT_FIELDS, dict(cur, next=nxt))
    assert w.w_router == cur["w_router"]
    assert w.next == ctypes.addressof(w._next)
    n = lib.MoeWeights.from_address(w.next)
    for f in lib.WEIGHT_FIELDS:
        assert getattr(n, f) == nxt[f], f
    assert n.next is None                    # the hinted layer names no further layer
    assert lib._struct(lib.MoeWeights, lib.WEIGHT_FIELDS, cur).next is None
