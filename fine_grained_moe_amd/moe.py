"""Python binding of libfgmoe.so, the gfx950 MoE-layer library (include/moe.h).

Argument marshalling only: every step of the layer runs in the library's HIP
kernels.  torch provides device memory and the current stream.  Importing
this module loads the library and raises if it is missing; there is no other
implementation to fall back to.

The functions carry the C names: moe_workspace_bytes, moe_route, moe_forward,
moe_forward_bias_step, moe_forward_block, moe_bias_update, moe_bias_update_stats,
moe_backward, moe_quantize_int4, moe_pack_routed_bf16, moe_forward_cached, moe_cache_create, moe_cache_prepare,
moe_cache_state, moe_cache_destroy, moe_forward_events (instrumentation), moe_status_str.  Weights, routing buffers and
gradients are passed as dicts of torch tensors keyed by the C field names.
"""
from __future__ import annotations

import ctypes
import os
from typing import Dict, Optional

import torch  # first: the library binds to the HIP runtime torch has loaded

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libfgmoe.so")

MOE_OK, MOE_E_ARG, MOE_E_UNSUPPORTED, MOE_E_WORKSPACE, MOE_E_ALIAS, MOE_E_DEVICE = range(6)
MOE_F32, MOE_BF16, MOE_INT4_G128, MOE_BF16_STAGED = 0, 1, 2, 3
MOE_CACHE_DRY_RUN, MOE_CACHE_COPY_FILLS = 1, 2
MOE_NOALLOC_SCRATCH_BYTES = 8 << 20      # the static workspace of moe_forward_noalloc

DTYPES = {"f32": MOE_F32, "bf16": MOE_BF16, "int4": MOE_INT4_G128, "bf16_staged": MOE_BF16_STAGED}
TORCH_DTYPE = {MOE_F32: torch.float32, MOE_BF16: torch.bfloat16}

WEIGHT_FIELDS = ("w_router", "w_gate_up", "w_down", "s_gate_up", "s_down", "w_sh_gate_up", "w_sh_down")
ROUTING_FIELDS = ("idx", "gate", "counts", "offsets", "perm", "pos")
GRAD_FIELDS = ("dw_router", "dw_gate_up", "dw_down", "dw_sh_gate_up", "dw_sh_down")


class MoeDims(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in ("T", "d", "E", "F", "Fs", "k", "act", "w_routed")]


class MoeWeights(ctypes.Structure):
    # next: another MoeWeights (the following layer's, a prefetch hint), or null
    _fields_ = [(n, ctypes.c_void_p) for n in WEIGHT_FIELDS] + [("next", ctypes.c_void_p)]


class MoeRouting(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in ROUTING_FIELDS]


class MoeGrads(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in GRAD_FIELDS]


class MoeError(RuntimeError):
    def __init__(self, code: int, where: str):
        super().__init__(f"{where}: {moe_status_str(code)} (status {code})")
        self.code = code


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing; build it with `python -m fine_grained_moe_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    P, I32, I64, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    dims_p = ctypes.POINTER(MoeDims)
    lib.moe_workspace_bytes.argtypes = [dims_p, ctypes.c_int]
    lib.moe_workspace_bytes.restype = SZ
    lib.moe_route.argtypes = [dims_p, P, P, P, ctypes.POINTER(MoeRouting), P, SZ, P]
    lib.moe_route.restype = ctypes.c_int
    lib.moe_forward.argtypes = [dims_p, P, ctypes.POINTER(MoeWeights), P, P, ctypes.POINTER(MoeRouting),
                                ctypes.c_int, P, SZ, P]
    lib.moe_forward.restype = ctypes.c_int
    lib.moe_forward_noalloc.argtypes = [dims_p, P, ctypes.POINTER(MoeWeights), P, P, ctypes.POINTER(MoeRouting), P]
    lib.moe_forward_noalloc.restype = ctypes.c_int
    lib.moe_forward_block.argtypes = [dims_p, P, P, ctypes.c_float, ctypes.POINTER(MoeWeights), P, P,
                                      ctypes.POINTER(MoeRouting), P, SZ, P]
    lib.moe_forward_block.restype = ctypes.c_int
    lib.moe_bias_update.argtypes = [I32, I64, P, ctypes.c_float, P, P]
    lib.moe_bias_update.restype = ctypes.c_int
    lib.moe_bias_update_stats.argtypes = [I32, I64, P, ctypes.c_float, P, P, P]
    lib.moe_bias_update_stats.restype = ctypes.c_int
    lib.moe_backward.argtypes = [dims_p, P, ctypes.POINTER(MoeWeights), ctypes.POINTER(MoeRouting), P, P,
                                 ctypes.POINTER(MoeGrads), P, SZ, P]
    lib.moe_backward.restype = ctypes.c_int
    lib.moe_forward_bias_step.argtypes = [dims_p, P, ctypes.POINTER(MoeWeights), P, ctypes.c_float, P, P,
                                          ctypes.POINTER(MoeRouting), ctypes.c_int, P, SZ, P]
    lib.moe_forward_bias_step.restype = ctypes.c_int
    lib.moe_forward_cached.argtypes = [dims_p, P, ctypes.POINTER(MoeWeights), P, I32, P, P,
                                       ctypes.POINTER(MoeRouting), P, SZ, P]
    lib.moe_forward_cached.restype = ctypes.c_int
    lib.moe_cache_create.argtypes = [dims_p, I32, ctypes.POINTER(MoeWeights), ctypes.POINTER(MoeWeights), P, I32,
                                     ctypes.POINTER(ctypes.c_void_p)]
    lib.moe_cache_create.restype = ctypes.c_int
    lib.moe_cache_prepare.argtypes = [P, P, P, ctypes.POINTER(I32)]
    lib.moe_cache_prepare.restype = ctypes.c_int
    lib.moe_cache_state.argtypes = [P, P, P]
    lib.moe_cache_state.restype = ctypes.c_int
    lib.moe_cache_destroy.argtypes = [P]
    lib.moe_cache_destroy.restype = None
    lib.moe_quantize_int4.argtypes = [I32, P, I64, I32, P, P, P]
    lib.moe_quantize_int4.restype = ctypes.c_int
    lib.moe_pack_routed_bf16.argtypes = [ctypes.POINTER(MoeDims), P, P, P, P, P]
    lib.moe_pack_routed_bf16.restype = ctypes.c_int
    lib.moe_forward_events.argtypes = [dims_p, P, ctypes.POINTER(MoeWeights), P, I32, ctypes.c_float, P, P,
                                       ctypes.POINTER(MoeRouting), ctypes.c_int, P, SZ, P,
                                       ctypes.POINTER(ctypes.c_void_p), I32]
    lib.moe_forward_events.restype = ctypes.c_int
    lib.moe_status_str.argtypes = [ctypes.c_int]
    lib.moe_status_str.restype = ctypes.c_char_p
    return lib


LIB = _load()


def moe_status_str(code: int) -> str:
    return LIB.moe_status_str(int(code)).decode()


def make_dims(T: int, d: int, E: int, F: int, Fs: int, k: int, act: str = "bf16", w_routed: Optional[str] = None) -> MoeDims:
    a = DTYPES[act]
    return MoeDims(T, d, E, F, Fs, k, a, DTYPES[w_routed] if w_routed else a)


def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"expected a torch tensor, got {type(t).__name__}")
    if not t.is_contiguous():
        raise ValueError("tensors passed to the MoE library must be contiguous")
    if t.numel() and t.device.type != "cuda":
        raise ValueError("tensors passed to the MoE library must be on the GPU")
    return t.data_ptr() if t.numel() else None


def _stream(stream) -> int:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _host_ptr(t) -> Optional[int]:
    """A pinned host tensor (the expert cache's source of copies)."""
    if t is None:
        return None
    if not isinstance(t, torch.Tensor) or t.device.type != "cpu" or not t.is_contiguous() or not t.is_pinned():
        raise ValueError("the expert cache's host copy must be contiguous pinned CPU tensors")
    return t.data_ptr()


def _struct(cls, fields, tensors: Dict[str, torch.Tensor]):
    s = cls(*[_ptr(tensors.get(f)) for f in fields])
    nxt = tensors.get("next") if cls is MoeWeights else None
    if nxt is not None:
        # the following layer's weights (a prefetch hint); kept alive with s
        s._next = _struct(MoeWeights, WEIGHT_FIELDS, nxt)
        s.next = ctypes.addressof(s._next)
    return s


def _check(code: int, where: str) -> None:
    if code != MOE_OK:
        raise MoeError(code, where)


def moe_workspace_bytes(dims: MoeDims, training: bool = False) -> int:
    return int(LIB.moe_workspace_bytes(ctypes.byref(dims), int(bool(training))))


def moe_route(dims: MoeDims, x, w_router, bias, routing: Dict[str, torch.Tensor], ws, stream=None) -> None:
    r = _struct(MoeRouting, ROUTING_FIELDS, routing)
    _check(LIB.moe_route(ctypes.byref(dims), _ptr(x), _ptr(w_router), _ptr(bias), ctypes.byref(r), _ptr(ws),
                         ws.numel() * ws.element_size(), _stream(stream)), "moe_route")


def moe_forward(dims: MoeDims, x, weights: Dict[str, torch.Tensor], bias, y, routing: Dict[str, torch.Tensor],
                ws, training: bool = False, stream=None) -> None:
    w = _struct(MoeWeights, WEIGHT_FIELDS, weights)
    r = _struct(MoeRouting, ROUTING_FIELDS, routing)
    _check(LIB.moe_forward(ctypes.byref(dims), _ptr(x), ctypes.byref(w), _ptr(bias), _ptr(y), ctypes.byref(r),
                           int(bool(training)), _ptr(ws), ws.numel() * ws.element_size(), _stream(stream)),
           "moe_forward")


def moe_forward_noalloc(dims: MoeDims, x, weights: Dict[str, torch.Tensor], bias, y,
                        routing: Dict[str, torch.Tensor], stream=None) -> None:
    """moe_forward on the library's static device workspace (no workspace
    argument, nothing allocated; inference only)."""
    w = _struct(MoeWeights, WEIGHT_FIELDS, weights)
    r = _struct(MoeRouting, ROUTING_FIELDS, routing)
    _check(LIB.moe_forward_noalloc(ctypes.byref(dims), _ptr(x), ctypes.byref(w), _ptr(bias), _ptr(y),
                                   ctypes.byref(r), _stream(stream)), "moe_forward_noalloc")


def moe_forward_bias_step(dims: MoeDims, x, weights: Dict[str, torch.Tensor], bias, gamma: float, stats, y,
                          routing: Dict[str, torch.Tensor], ws, training: bool = False, stream=None) -> None:
    """moe_forward with bias, then the bias step on bias (in place) and, with a
    stats tensor (float32, >= 4 elements; None skips it), the balance figures."""
    w = _struct(MoeWeights, WEIGHT_FIELDS, weights)
    r = _struct(MoeRouting, ROUTING_FIELDS, routing)
    _check(LIB.moe_forward_bias_step(ctypes.byref(dims), _ptr(x), ctypes.byref(w), _ptr(bias), float(gamma),
                                     _ptr(stats), _ptr(y), ctypes.byref(r), int(bool(training)), _ptr(ws),
                                     ws.numel() * ws.element_size(), _stream(stream)), "moe_forward_bias_step")


def moe_forward_block(dims: MoeDims, h, norm_weight, eps: float, weights: Dict[str, torch.Tensor], bias, h_out,
                      routing: Dict[str, torch.Tensor], ws, stream=None) -> None:
    """h_out = h + MoE(RMSNorm(h) * norm_weight); norm_weight: [d] float32."""
    w = _struct(MoeWeights, WEIGHT_FIELDS, weights)
    r = _struct(MoeRouting, ROUTING_FIELDS, routing)
    _check(LIB.moe_forward_block(ctypes.byref(dims), _ptr(h), _ptr(norm_weight), float(eps), ctypes.byref(w),
                                 _ptr(bias), _ptr(h_out), ctypes.byref(r), _ptr(ws), ws.numel() * ws.element_size(),
                                 _stream(stream)), "moe_forward_block")


def moe_bias_update(E: int, total_assignments: int, counts, gamma: float, bias, stream=None) -> None:
    _check(LIB.moe_bias_update(int(E), int(total_assignments), _ptr(counts), float(gamma), _ptr(bias),
                               _stream(stream)), "moe_bias_update")


def moe_bias_update_stats(E: int, total_assignments: int, counts, gamma: float, bias, stats, stream=None) -> None:
    """stats: a float32 device tensor of (at least) 4 elements, e.g. one row of a [steps, 4] buffer."""
    _check(LIB.moe_bias_update_stats(int(E), int(total_assignments), _ptr(counts), float(gamma), _ptr(bias),
                                     _ptr(stats), _stream(stream)), "moe_bias_update_stats")


def moe_pack_routed_bf16(dims: MoeDims, w_gate_up, w_down, out_gate_up, out_down, stream=None) -> None:
    """Routed bf16 weights into the stage-major layout that w_routed = "bf16_staged" reads."""
    for a, b in ((w_gate_up, out_gate_up), (w_down, out_down)):
        if a.dtype != torch.bfloat16 or b.dtype != torch.bfloat16 or a.numel() != b.numel():
            raise MoeError(MOE_E_ARG, "moe_pack_routed_bf16")
    _check(LIB.moe_pack_routed_bf16(ctypes.byref(dims), _ptr(w_gate_up), _ptr(w_down), _ptr(out_gate_up),
                                    _ptr(out_down), _stream(stream)), "moe_pack_routed_bf16")


def moe_quantize_int4(w, packed, scales, stream=None) -> None:
    """w: [..., K] bf16 or float32 device tensor (rows = product of the leading
    dims); packed: uint8 [..., K/2]; scales: bf16 [..., K/128]."""
    dt = {torch.bfloat16: MOE_BF16, torch.float32: MOE_F32}.get(w.dtype)
    if dt is None:
        raise MoeError(MOE_E_UNSUPPORTED, "moe_quantize_int4")
    K = int(w.shape[-1])
    rows = w.numel() // K if K else 0
    if packed.numel() != rows * (K // 2) or scales.numel() != rows * (K // 128) or not w.is_contiguous():
        raise MoeError(MOE_E_ARG, "moe_quantize_int4")
    _check(LIB.moe_quantize_int4(dt, _ptr(w), rows, K, _ptr(packed), _ptr(scales), _stream(stream)),
           "moe_quantize_int4")


def moe_forward_cached(dims: MoeDims, x, weights: Dict[str, torch.Tensor], slot, n_slots: int, bias, y,
                       routing: Dict[str, torch.Tensor], ws, stream=None) -> None:
    w = _struct(MoeWeights, WEIGHT_FIELDS, weights)
    r = _struct(MoeRouting, ROUTING_FIELDS, routing)
    _check(LIB.moe_forward_cached(ctypes.byref(dims), _ptr(x), ctypes.byref(w), _ptr(slot), int(n_slots), _ptr(bias),
                                  _ptr(y), ctypes.byref(r), _ptr(ws), ws.numel() * ws.element_size(),
                                  _stream(stream)), "moe_forward_cached")


class ExpertCache:
    """The library's LRU expert cache (moe_cache_*).  host: dict of pinned CPU
    tensors (int4 fields of all E experts); dev: dict of device tensors of
    n_slots slots; slot: [E] int32 device tensor.  dry_run keeps only the
    bookkeeping; copy_fills fills misses with hipMemcpyAsync calls instead
    of one launch reading the host copy in place.  The tensors must outlive
    the cache."""

    def __init__(self, dims: MoeDims, n_slots: int, host=None, dev=None, slot=None, dry_run: bool = False,
                 copy_fills: bool = False):
        self._keep = (host, dev, slot)
        self.dry = bool(dry_run)
        hw = MoeWeights(*[_host_ptr((host or {}).get(f)) for f in WEIGHT_FIELDS])
        dw = _struct(MoeWeights, WEIGHT_FIELDS, dev or {})
        h = ctypes.c_void_p()
        _check(LIB.moe_cache_create(ctypes.byref(dims), int(n_slots), ctypes.byref(hw), ctypes.byref(dw),
                                    _ptr(slot) if slot is not None else None,
                                    (MOE_CACHE_DRY_RUN if dry_run else 0) | (MOE_CACHE_COPY_FILLS if copy_fills else 0),
                                    ctypes.byref(h)),
               "moe_cache_create")
        self.handle = h
        self.E = dims.E

    def prepare(self, counts_host, stream=None) -> int:
        import numpy as np
        c = np.ascontiguousarray(np.asarray(counts_host, dtype=np.int32))
        m = ctypes.c_int32(0)
        _check(LIB.moe_cache_prepare(self.handle, c.ctypes.data, 0 if self.dry else _stream(stream), ctypes.byref(m)),
               "moe_cache_prepare")
        return m.value

    def state(self):
        import numpy as np
        so = np.zeros(self.E, np.int32)
        hm = np.zeros(3, np.int64)
        _check(LIB.moe_cache_state(self.handle, so.ctypes.data, hm.ctypes.data), "moe_cache_state")
        self.zero_copy = bool(hm[2])
        return so, int(hm[0]), int(hm[1])

    def close(self) -> None:
        if self.handle:
            LIB.moe_cache_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def moe_backward(dims: MoeDims, x, weights: Dict[str, torch.Tensor], routing: Dict[str, torch.Tensor], dy, dx,
                 grads: Dict[str, torch.Tensor], ws, stream=None) -> None:
    w = _struct(MoeWeights, WEIGHT_FIELDS, weights)
    r = _struct(MoeRouting, ROUTING_FIELDS, routing)
    g = _struct(MoeGrads, GRAD_FIELDS, grads)
    _check(LIB.moe_backward(ctypes.byref(dims), _ptr(x), ctypes.byref(w), ctypes.byref(r), _ptr(dy), _ptr(dx),
                            ctypes.byref(g), _ptr(ws), ws.numel() * ws.element_size(), _stream(stream)),
           "moe_backward")


def moe_forward_events(dims: MoeDims, x, weights: Dict[str, torch.Tensor], bias, y, routing: Dict[str, torch.Tensor],
                       ws, events, bias_step: bool = False, gamma: float = 0.0, stats=None, training: bool = False,
                       stream=None) -> None:
    """Instrumentation: moe_forward (bias_step False) or moe_forward_bias_step
    (True) recording the raw hipEvent_t handles `events` (ints, at most 8) at
    the phase boundaries."""
    events = list(events or [])
    arr = (ctypes.c_void_p * max(1, len(events)))(*[int(e) for e in events])
    w = _struct(MoeWeights, WEIGHT_FIELDS, weights)
    r = _struct(MoeRouting, ROUTING_FIELDS, routing)
    _check(LIB.moe_forward_events(ctypes.byref(dims), _ptr(x), ctypes.byref(w), _ptr(bias), int(bool(bias_step)),
                                  float(gamma), _ptr(stats), _ptr(y), ctypes.byref(r), int(bool(training)), _ptr(ws),
                                  ws.numel() * ws.element_size(), _stream(stream), arr, len(events)),
           "moe_forward_events")


# ---------------------------------------------------------------- allocation helpers

def alloc_routing(dims: MoeDims, device="cuda") -> Dict[str, torch.Tensor]:
    T, k, E = dims.T, dims.k, dims.E
    i32 = dict(dtype=torch.int32, device=device)
    return dict(idx=torch.empty(T, k, **i32), gate=torch.empty(T, k, dtype=torch.float32, device=device),
                counts=torch.empty(E, **i32), offsets=torch.empty(E + 1, **i32),
                perm=torch.empty(T * k, **i32), pos=torch.empty(T, k, **i32))


def alloc_workspace(dims: MoeDims, training: bool = False, device="cuda") -> torch.Tensor:
    n = moe_workspace_bytes(dims, training)
    if n == 0:
        raise MoeError(MOE_E_UNSUPPORTED, "moe_workspace_bytes")
    return torch.empty(n, dtype=torch.uint8, device=device)


def alloc_grads(dims: MoeDims, device="cuda") -> Dict[str, torch.Tensor]:
    E, d, F, Fs = dims.E, dims.d, dims.F, dims.Fs
    f = dict(dtype=torch.float32, device=device)
    return dict(dw_router=torch.empty(E, d, **f), dw_gate_up=torch.empty(E, 2 * F, d, **f),
                dw_down=torch.empty(E, d, F, **f), dw_sh_gate_up=torch.empty(2 * Fs, d, **f),
                dw_sh_down=torch.empty(d, Fs, **f))
