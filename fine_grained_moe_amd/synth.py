"""Seeded synthetic inputs for the NanoColibri MoE layer workloads.

This module only draws random numbers and stores them in the dtypes the layer
takes.  It holds none of the layer's arithmetic (no routing, no expert FFN, no
bias rule, no quantiser): both the GPU path and the CPU oracle read its arrays,
and it imports neither.

Shapes follow the NanoColibri article ("A relay race of rented GPUs trained
NanoColibri's 2.7B MoE for $200", seventnews; opening section, architecture
paragraph): hidden 1024, 64 routed experts of width 512, top-2, one shared
expert of width 2048.  Value distributions are the workload recipe: x ~ N(0,1)
(optionally RMS-normalised per token), every weight ~ N(0, std 0.02), bias 0.

Every tensor is returned as float32 numpy values that are exactly
representable in the layer's activation dtype: for bf16 workloads each value
has already been rounded to bfloat16 (round to nearest, ties to even), so
converting it to torch.bfloat16 is exact and the oracle can read the same
values in float64.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional

import numpy as np

# Fixed order of the per-tensor random streams; a workload seed spawns one
# child stream per name so that adding a tensor never shifts another's values.
STREAMS = ("x", "w_router", "w_gate_up", "w_down", "w_sh_gate_up", "w_sh_down",
           "dy", "redraw", "int4")

WEIGHT_STD = 0.02
RMS_EPS = 1e-6


def round_to_bf16(a: np.ndarray) -> np.ndarray:
    """float32 -> nearest bfloat16 value (ties to even), returned as float32."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    bits = a.view(np.uint32).astype(np.uint64)
    lsb = (bits >> 16) & 1
    rounded = ((bits + 0x7FFF + lsb) >> 16) << 16
    return rounded.astype(np.uint32).view(np.float32).reshape(a.shape)


def bf16_bits(a: np.ndarray) -> np.ndarray:
    """Upper 16 bits of float32 values that are already bf16-exact."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    return (a.view(np.uint32) >> 16).astype(np.uint16)


def _streams(seed: int) -> dict:
    children = np.random.SeedSequence(seed).spawn(len(STREAMS))
    return {n: np.random.Generator(np.random.PCG64(c)) for n, c in zip(STREAMS, children)}


def _store(a: np.ndarray, act: str) -> np.ndarray:
    a = a.astype(np.float32)
    return round_to_bf16(a) if act == "bf16" else a


def _draw_x(rng: np.random.Generator, rows: int, d: int, rms_norm: bool, act: str) -> np.ndarray:
    x = rng.standard_normal((rows, d), dtype=np.float32)
    if rms_norm:
        ms = np.mean(x.astype(np.float64) ** 2, axis=1, keepdims=True)
        x = (x / np.sqrt(ms + RMS_EPS)).astype(np.float32)
    return _store(x, act)


@dataclass
class LayerInputs:
    """One MoE layer's weights, one batch of activations and the router bias.

    Layouts (row-major, the contraction dimension last, as the C ABI takes them):
      x            [T, d]
      w_router     [E, d]
      w_gate_up    [E, 2F, d]   rows 0..F-1 gate projection, F..2F-1 up projection
      w_down       [E, d, F]
      w_sh_gate_up [2Fs, d]     same split as w_gate_up
      w_sh_down    [d, Fs]
      bias         [E] float32
      dy           [T, d] (training workloads only)
    """
    T: int
    d: int
    E: int
    F: int
    Fs: int
    k: int
    act: str                      # "f32" or "bf16"
    seed: int
    rms_norm: bool
    x: np.ndarray
    w_router: np.ndarray
    w_gate_up: np.ndarray
    w_down: np.ndarray
    w_sh_gate_up: np.ndarray
    w_sh_down: np.ndarray
    bias: np.ndarray
    dy: Optional[np.ndarray] = None
    redraw_rounds: int = field(default=0)

    @property
    def total_assignments(self) -> int:
        return self.T * self.k


def make_layer(T: int, d: int, E: int, F: int, Fs: int, k: int, act: str, seed: int = 0,
               rms_norm: bool = True, with_dy: bool = False) -> LayerInputs:
    """Draw one workload.  Weights ~ N(0, 0.02); x ~ N(0,1), RMS-normalised if asked."""
    if act not in ("f32", "bf16"):
        raise ValueError(act)
    st = _streams(seed)
    x = _draw_x(st["x"], T, d, rms_norm, act)

    def w(name, shape):
        return _store(st[name].standard_normal(shape, dtype=np.float32) * np.float32(WEIGHT_STD), act)

    inp = LayerInputs(
        T=T, d=d, E=E, F=F, Fs=Fs, k=k, act=act, seed=seed, rms_norm=rms_norm, x=x,
        w_router=w("w_router", (E, d)),
        w_gate_up=w("w_gate_up", (E, 2 * F, d)),
        w_down=w("w_down", (E, d, F)),
        w_sh_gate_up=w("w_sh_gate_up", (2 * Fs, d)),
        w_sh_down=w("w_sh_down", (d, Fs)),
        bias=np.zeros(E, dtype=np.float32),
    )
    if with_dy:
        inp.dy = _store(st["dy"].standard_normal((T, d), dtype=np.float32), act)
    return inp


def redraw_rows(inp: LayerInputs, rows: np.ndarray) -> None:
    """Replace the given token rows of x with fresh draws (same recipe).

    Each call uses the next round of the workload's redraw stream, so a
    sequence of calls is reproducible from the seed alone.  Which rows to
    redraw is the caller's decision.
    """
    rows = np.asarray(rows, dtype=np.int64)
    if rows.size == 0:
        return
    ss = np.random.SeedSequence([inp.seed, 0x7E5D, inp.redraw_rounds])
    rng = np.random.Generator(np.random.PCG64(ss))
    inp.x[rows] = _draw_x(rng, rows.size, inp.d, inp.rms_norm, inp.act)
    inp.redraw_rounds += 1


def random_int4(E: int, N: int, K: int, seed: int = 0, group: int = 128):
    """Random int4 weights already in the packed container format.

    Returns (packed uint8 [E, N, K/2], scales float32 bf16-exact [E, N, K/group]).
    Nibble values are drawn from a rounded N(0, 2.5) clipped to [-8, 7] (two's
    complement, element 2i in the low nibble), scales from bf16(0.02*|N(2.8,0.3)|/7).
    Used where only the traffic matters (throughput runs); parity tests quantise
    N(0, 0.02) weights instead.
    """
    st = _streams(seed)["int4"]
    q = np.clip(np.rint(st.standard_normal((E, N, K), dtype=np.float32) * 2.5), -8, 7).astype(np.int8)
    nib = (q.astype(np.int16) & 0xF).astype(np.uint8)
    packed = (nib[..., 0::2] | (nib[..., 1::2] << 4)).astype(np.uint8)
    sc = np.abs(st.standard_normal((E, N, K // group), dtype=np.float32) * 0.3 + 2.8) * 0.02 / 7
    return packed, round_to_bf16(sc.astype(np.float32))


# The workloads.  Sizes only; the bias preset of the Zipf-skewed workload and
# the no-near-tie redraws are made by the tests with the oracle.
WORKLOADS = {
    # tiny fp32 correctness case: x ~ N(0,1) without RMS normalisation
    "tiny_f32": dict(T=64, d=128, E=8, F=64, Fs=256, k=2, act="f32", rms_norm=False),
    # one NanoColibri layer forward, batch 2 x seq 2048
    "layer_t4096": dict(T=4096, d=1024, E=64, F=512, Fs=2048, k=2, act="bf16", rms_norm=True),
    # Zipf-skewed routing stress, same layer shape
    "zipf_t16384": dict(T=16384, d=1024, E=64, F=512, Fs=2048, k=2, act="bf16", rms_norm=True),
    # training step, batch 16 x seq 2048
    "train_t32768": dict(T=32768, d=1024, E=64, F=512, Fs=2048, k=2, act="bf16", rms_norm=True),
    # top-1 serving decode (routed experts int4, shared expert bf16)
    "decode_t1": dict(T=1, d=1024, E=64, F=512, Fs=2048, k=1, act="bf16", rms_norm=True),
    "decode_t8": dict(T=8, d=1024, E=64, F=512, Fs=2048, k=1, act="bf16", rms_norm=True),
    "decode_t64": dict(T=64, d=1024, E=64, F=512, Fs=2048, k=1, act="bf16", rms_norm=True),
}


def make_workload(name: str, seed: int = 0, T: Optional[int] = None, with_dy: bool = False) -> LayerInputs:
    cfg = dict(WORKLOADS[name])
    if T is not None:
        cfg["T"] = T
    return make_layer(seed=seed, with_dy=with_dy, **cfg)
