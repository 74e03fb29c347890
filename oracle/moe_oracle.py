"""CPU oracle for the NanoColibri fine-grained MoE layer.  TEST INFRASTRUCTURE ONLY.

Only the tests, the package's smoke check and the CPU-baseline leg of the
benchmark may import this module.  The GPU library never calls it, and the two
share no code: the oracle reads the same seeded input arrays and nothing else.

It is the plain definition of the layer, evaluated in float64 from the exact
values of the (fp32, bf16 or dequantised int4) inputs, with no intermediate
rounding, no blocking and no fusion.  Library matmuls, sorts and reductions
serve as steps.

Source: the seventnews article "A relay race of rented GPUs trained
NanoColibri's 2.7B MoE for $200" (Chinese, Spanish and Arabic editions).
Citations below name its sections:
  * opening section, architecture paragraph: 64 routed experts of width 512 on
    hidden 1024 with top-2 routing, a shared expert of width 2048, a
    sigmoid-plus-bias router, and the per-layer bias nudge gamma*sign(target-load)
    following the DeepSeek-V3 recipe;
  * opening section, proof-of-loop paragraph: every token touches the
    always-resident shared expert plus a couple of routed experts; containers
    are int4;
  * "Relay training" section, top-2 paragraph: at top_k=1 the routing weight is
    a constant and the router gets no gradient; two winners competing restore
    the gradient; serving runs one expert per token; aux-loss-free balancing
    held, with a low dead-expert fraction;
  * "Relay training" section, baton paragraph: the read-only training
    dashboard shows expert balance.

Readings where the article is silent (each is listed with its reason in the
design notes of the repository):
  R1 expert FFN = SwiGLU without biases: FFN(x) = Wd (silu(Wg x) * (Wu x));
  R2 gate g_j = s_j / sum of the selected s (no extra scale), so k=1 gives g=1;
  R3 the bias only affects selection; gates use the plain sigmoid scores;
  R4 sign(0) = 0: an expert exactly at target keeps its bias;
  R5 target = T*k/E, compared exactly in integers: sign(T*k - E*load);
  R6 load = this batch's assignment count; the update follows the forward;
  R7 the new bias is one IEEE float32 add: fl32(b + gamma*sign);
  R8 top-k order: v = s + b descending, an exact tie goes to the lower expert;
  R9 the shared expert's output is added ungated; no residual, no norm;
  R10 int4: symmetric, groups of 128 along the contraction dim, scale =
      bf16(absmax/7), q = clamp(rne(w/scale), -8, 7), two's-complement
      nibbles, element 2i in the low nibble;
  R11 backward: exact derivatives with the selection held fixed; the router
      gradient flows only through the normalised gates;
  R19 expert balance of one batch = (dead fraction: experts with zero load
      over E; max load over the mean load T*k/E; entropy -sum p ln p of the
      load shares p = load/(T*k), 0 ln 0 = 0; that entropy over ln E, 1 for
      E = 1); a batch with no assignments reads (1, 0, 0, 0);
  R20 the MoE block around the layer (the article's 23 MoE layers of a
      pre-norm transformer): x = bf16(h / sqrt(mean(h^2) + 1e-6) * gamma)
      (RMSNorm with a learned per-channel scale gamma, eps as R13), and the
      block returns h + y, rounded once to the activation dtype.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

f64 = np.float64


# --------------------------------------------------------------------------
# scalar functions
# --------------------------------------------------------------------------

def sigmoid(z):
    """Logistic function 1 / (1 + e^-z) (architecture paragraph: sigmoid router)."""
    z = np.asarray(z, dtype=f64)
    return 1.0 / (1.0 + np.exp(-z))


def silu(z):
    """z * sigmoid(z), the SwiGLU activation (reading R1)."""
    z = np.asarray(z, dtype=f64)
    return z * sigmoid(z)


def dsilu(z):
    """d/dz silu(z) = sigmoid(z) * (1 + z * (1 - sigmoid(z)))."""
    z = np.asarray(z, dtype=f64)
    s = sigmoid(z)
    return s * (1.0 + z * (1.0 - s))


# --------------------------------------------------------------------------
# routing
# --------------------------------------------------------------------------

@dataclass
class Routing:
    idx: np.ndarray      # [T, k] int64, experts in selection order
    gate: np.ndarray     # [T, k] float64
    scores: np.ndarray   # [T, E] sigmoid scores s
    v: np.ndarray        # [T, E] selection keys s + b
    logits: np.ndarray   # [T, E]


def route(x, w_router, bias, k: int) -> Routing:
    """Sigmoid-plus-bias router with top-k selection.

    Architecture paragraph: the router is a sigmoid plus a bias.  Logits are
    x . W_r[e]; scores s = sigmoid(logits); the bias enters selection only
    (R3); the k experts with the largest s + b are taken, largest first, an
    exact tie going to the lower index (R8); gates are the selected scores
    normalised to sum to one (R2).
    """
    x = np.asarray(x, dtype=f64)
    W = np.asarray(w_router, dtype=f64)
    b = np.asarray(bias, dtype=f64)
    E = W.shape[0]
    if not (1 <= k <= E):
        raise ValueError("k must be in [1, E]")
    logits = x @ W.T
    s = sigmoid(logits)
    v = s + b[None, :]
    idx = select_topk(v, k)
    s_sel = np.take_along_axis(s, idx, axis=1)
    gate = s_sel / s_sel.sum(axis=1, keepdims=True)
    return Routing(idx=idx, gate=gate, scores=s, v=v, logits=logits)


def select_topk(v, k: int) -> np.ndarray:
    """The k largest keys of each row, largest first; an exact tie goes to the
    lower index (R8).  A stable sort of -v keeps equal keys in index order."""
    return np.argsort(-np.asarray(v, dtype=f64), axis=1, kind="stable")[:, :k]


def expert_counts(idx, E: int) -> np.ndarray:
    """load_e = number of (token, slot) assignments to expert e (R6)."""
    return np.bincount(np.asarray(idx).ravel(), minlength=E).astype(np.int64)


def expert_offsets(counts) -> np.ndarray:
    """Exclusive prefix sum of the loads: expert e's rows start at offsets[e]."""
    c = np.asarray(counts, dtype=np.int64)
    return np.concatenate([[0], np.cumsum(c)]).astype(np.int64)


def dispatch_order(idx, E: int):
    """Slots grouped by expert, ascending (token, slot) inside each expert.

    perm[slot] = t*k + j of the assignment in that slot; pos[t, j] = its slot.
    The order inside an expert does not change any result of the layer; this
    one is the stable order.
    """
    idx = np.asarray(idx)
    T, k = idx.shape
    flat = idx.ravel()
    perm = np.argsort(flat, kind="stable").astype(np.int64)
    pos = np.empty(T * k, dtype=np.int64)
    pos[perm] = np.arange(T * k)
    return perm, pos.reshape(T, k)


def topk_margin(v, k: int) -> np.ndarray:
    """Per token, the smallest gap between consecutive entries of the k+1
    largest selection keys (k largest when E == k).  Used to keep test inputs
    away from ties that a different summation order could flip."""
    v = np.asarray(v, dtype=f64)
    m = min(k + 1, v.shape[1])
    top = -np.sort(-v, axis=1)[:, :m]
    if m < 2:
        return np.full(v.shape[0], np.inf)
    return (top[:, :-1] - top[:, 1:]).min(axis=1)


# --------------------------------------------------------------------------
# experts and the layer
# --------------------------------------------------------------------------

def swiglu_ffn(X, Wg, Wu, Wd):
    """SwiGLU FFN (R1): Wd (silu(Wg x) * (Wu x)) for each row x of X.

    X [n, d]; Wg, Wu [F, d]; Wd [d, F]."""
    X = np.asarray(X, dtype=f64)
    a = X @ np.asarray(Wg, dtype=f64).T
    u = X @ np.asarray(Wu, dtype=f64).T
    return (silu(a) * u) @ np.asarray(Wd, dtype=f64).T


def split_gate_up(w_gate_up):
    """[..., 2F, d] -> (gate rows 0..F-1, up rows F..2F-1)."""
    F = w_gate_up.shape[-2] // 2
    return w_gate_up[..., :F, :], w_gate_up[..., F:, :]


def forward(x, w_router, w_gate_up, w_down, w_sh_gate_up, w_sh_down, bias, k: int):
    """The MoE layer output and its routing.

    y_t = Shared(x_t) + sum_j g_tj * Expert_{idx_tj}(x_t)

    Proof-of-loop paragraph: every token runs the always-resident shared
    expert (added ungated, R9) plus its routed experts; architecture
    paragraph: top-k of 64 experts of width 512; the top-2 paragraph names the
    routing weight that scales each routed expert's output.
    w_gate_up [E, 2F, d], w_down [E, d, F], w_sh_gate_up [2Fs, d], w_sh_down [d, Fs].
    """
    x = np.asarray(x, dtype=f64)
    r = route(x, w_router, bias, k)
    Wsg, Wsu = split_gate_up(np.asarray(w_sh_gate_up, dtype=f64))
    y = swiglu_ffn(x, Wsg, Wsu, w_sh_down)
    Wg, Wu = split_gate_up(np.asarray(w_gate_up, dtype=f64))
    Wd = np.asarray(w_down, dtype=f64)
    E = Wd.shape[0]
    for e in range(E):
        t, j = np.nonzero(r.idx == e)       # a token selects an expert at most once
        if t.size:
            y[t] += r.gate[t, j][:, None] * swiglu_ffn(x[t], Wg[e], Wu[e], Wd[e])
    return y, r


def bias_update(bias, counts, total_assignments: int, gamma: float) -> np.ndarray:
    """Aux-loss-free balancing step (architecture paragraph: bias += gamma *
    sign(target - load), DeepSeek-V3 recipe).

    target = T*k/E is compared exactly as sign(T*k - E*load) (R5), sign(0) = 0
    (R4), and the result is one float32 addition b + gamma*sign (R7).
    """
    b = np.asarray(bias, dtype=np.float32)
    c = np.asarray(counts, dtype=np.int64)
    E = c.size
    sgn = np.sign(np.int64(total_assignments) - np.int64(E) * c).astype(np.float32)
    return (b + np.float32(gamma) * sgn).astype(np.float32)


RMS_EPS = 1e-6


def rms_norm(h, gamma, eps: float = RMS_EPS) -> np.ndarray:
    """Pre-norm of the MoE block (R20): each token row of h divided by its root
    mean square (plus eps under the root), times gamma, rounded to bf16."""
    h = np.asarray(h, dtype=f64)
    ms = np.mean(h * h, axis=-1, keepdims=True)
    return to_bf16_nearest(h / np.sqrt(ms + eps) * np.asarray(gamma, dtype=f64))


def block_forward(h, gamma, w_router, w_gate_up, w_down, w_sh_gate_up, w_sh_down, bias, k: int,
                  eps: float = RMS_EPS):
    """The MoE block (R20): h + MoE(rms_norm(h)).  Returns (h_out, x, routing),
    h_out exact (float64), x the bf16 values the layer reads."""
    x = rms_norm(h, gamma, eps)
    y, routing = forward(x, w_router, w_gate_up, w_down, w_sh_gate_up, w_sh_down, bias, k)
    return np.asarray(h, dtype=f64) + y, x, routing


def load_stats(counts, total_assignments: int) -> np.ndarray:
    """Expert-balance telemetry of one batch (R19): [dead fraction, max/mean
    load, load entropy in nats, entropy / ln E], from the per-expert loads.

    The article's top-2 paragraph ("Relay training" section) reports that the
    dead-expert fraction stayed low under aux-loss-free balancing, and its
    baton paragraph puts expert balance on the training dashboard; it defines
    neither figure, so these are the plain readings of R19.
    """
    c = np.asarray(counts, dtype=f64)
    E = c.size
    total = f64(total_assignments)
    dead = f64(np.count_nonzero(c == 0)) / E
    if total <= 0:
        return np.array([1.0, 0.0, 0.0, 0.0], dtype=f64)
    p = c / total
    nz = p[p > 0]
    ent = f64(-np.sum(nz * np.log(nz)))
    return np.array([dead, c.max() / (total / E), ent, ent / np.log(E) if E > 1 else 1.0], dtype=f64)


# --------------------------------------------------------------------------
# backward (training workload)
# --------------------------------------------------------------------------

@dataclass
class Grads:
    dx: np.ndarray
    dw_router: np.ndarray
    dw_gate_up: np.ndarray
    dw_down: np.ndarray
    dw_sh_gate_up: np.ndarray
    dw_sh_down: np.ndarray


def _swiglu_ffn_backward(X, Wg, Wu, Wd, dY):
    """Gradients of Y = Wd (silu(Wg x) * (Wu x)) for each row; returns
    (dX, dWg, dWu, dWd, Y)."""
    a = X @ Wg.T
    u = X @ Wu.T
    h = silu(a) * u
    Y = h @ Wd.T
    dWd = dY.T @ h
    dh = dY @ Wd
    da = dh * u * dsilu(a)
    du = dh * silu(a)
    dX = da @ Wg + du @ Wu
    return dX, da.T @ X, du.T @ X, dWd, Y


def backward(x, w_router, w_gate_up, w_down, w_sh_gate_up, w_sh_down, routing: Routing, dy) -> Grads:
    """Exact derivatives of the layer with the selection held fixed (R11).

    The routed expert outputs o_j enter y scaled by g_j, so dL/do_j = g_j dy
    and dL/dg_j = <dy, o_j>.  With g_j = s_j / S (S = sum of selected s),
    dL/ds_i = (dL/dg_i - sum_j g_j dL/dg_j) / S for a selected i, and
    dL/dlogit_i = dL/ds_i * s_i (1 - s_i); unselected experts and the bias get
    nothing.  The "Relay training" section's top-2 paragraph states the
    consequence checked in the tests: with k = 1, g = 1 and the router
    gradient vanishes.
    """
    x = np.asarray(x, dtype=f64)
    dy = np.asarray(dy, dtype=f64)
    Wr = np.asarray(w_router, dtype=f64)
    Wsg, Wsu = split_gate_up(np.asarray(w_sh_gate_up, dtype=f64))
    Wsd = np.asarray(w_sh_down, dtype=f64)
    Wg, Wu = split_gate_up(np.asarray(w_gate_up, dtype=f64))
    Wd = np.asarray(w_down, dtype=f64)
    E, d, F = Wd.shape
    T, k = routing.idx.shape

    dx, dWsg, dWsu, dWsd, _ = _swiglu_ffn_backward(x, Wsg, Wsu, Wsd, dy)
    dWg = np.zeros_like(Wg)
    dWu = np.zeros_like(Wu)
    dWd = np.zeros_like(Wd)
    dg = np.zeros((T, k), dtype=f64)
    for e in range(E):
        t, j = np.nonzero(routing.idx == e)
        if t.size == 0:
            continue
        g = routing.gate[t, j][:, None]
        dX_e, dWg[e], dWu[e], dWd[e], o = _swiglu_ffn_backward(x[t], Wg[e], Wu[e], Wd[e], g * dy[t])
        dx[t] += dX_e
        dg[t, j] = np.sum(dy[t] * o, axis=1)

    s_sel = np.take_along_axis(routing.scores, routing.idx, axis=1)
    S = s_sel.sum(axis=1, keepdims=True)
    ds = (dg - np.sum(routing.gate * dg, axis=1, keepdims=True)) / S
    dl_sel = ds * s_sel * (1.0 - s_sel)
    dlogits = np.zeros((T, E), dtype=f64)
    np.put_along_axis(dlogits, routing.idx, dl_sel, axis=1)
    dWr = dlogits.T @ x
    dx += dlogits @ Wr
    return Grads(dx=dx, dw_router=dWr,
                 dw_gate_up=np.concatenate([dWg, dWu], axis=1), dw_down=dWd,
                 dw_sh_gate_up=np.concatenate([dWsg, dWsu], axis=0), dw_sh_down=dWsd)


# --------------------------------------------------------------------------
# int4 container (reading R10) and top-1 serving
# --------------------------------------------------------------------------

INT4_GROUP = 128


def to_bf16_nearest(v) -> np.ndarray:
    """Round float64 values to the nearest bfloat16 (8 significant bits), ties
    to even.  Normal range only, which is all the int4 scales need."""
    v = np.asarray(v, dtype=f64)
    m, e = np.frexp(v)                       # v = m * 2^e, 0.5 <= |m| < 1
    return np.ldexp(np.rint(m * 256.0) / 256.0, e)


def quantize_int4(w, group: int = INT4_GROUP):
    """w [..., N, K] -> (packed uint8 [..., N, K/2], scales float64 [..., N, K/group]).

    Symmetric per-group quantisation along K: scale = bf16(absmax / 7),
    q = clamp(rne(w / scale), -8, 7) (q = 0 for an all-zero group).
    """
    w = np.asarray(w, dtype=f64)
    *lead, N, K = w.shape
    if K % group:
        raise ValueError("K must be a multiple of the group size")
    g = w.reshape(*lead, N, K // group, group)
    scale = to_bf16_nearest(np.abs(g).max(axis=-1) / 7.0)
    safe = np.where(scale == 0, 1.0, scale)
    q = np.clip(np.rint(g / safe[..., None]), -8, 7)
    q = np.where(scale[..., None] == 0, 0, q).astype(np.int64).reshape(*lead, N, K)
    nib = (q & 0xF).astype(np.uint8)
    packed = nib[..., 0::2] | (nib[..., 1::2] << 4)
    return packed.astype(np.uint8), scale


def unpack_int4(packed) -> np.ndarray:
    """packed uint8 [..., K/2] -> int64 q [..., K] in [-8, 7]."""
    p = np.asarray(packed, dtype=np.uint8)
    lo = (p & 0xF).astype(np.int64)
    hi = (p >> 4).astype(np.int64)
    q = np.stack([lo, hi], axis=-1).reshape(*p.shape[:-1], p.shape[-1] * 2)
    return np.where(q >= 8, q - 16, q)


def dequantize_int4(packed, scales, group: int = INT4_GROUP) -> np.ndarray:
    """w = q * scale, exact in float64."""
    q = unpack_int4(packed).astype(f64)
    sc = np.repeat(np.asarray(scales, dtype=f64), group, axis=-1)
    return q * sc


def forward_int4_top1(x, w_router, q_gate_up, s_gate_up, q_down, s_down, w_sh_gate_up, w_sh_down, bias):
    """Top-1 serving: the routed experts are int4 (R10); one expert per token
    with gate exactly 1 ("Relay training" section, top-2 paragraph: serving
    runs one expert per token; proof-of-loop paragraph: int4 containers)."""
    return forward(x, w_router, dequantize_int4(q_gate_up, s_gate_up), dequantize_int4(q_down, s_down),
                   w_sh_gate_up, w_sh_down, bias, k=1)
