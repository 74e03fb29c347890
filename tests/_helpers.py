"""Shared test helpers: input preparation with the oracle, GPU upload, error metrics.

Decisions that need the layer's arithmetic (which rows sit too close to a
top-k tie, the Zipf bias preset) are taken here with the CPU oracle; the
seeded generator only draws numbers.
"""
from __future__ import annotations

import numpy as np

import oracle.moe_oracle as om
from fine_grained_moe_amd import synth

NEAR_TIE = 1e-3   # minimum fp64 gap between consecutive top-(k+1) keys


def rel_fro(a, b) -> float:
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    nb = np.linalg.norm(b)
    return float(np.linalg.norm(a - b) / (nb if nb > 0 else 1.0))


def row_rel_max(a, b) -> float:
    """Largest per-row relative error max_t ||a_t - b_t|| / ||b_t|| over the
    token rows (the last axis is the row); a row whose reference is zero must
    be zero.  A localised fault (one wrong MFMA tile, one wrong column band of
    a ragged tile) that the whole-tensor norm would average away shows here."""
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    a = a.reshape(-1, a.shape[-1])
    b = b.reshape(-1, b.shape[-1])
    if a.shape[0] == 0:
        return 0.0
    num = np.linalg.norm(a - b, axis=1)
    den = np.linalg.norm(b, axis=1)
    zero = den == 0
    r = np.where(zero, np.where(num == 0, 0.0, np.inf), num / np.where(zero, 1.0, den))
    return float(r.max())


def check_close(a, b, act: str, what: str = "", tol=None) -> float:
    """The output bar: relative Frobenius error over the whole tensor within
    the layer's tolerance (1e-2 bf16, 1e-4 fp32), and every token row within
    three times that.  Returns the whole-tensor error."""
    tol = {"f32": 1e-4, "bf16": 1e-2}[act] if tol is None else tol
    err = rel_fro(a, b)
    row = row_rel_max(a, b)
    print(f"{what} rel_fro = {err:.3e}, worst row {row:.3e}", flush=True)
    assert err <= tol, (what, err)
    assert row <= 3 * tol, (what, "worst row", row)
    return err


def scores(inp: synth.LayerInputs) -> np.ndarray:
    """Sigmoid scores of every (token, expert) from the oracle's router."""
    return om.route(inp.x, inp.w_router, np.zeros(inp.E, np.float32), inp.k).scores


def bias_sequence(inp: synth.LayerInputs, b0: np.ndarray, steps: int, gamma: float = 1e-3):
    """Oracle bias after 0..steps balancing steps on a fixed batch."""
    s = scores(inp)
    out = [np.asarray(b0, np.float32)]
    for _ in range(steps):
        r_idx = om.select_topk(s + out[-1].astype(np.float64), inp.k)
        c = om.expert_counts(r_idx, inp.E)
        out.append(om.bias_update(out[-1], c, inp.T * inp.k, gamma))
    return out


def remove_near_ties(inp: synth.LayerInputs, bias_states=None, steps_after: int = 0, max_rounds: int = 20) -> int:
    """Redraw token rows whose top-(k+1) keys come within NEAR_TIE of a tie,
    for every bias state the test will use, until none is left.  Returns the
    number of rows redrawn."""
    total = 0
    for _ in range(max_rounds):
        states = bias_states if bias_states is not None else [inp.bias]
        if steps_after:
            states = bias_sequence(inp, states[0], steps_after)
        s = scores(inp)
        bad = np.zeros(inp.T, dtype=bool)
        for b in states:
            bad |= om.topk_margin(s + np.asarray(b, np.float64), inp.k) < NEAR_TIE
        if not bad.any():
            return total
        total += int(bad.sum())
        synth.redraw_rows(inp, np.nonzero(bad)[0])
    raise RuntimeError("near-tie redraw did not converge")


def zipf_bias(inp: synth.LayerInputs, iters: int = 400) -> np.ndarray:
    """Bias preset that makes the expected load follow Zipf(1) over the experts
    (expert 0 hottest): iterate b_e += eta * sign(T*k*p_e - load_e) on this
    batch, eta = 0.02 * 2^-(it // 100)."""
    E = inp.E
    p = 1.0 / np.arange(1, E + 1)
    p /= p.sum()
    target = inp.T * inp.k * p
    s = scores(inp)
    b = np.zeros(E, np.float32)
    for it in range(iters):
        idx = om.select_topk(s + b.astype(np.float64), inp.k)
        load = om.expert_counts(idx, E)
        eta = np.float32(0.02 * 2.0 ** -(it // 100))
        b = (b + eta * np.sign(target - load).astype(np.float32)).astype(np.float32)
    return b


def oracle_forward(inp: synth.LayerInputs, bias=None):
    b = inp.bias if bias is None else bias
    return om.forward(inp.x, inp.w_router, inp.w_gate_up, inp.w_down, inp.w_sh_gate_up, inp.w_sh_down, b, inp.k)


# ---------------------------------------------------------------- GPU side

def to_gpu(inp: synth.LayerInputs):
    import torch
    dt = torch.bfloat16 if inp.act == "bf16" else torch.float32

    def up(a):
        return torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(device="cuda", dtype=dt)

    w = dict(w_router=up(inp.w_router), w_gate_up=up(inp.w_gate_up), w_down=up(inp.w_down),
             w_sh_gate_up=up(inp.w_sh_gate_up), w_sh_down=up(inp.w_sh_down))
    return up(inp.x), w


def run_forward(inp: synth.LayerInputs, bias=None, training=False, x=None, w=None):
    """moe_forward through the C ABI; returns (y float64 numpy, routing numpy dict, device handles)."""
    import torch
    from fine_grained_moe_amd import moe
    dims = moe.make_dims(inp.T, inp.d, inp.E, inp.F, inp.Fs, inp.k, inp.act)
    if x is None:
        x, w = to_gpu(inp)
    b = torch.from_numpy(np.asarray(inp.bias if bias is None else bias, np.float32)).cuda()
    y = torch.empty_like(x)
    r = moe.alloc_routing(dims)
    ws = moe.alloc_workspace(dims, training)
    moe.moe_forward(dims, x, w, b, y, r, ws, training=training)
    torch.cuda.synchronize()
    rn = {k: v.cpu().numpy() for k, v in r.items()}
    return y.float().cpu().numpy().astype(np.float64), rn, dict(dims=dims, x=x, w=w, b=b, y=y, r=r, ws=ws)


def check_routing_exact(rn, ref, E: int):
    """GPU routing vs oracle: idx, counts, offsets, perm, pos bit-exact."""
    idx = ref.idx
    np.testing.assert_array_equal(rn["idx"], idx)
    counts = om.expert_counts(idx, E)
    np.testing.assert_array_equal(rn["counts"], counts)
    np.testing.assert_array_equal(rn["offsets"], om.expert_offsets(counts))
    perm, pos = om.dispatch_order(idx, E)
    np.testing.assert_array_equal(rn["perm"], perm)
    np.testing.assert_array_equal(rn["pos"], pos)
