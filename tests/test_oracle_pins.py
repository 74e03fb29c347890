"""Pins of the CPU oracle against facts that do not come from the oracle itself.

Each test ties one part of the oracle to a closed form, a hand-derived worked
example, a brute-force computation on tiny inputs, an invariant the NanoColibri
article fixes, or an independent library (torch autograd).  The article is the
seventnews piece "A relay race of rented GPUs trained NanoColibri's 2.7B MoE for
$200"; sections are named in each test.
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle.moe_oracle as om
from fine_grained_moe_amd import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
L = math.log(3.0)


def _poly(c):
    """[c0, c1, c2] (fractions as strings) -> c0 + c1 L + c2 L^2."""
    if not isinstance(c, list):
        c = [c]
    return sum(float(Fraction(str(ci))) * L ** p for p, ci in enumerate(c))


def _arr(nested):
    """Nested lists whose leaves are coefficient lists -> float64 array."""
    def is_leaf(v):
        return isinstance(v, list) and all(not isinstance(u, list) for u in v)

    def walk(v):
        return _poly(v) if is_leaf(v) else [walk(u) for u in v]
    return np.array(walk(nested), dtype=np.float64)


@pytest.fixture(scope="module")
def worked():
    with open(os.path.join(GOLDEN, "worked_example.json")) as f:
        d = json.load(f)
    i = d["inputs"]
    inp = dict(x=_arr(i["x"]), w_router=_arr(i["w_router"]), bias=np.array(i["bias_f32"], np.float32),
               w_gate_up=_arr(i["w_gate_up"]), w_down=_arr(i["w_down"]),
               w_sh_gate_up=_arr(i["w_sh_gate_up"]), w_sh_down=_arr(i["w_sh_down"]))
    return inp, _arr(i["dy"]), i["k"], i["gamma"], d["expected"]


# ---------------------------------------------------------------- closed forms

def test_sigmoid_silu_closed_forms():
    assert om.sigmoid(0.0) == 0.5
    assert om.sigmoid(L) == pytest.approx(0.75, abs=1e-15)
    assert om.sigmoid(-L) == pytest.approx(0.25, abs=1e-15)
    assert om.silu(L) == pytest.approx(0.75 * L, abs=1e-15)
    assert om.silu(0.0) == 0.0
    # silu'(z) against a central difference of silu (different computation)
    z = np.linspace(-6, 6, 25)
    h = 1e-5
    fd = (om.silu(z + h) - om.silu(z - h)) / (2 * h)
    np.testing.assert_allclose(om.dsilu(z), fd, rtol=0, atol=1e-9)
    # silu'(ln 3) = 3/4 (1 + ln3 / 4)
    assert om.dsilu(L) == pytest.approx(0.75 * (1 + L / 4), abs=1e-15)


# ------------------------------------------------------------ worked example

def test_worked_example_forward(worked):
    inp, _, k, gamma, ex = worked
    y, r = om.forward(k=k, **inp)
    assert r.idx.tolist() == ex["idx"]
    np.testing.assert_allclose(r.gate, _arr(ex["gate"]), rtol=0, atol=1e-14)
    np.testing.assert_allclose(y, _arr(ex["y"]), rtol=0, atol=1e-14)
    counts = om.expert_counts(r.idx, 3)
    assert counts.tolist() == ex["counts"]


def test_worked_example_bias_update(worked):
    inp, _, k, gamma, ex = worked
    _, r = om.forward(k=k, **inp)
    counts = om.expert_counts(r.idx, 3)
    b = om.bias_update(inp["bias"], counts, total_assignments=1 * k, gamma=gamma)
    g32 = np.float32(gamma)
    assert g32.view(np.uint32) == 0x3A83126F          # fp32 of 1e-3
    sgn = ex["bias_sign"]
    want = np.array([np.float32(inp["bias"][e]) + np.float32(sgn[e]) * g32 for e in range(3)], np.float32)
    assert b.view(np.uint32).tolist() == want.view(np.uint32).tolist()
    assert b[0] == g32 and b[1] == -g32               # from 0: exactly +-gamma


def test_worked_example_backward(worked):
    inp, dy, k, _, ex = worked
    _, r = om.forward(k=k, **inp)
    g = om.backward(inp["x"], inp["w_router"], inp["w_gate_up"], inp["w_down"], inp["w_sh_gate_up"],
                    inp["w_sh_down"], r, dy)
    for name in ("dx", "dw_router", "dw_gate_up", "dw_down", "dw_sh_gate_up", "dw_sh_down"):
        np.testing.assert_allclose(getattr(g, name), _arr(ex[name]), rtol=0, atol=1e-13, err_msg=name)


def test_worked_example_top1(worked):
    """'Relay training' section, top-2 paragraph: at top_k=1 the routing
    weight is a constant and the router gets no gradient."""
    inp, dy, _, _, ex = worked
    y, r = om.forward(k=1, **inp)
    assert r.idx.tolist() == ex["top1_idx"]
    assert np.all(r.gate == 1.0)
    np.testing.assert_allclose(y, _arr(ex["top1_y"]), rtol=0, atol=1e-14)
    g = om.backward(inp["x"], inp["w_router"], inp["w_gate_up"], inp["w_down"], inp["w_sh_gate_up"],
                    inp["w_sh_down"], r, dy)
    assert np.all(g.dw_router == 0.0)


# --------------------------------------------------------------- selection

def _random_small(T=24, d=16, E=8, F=8, Fs=16, k=2, seed=3):
    rng = np.random.default_rng(seed)
    return dict(x=rng.standard_normal((T, d)), w_router=rng.standard_normal((E, d)) * 0.3,
                w_gate_up=rng.standard_normal((E, 2 * F, d)) * 0.2, w_down=rng.standard_normal((E, d, F)) * 0.2,
                w_sh_gate_up=rng.standard_normal((2 * Fs, d)) * 0.2, w_sh_down=rng.standard_normal((d, Fs)) * 0.2,
                bias=(rng.standard_normal(E) * 0.05).astype(np.float32))


def _brute_topk(v, k):
    """Rank-counting selection: rank(e) = #experts strictly ahead of e, where
    ahead means a larger key, or an equal key and a lower index."""
    T, E = v.shape
    out = np.zeros((T, k), dtype=np.int64)
    for t in range(T):
        for e in range(E):
            rank = sum(1 for f in range(E) if v[t, f] > v[t, e] or (v[t, f] == v[t, e] and f < e))
            if rank < k:
                out[t, rank] = e
    return out


@pytest.mark.parametrize("k", [1, 2, 3, 8])
def test_topk_matches_rank_counting(k):
    p = _random_small(E=8, seed=11 + k)
    r = om.route(p["x"], p["w_router"], p["bias"], k)
    assert np.array_equal(r.idx, _brute_topk(r.v, k))
    # selection is on score + bias (architecture paragraph): a large bias forces an expert in
    b = p["bias"].copy()
    b[5] = 10.0
    r2 = om.route(p["x"], p["w_router"], b, k)
    assert np.all(r2.idx[:, 0] == 5)


def test_exact_ties_go_to_lower_index():
    # x = 0: every logit 0, every score 1/2, every key equal -> experts 0..k-1
    E, d, k = 8, 16, 3
    r = om.route(np.zeros((4, d)), np.random.default_rng(0).standard_normal((E, d)), np.zeros(E, np.float32), k)
    assert r.idx.tolist() == [[0, 1, 2]] * 4
    np.testing.assert_array_equal(r.gate, np.full((4, k), 1.0 / k))
    # duplicated router rows 6 and 2 with equal bias: 2 always precedes 6
    rng = np.random.default_rng(1)
    W = rng.standard_normal((E, d))
    W[6] = W[2]
    x = rng.standard_normal((64, d))
    r = om.route(x, W, np.zeros(E, np.float32), 8)
    for row in r.idx:
        assert list(row).index(2) < list(row).index(6)
    assert np.array_equal(r.idx, _brute_topk(r.v, 8))


def test_counts_offsets_dispatch_invariants():
    p = _random_small(T=50, E=8, k=2)
    r = om.route(p["x"], p["w_router"], p["bias"], 2)
    c = om.expert_counts(r.idx, 8)
    assert c.sum() == 50 * 2                     # every token picks exactly k experts
    assert np.array_equal(c, np.array([(r.idx == e).sum() for e in range(8)]))
    off = om.expert_offsets(c)
    perm, pos = om.dispatch_order(r.idx, 8)
    assert sorted(perm.tolist()) == list(range(100))
    for t in range(50):
        for j in range(2):
            s = pos[t, j]
            assert perm[s] == t * 2 + j
            e = r.idx[t, j]
            assert off[e] <= s < off[e + 1]
    np.testing.assert_allclose(r.gate.sum(axis=1), 1.0, atol=1e-15)
    assert len(set(map(tuple, np.sort(r.idx, axis=1)))) > 1


def test_topk_margin_brute_force():
    v = np.array([[0.9, 0.1, 0.5, 0.45], [0.3, 0.3, 0.2, 0.0]])
    # k=2: three largest 0.9, 0.5, 0.45 -> gaps 0.4, 0.05; second row 0.3, 0.3, 0.2 -> 0, 0.1
    np.testing.assert_allclose(om.topk_margin(v, 2), [0.05, 0.0])


# ------------------------------------------------------- experts and combine

def _dense_masked_forward(p, k):
    """Every expert on every token, masked by rank-counting selection and
    weighted by normalised selected scores; a different evaluation order from
    the oracle's per-expert dispatch."""
    x = p["x"]
    s = 1.0 / (1.0 + np.exp(-(x @ p["w_router"].T)))
    v = s + p["bias"].astype(np.float64)
    idx = _brute_topk(v, k)
    E = p["w_router"].shape[0]
    mask = np.zeros_like(s)
    for t in range(x.shape[0]):
        mask[t, idx[t]] = 1.0
    G = mask * s / (mask * s).sum(axis=1, keepdims=True)
    F = p["w_gate_up"].shape[1] // 2
    A = np.einsum("td,efd->tef", x, p["w_gate_up"][:, :F])
    U = np.einsum("td,efd->tef", x, p["w_gate_up"][:, F:])
    H = A / (1 + np.exp(-A)) * U
    O = np.einsum("tef,edf->ted", H, p["w_down"])
    Fs = p["w_sh_gate_up"].shape[0] // 2
    a = x @ p["w_sh_gate_up"][:Fs].T
    u = x @ p["w_sh_gate_up"][Fs:].T
    S = (a / (1 + np.exp(-a)) * u) @ p["w_sh_down"].T
    return S + np.einsum("te,ted->td", G, O), E


@pytest.mark.parametrize("k", [1, 2, 4])
def test_forward_matches_dense_masked(k):
    p = _random_small(T=40, k=k, seed=7)
    y, _ = om.forward(k=k, **p)
    yd, _ = _dense_masked_forward(p, k)
    np.testing.assert_allclose(y, yd, rtol=1e-12, atol=1e-13)


def test_x_zero_gives_zero_output():
    p = _random_small()
    p["x"] = np.zeros_like(p["x"])
    p["bias"] = np.zeros_like(p["bias"])
    y, r = om.forward(k=2, **p)
    assert np.all(y == 0.0)
    assert r.idx.tolist() == [[0, 1]] * p["x"].shape[0]


def test_identical_experts_reduce_to_dense_ffn():
    """With identical experts the routed part is (sum of gates) * FFN(x) = FFN(x)."""
    p = _random_small(T=30)
    p["w_gate_up"][:] = p["w_gate_up"][0]
    p["w_down"][:] = p["w_down"][0]
    y, _ = om.forward(k=2, **p)
    F = p["w_gate_up"].shape[1] // 2
    x = p["x"]
    a = x @ p["w_gate_up"][0, :F].T
    u = x @ p["w_gate_up"][0, F:].T
    dense = (a * (1 / (1 + np.exp(-a))) * u) @ p["w_down"][0].T
    Fs = p["w_sh_gate_up"].shape[0] // 2
    a = x @ p["w_sh_gate_up"][:Fs].T
    u = x @ p["w_sh_gate_up"][Fs:].T
    shared = (a * (1 / (1 + np.exp(-a))) * u) @ p["w_sh_down"].T
    np.testing.assert_allclose(y, shared + dense, rtol=1e-12, atol=1e-13)


def test_unloaded_expert_contributes_nothing():
    p = _random_small(T=30, E=8)
    p["bias"][:] = 0
    p["bias"][7] = -5.0                       # expert 7 can never be selected
    y0, r = om.forward(k=2, **p)
    assert not np.any(r.idx == 7)
    p["w_gate_up"][7] *= 100.0
    p["w_down"][7] = 1e3
    y1, _ = om.forward(k=2, **p)
    assert np.array_equal(y0, y1)


def test_shared_expert_applies_to_every_token():
    """Proof-of-loop paragraph: every token touches the shared expert."""
    p = _random_small(T=20)
    y0, _ = om.forward(k=2, **p)
    p2 = dict(p)
    p2["w_sh_down"] = p["w_sh_down"] * 2.0
    y1, _ = om.forward(k=2, **p2)
    Fs = p["w_sh_gate_up"].shape[0] // 2
    a = p["x"] @ p["w_sh_gate_up"][:Fs].T
    u = p["x"] @ p["w_sh_gate_up"][Fs:].T
    S = (a / (1 + np.exp(-a)) * u) @ p["w_sh_down"].T
    np.testing.assert_allclose(y1 - y0, S, rtol=1e-10, atol=1e-12)
    assert np.all(np.abs(S).sum(axis=1) > 0)


# ---------------------------------------------------------------- bias rule

def test_bias_rule_direction_and_magnitude():
    """Architecture paragraph: the bias moves by gamma * sign(target - load)."""
    E, T, k = 8, 100, 2                      # target 25
    counts = np.array([0, 10, 24, 25, 26, 40, 50, 25])
    b = om.bias_update(np.zeros(E, np.float32), counts, T * k, 1e-3)
    g = np.float32(1e-3)
    assert b.tolist() == [g, g, g, 0, -g, -g, -g, 0]
    # a fractional target (T*k/E = 2/3) is compared exactly
    b = om.bias_update(np.zeros(3, np.float32), np.array([0, 1, 1]), 2, 1e-3)
    assert b.tolist() == [g, -g, -g]


def test_bias_rule_replay_is_bit_exact():
    rng = np.random.default_rng(5)
    E, Tk = 64, 8192
    b = np.zeros(E, np.float32)
    ref = np.zeros(E, np.float32)
    for step in range(50):
        counts = rng.multinomial(Tk, np.ones(E) / E)
        b = om.bias_update(b, counts, Tk, 1e-3)
        sgn = np.sign(Tk - E * counts)
        for e in range(E):    # one float32 add per expert, by hand
            ref[e] = np.float32(ref[e] + np.float32(sgn[e]) * np.float32(1e-3))
        assert b.view(np.uint32).tolist() == ref.view(np.uint32).tolist()
    n = np.rint(b.astype(np.float64) / 1e-3)
    assert np.all(np.abs(n) <= 50)
    np.testing.assert_allclose(b, n * 1e-3, atol=1e-6)


# ------------------------------------------------------------------- int4

def test_int4_format_golden():
    with open(os.path.join(GOLDEN, "int4_format.json")) as f:
        d = json.load(f)
    for g in d["groups"]:
        w = np.zeros((1, 128))
        w[0, :len(g["w_head"])] = g["w_head"]
        packed, scale = om.quantize_int4(w)
        assert scale[0, 0] == g["scale"], g["why"]
        q = om.unpack_int4(packed)[0]
        assert q[:len(g["q_head"])].tolist() == g["q_head"], g["why"]
        assert packed[0, :len(g["bytes_head"])].tolist() == g["bytes_head"], g["why"]
    assert om.unpack_int4(np.array([d["decode"]["byte"]], np.uint8)).tolist() == d["decode"]["q"]


def test_int4_round_trip_bound():
    rng = np.random.default_rng(2)
    w = rng.standard_normal((16, 512)) * 0.02
    packed, scale = om.quantize_int4(w)
    wq = om.dequantize_int4(packed, scale)
    sc = np.repeat(scale, 128, axis=-1)
    assert np.all(np.abs(w - wq) <= sc / 2 + 1e-18)
    assert np.all(np.abs(om.unpack_int4(packed)) <= 7)
    # scales are bf16 values: 8 significant bits
    m, _ = np.frexp(scale)
    assert np.all(m * 256 == np.rint(m * 256))


def test_int4_top1_is_the_dequantised_layer():
    p = _random_small(T=10, d=128, F=128)
    qg, sg = om.quantize_int4(p["w_gate_up"])
    qd, sd = om.quantize_int4(p["w_down"])
    y, r = om.forward_int4_top1(p["x"], p["w_router"], qg, sg, qd, sd, p["w_sh_gate_up"], p["w_sh_down"], p["bias"])
    assert np.all(r.gate == 1.0) and r.idx.shape == (10, 1)
    y2, _ = om.forward(p["x"], p["w_router"], om.dequantize_int4(qg, sg), om.dequantize_int4(qd, sd),
                       p["w_sh_gate_up"], p["w_sh_down"], p["bias"], k=1)
    assert np.array_equal(y, y2)


# ---------------------------------------------------------------- backward

def _loss(p, k, dy, routing_idx):
    y, r = om.forward(k=k, **p)
    assert np.array_equal(r.idx, routing_idx), "selection moved under the finite-difference step"
    return float(np.sum(y * dy))


@pytest.mark.parametrize("k", [1, 2])
def test_backward_finite_differences(k):
    p = _random_small(T=12, d=8, E=6, F=4, Fs=8, k=k, seed=21)
    dy = np.random.default_rng(4).standard_normal((12, 8))
    _, r = om.forward(k=k, **p)
    assert om.topk_margin(r.v, k).min() > 1e-4
    g = om.backward(p["x"], p["w_router"], p["w_gate_up"], p["w_down"], p["w_sh_gate_up"], p["w_sh_down"], r, dy)
    h = 1e-6
    rng = np.random.default_rng(9)
    for name, grad in (("x", g.dx), ("w_router", g.dw_router), ("w_gate_up", g.dw_gate_up),
                       ("w_down", g.dw_down), ("w_sh_gate_up", g.dw_sh_gate_up), ("w_sh_down", g.dw_sh_down)):
        arr = p[name]
        for _ in range(12):
            i = tuple(rng.integers(0, s) for s in arr.shape)
            old = arr[i]
            arr[i] = old + h
            lp = _loss(p, k, dy, r.idx)
            arr[i] = old - h
            lm = _loss(p, k, dy, r.idx)
            arr[i] = old
            fd = (lp - lm) / (2 * h)
            assert grad[i] == pytest.approx(fd, rel=1e-6, abs=1e-9), (name, i)
    if k == 1:
        assert np.all(g.dw_router == 0.0)


def test_backward_matches_torch_autograd():
    torch = pytest.importorskip("torch")
    p = _random_small(T=20, d=16, E=8, F=8, Fs=16, k=2, seed=33)
    dy = np.random.default_rng(6).standard_normal((20, 16))
    _, r = om.forward(k=2, **p)
    g = om.backward(p["x"], p["w_router"], p["w_gate_up"], p["w_down"], p["w_sh_gate_up"], p["w_sh_down"], r, dy)
    T = {n: torch.tensor(np.asarray(p[n], np.float64), requires_grad=True)
         for n in ("x", "w_router", "w_gate_up", "w_down", "w_sh_gate_up", "w_sh_down")}
    mask = torch.zeros(20, 8, dtype=torch.float64)
    mask[torch.arange(20)[:, None], torch.tensor(r.idx)] = 1.0
    s = torch.sigmoid(T["x"] @ T["w_router"].T)
    G = mask * s / (mask * s).sum(dim=1, keepdim=True)
    F = 8
    A = torch.einsum("td,efd->tef", T["x"], T["w_gate_up"][:, :F])
    U = torch.einsum("td,efd->tef", T["x"], T["w_gate_up"][:, F:])
    O = torch.einsum("tef,edf->ted", torch.nn.functional.silu(A) * U, T["w_down"])
    a = T["x"] @ T["w_sh_gate_up"][:16].T
    u = T["x"] @ T["w_sh_gate_up"][16:].T
    y = (torch.nn.functional.silu(a) * u) @ T["w_sh_down"].T + torch.einsum("te,ted->td", G, O)
    (y * torch.tensor(dy)).sum().backward()
    for mine, theirs in ((g.dx, "x"), (g.dw_router, "w_router"), (g.dw_gate_up, "w_gate_up"),
                         (g.dw_down, "w_down"), (g.dw_sh_gate_up, "w_sh_gate_up"), (g.dw_sh_down, "w_sh_down")):
        np.testing.assert_allclose(mine, T[theirs].grad.numpy(), rtol=1e-10, atol=1e-12, err_msg=theirs)


def test_identical_experts_have_no_router_gradient():
    p = _random_small(T=16, k=2, seed=8)
    p["w_gate_up"][:] = p["w_gate_up"][0]
    p["w_down"][:] = p["w_down"][0]
    dy = np.random.default_rng(3).standard_normal(p["x"].shape)
    _, r = om.forward(k=2, **p)
    g = om.backward(p["x"], p["w_router"], p["w_gate_up"], p["w_down"], p["w_sh_gate_up"], p["w_sh_down"], r, dy)
    assert np.abs(g.dw_router).max() < 1e-14


# -------------------------------------------------------- generator sanity

def test_generator_is_deterministic_and_exact():
    a = synth.make_workload("tiny_f32", seed=0)
    b = synth.make_workload("tiny_f32", seed=0)
    c = synth.make_workload("tiny_f32", seed=1)
    assert np.array_equal(a.x, b.x) and np.array_equal(a.w_down, b.w_down)
    assert not np.array_equal(a.x, c.x)
    w = synth.make_layer(T=8, d=64, E=4, F=64, Fs=64, k=2, act="bf16", seed=0)
    assert np.array_equal(synth.round_to_bf16(w.x), w.x)
    assert np.array_equal(synth.round_to_bf16(w.w_gate_up), w.w_gate_up)
    rms = np.sqrt(np.mean(w.x.astype(np.float64) ** 2, axis=1))
    np.testing.assert_allclose(rms, 1.0, atol=1e-2)
    assert abs(np.std(w.w_gate_up) - 0.02) < 2e-3
    # bf16 rounding: ties to even on hand-picked bit patterns
    v = np.array([0x3F808000, 0x3F818000, 0x3F80C000, 0x3F807FFF], np.uint32).view(np.float32)
    assert (synth.round_to_bf16(v).view(np.uint32) >> 16).tolist() == [0x3F80, 0x3F82, 0x3F81, 0x3F80]


# ---------------------------------------------------------------- expert balance (R19)

def test_load_stats_closed_forms():
    """Balance telemetry ("Relay training" section: a low dead-expert fraction,
    expert balance on the dashboard) against closed forms: uniform loads,
    everything on one expert, an even split over two of eight experts."""
    # uniform: nobody dead, max = mean, entropy ln E
    s = om.load_stats(np.full(64, 128), 64 * 128)
    np.testing.assert_allclose(s, [0.0, 1.0, math.log(64.0), 1.0], rtol=1e-15)
    # one-hot: E - 1 dead, max/mean = E, entropy 0
    c = np.zeros(64, np.int64)
    c[17] = 8192
    np.testing.assert_allclose(om.load_stats(c, 8192), [63 / 64, 64.0, 0.0, 0.0], rtol=1e-15, atol=0)
    # two of eight experts, 50/50: 6/8 dead, max/mean 4, entropy ln 2 (in nats: 1/3 of ln 8)
    c = np.array([0, 50, 0, 0, 50, 0, 0, 0])
    np.testing.assert_allclose(om.load_stats(c, 100), [0.75, 4.0, math.log(2.0), 1 / 3], rtol=1e-15)
    # one expert: normalised entropy reads 1; an empty batch reads (1, 0, 0, 0)
    np.testing.assert_allclose(om.load_stats(np.array([9]), 9), [0.0, 1.0, 0.0, 1.0], atol=0)
    np.testing.assert_array_equal(om.load_stats(np.zeros(8, np.int64), 0), [1.0, 0.0, 0.0, 0.0])


def test_load_stats_invariants():
    """Permuting experts changes nothing; 0 <= H <= ln E; max/mean >= 1; the
    entropy of a distribution equals ln E minus its KL divergence from uniform."""
    rng = np.random.default_rng(7)
    for E in (3, 8, 64):
        c = rng.multinomial(1000, rng.dirichlet(np.ones(E)))
        s = om.load_stats(c, 1000)
        np.testing.assert_allclose(om.load_stats(rng.permutation(c), 1000), s, rtol=1e-14)
        assert 0.0 <= s[2] <= math.log(E) + 1e-12 and s[1] >= 1.0
        p = c[c > 0] / 1000.0
        kl = float(np.sum(p * np.log(p * E)))
        assert abs(s[2] - (math.log(E) - kl)) < 1e-12
        assert s[0] == np.count_nonzero(c == 0) / E


# ---------------------------------------------------------------- MoE block (R20)

def test_rms_norm_closed_forms():
    """RMSNorm of the block: a hand-worked row, constant rows, gamma, and the
    invariance to a positive scale of the row."""
    # h = [3, 4]: mean square 12.5, so x = [3, 4] / sqrt(12.5 + 1e-6)
    x = om.rms_norm(np.array([[3.0, 4.0]]), np.ones(2))
    r = math.sqrt(12.5 + 1e-6)
    np.testing.assert_array_equal(x, om.to_bf16_nearest(np.array([[3 / r, 4 / r]])))
    assert abs(x[0, 0] - 0.84765625) < 1e-12 and abs(x[0, 1] - 1.1328125) < 1e-12   # bf16 of 0.8485, 1.1314
    # a constant row c maps to sign(c) |c| / sqrt(c^2 + eps) ~ sign(c), times gamma
    g = np.array([0.5, -2.0, 1.0, 3.0])
    x = om.rms_norm(np.full((1, 4), -7.0), g)
    np.testing.assert_array_equal(x, om.to_bf16_nearest(-g * 7 / math.sqrt(49 + 1e-6))[None])
    # scale invariance (eps negligible against the mean square)
    rng = np.random.default_rng(2)
    h = rng.standard_normal((5, 64))
    np.testing.assert_array_equal(om.rms_norm(h * 8.0, np.ones(64)), om.rms_norm(h, np.ones(64)))
    # the root mean square of a normalised row is 1 up to bf16 rounding
    xs = om.rms_norm(h, np.ones(64))
    np.testing.assert_allclose(np.sqrt(np.mean(xs * xs, axis=1)), 1.0, rtol=4e-3)


def test_block_with_silent_experts_is_the_identity():
    """With every expert's and the shared expert's output rows zero, the block
    returns its input exactly (the residual path), whatever the routing."""
    inp = synth.make_layer(T=40, d=128, E=8, F=64, Fs=128, k=2, act="f32", seed=8, rms_norm=False)
    w_down = np.zeros_like(inp.w_down)
    w_sh_down = np.zeros_like(inp.w_sh_down)
    h = inp.x * 3.0
    h_out, x, r = om.block_forward(h, np.ones(inp.d), inp.w_router, inp.w_gate_up, w_down, inp.w_sh_gate_up,
                                   w_sh_down, inp.bias, inp.k)
    np.testing.assert_array_equal(h_out, h.astype(np.float64))
    # and the layer inside reads the normalised rows
    np.testing.assert_array_equal(r.idx, om.route(x, inp.w_router, inp.bias, inp.k).idx)


def test_block_residual_hand_worked():
    """The block's residual adds the layer output (R20): a hand-worked token
    with one expert (so k = 1 and the gate is 1).  h = [1, 1] has mean square
    1, so x = bf16([1, 1] / sqrt(1 + 1e-6)) = [1, 1] exactly (the quotient
    0.9999995 is within half a bf16 step of 1).  Routed expert: a = x . [L/2,
    L/2] = L, u = x . [1, 0] = 1, h_e = silu(L) = 3L/4, out = [1, 2] * 3L/4.
    Shared expert: a = x . [-L/2, -L/2] = -L, u = x . [0, 1] = 1, h_s =
    silu(-L) = -L/4, out = [4, 0] * (-L/4).  So y = [3L/4 - L, 3L/2] and
    h_out = [1 - L/4, 1 + 3L/2] (h - y would give [1 + L/4, 1 - 3L/2])."""
    h = np.array([[1.0, 1.0]])
    w_router = np.array([[0.3, -0.2]])
    w_gate_up = np.array([[[L / 2, L / 2], [1.0, 0.0]]])       # [E=1, 2F=2, d=2]
    w_down = np.array([[[1.0], [2.0]]])                           # [E=1, d=2, F=1]
    w_sh_gate_up = np.array([[-L / 2, -L / 2], [0.0, 1.0]])       # [2Fs=2, d=2]
    w_sh_down = np.array([[4.0], [0.0]])                          # [d=2, Fs=1]
    h_out, x, r = om.block_forward(h, np.ones(2), w_router, w_gate_up, w_down, w_sh_gate_up, w_sh_down,
                                   np.zeros(1, np.float32), 1)
    np.testing.assert_array_equal(x, [[1.0, 1.0]])
    assert r.idx.tolist() == [[0]] and r.gate.tolist() == [[1.0]]
    np.testing.assert_allclose(h_out, [[1.0 - L / 4, 1.0 + 1.5 * L]], rtol=0, atol=1e-14)


def test_dispatch_order_hand_listed():
    """Dispatch order (R18): slots grouped by expert, ascending t*k + j inside
    each expert.  idx = [[2, 0], [0, 1], [2, 1]] flattens to experts
    [2, 0, 0, 1, 2, 1] at t*k + j = 0..5, so expert 0 holds assignments 1, 2;
    expert 1 holds 3, 5; expert 2 holds 0, 4."""
    idx = np.array([[2, 0], [0, 1], [2, 1]])
    perm, pos = om.dispatch_order(idx, 3)
    assert perm.tolist() == [1, 2, 3, 5, 0, 4]
    assert pos.tolist() == [[4, 0], [1, 2], [5, 3]]
    np.testing.assert_array_equal(om.expert_offsets(om.expert_counts(idx, 3)), [0, 2, 4, 6])


def test_bf16_rounding_ties_to_even():
    """bf16 keeps 8 significant bits.  1 + 2^-8 lies exactly halfway between
    1 and 1 + 2^-7 and goes to the even significand, 1; 1 + 3 * 2^-8 lies
    halfway between 1 + 2^-7 (odd) and 1 + 2^-6 (even) and goes up.  The same
    holds for negative values and in other binades; values off the midpoint
    go to the nearer neighbour."""
    cases = {1 + 2 ** -8: 1.0, 1 + 3 * 2 ** -8: 1 + 2 ** -6, -(1 + 2 ** -8): -1.0,
             -(1 + 3 * 2 ** -8): -(1 + 2 ** -6), 4 * (1 + 5 * 2 ** -8): 4 * (1 + 2 ** -6),
             2 ** -10 * (1 + 7 * 2 ** -8): 2 ** -10 * (1 + 2 ** -5), 1 + 2 ** -8 + 2 ** -30: 1 + 2 ** -7,
             1 + 2 ** -8 - 2 ** -30: 1.0, 0.75: 0.75}
    got = om.to_bf16_nearest(np.array(list(cases)))
    np.testing.assert_array_equal(got, np.array(list(cases.values())))
    # the int4 scale of a group whose absmax is 7 (1 + 2^-8): absmax / 7 is the
    # exact tie 1 + 2^-8, so the scale is 1 and the largest code 7
    w = np.zeros((1, 128))
    w[0, 5] = 7 * (1 + 2 ** -8)
    w[0, 9] = -3.5
    packed, scale = om.quantize_int4(w)
    assert scale.tolist() == [[1.0]]
    q = om.unpack_int4(packed)
    assert q[0, 5] == 7 and q[0, 9] == -4 and np.count_nonzero(q) == 2    # -3.5 is a tie: to even, -4
