#!/usr/bin/env python3
"""Throughput of the NanoColibri MoE layer's hot path on one MI355X.

A step is one pass of the whole path over one batch: the forward (router,
top-2, loads and dispatch, routed gate/up + SwiGLU, routed down + gate
scaling, shared expert, combine) and the bias step with the balance figures,
in one call (moe_forward_bias_step: the dispatch launch takes the bias step
once the loads are known; the same bits as moe_forward followed by
moe_bias_update_stats, one launch fewer), on the one-layer
workload T = 4096 tokens (batch 2 x seq 2048), d = 1024, 64 experts of width
512, top-2, shared expert 2048, bf16 with fp32 accumulation.  Inputs come from
the seeded generator and sit in HBM before timing starts; the routed expert
weights are packed into the stage-major layout (moe_pack_routed_bf16) once,
before timing, as a server does when it loads the model.

The bias step of every timed step also writes the batch's expert-balance
figures to a device buffer, read after timing.

Headline `value`: tokens/s with the expert weights rotated over several
distinct copies (each step reads its weights from HBM, not from the 256 MB
Infinity Cache); the same loop with one weight set is reported as `warm`.
Per-phase durations come from HIP events the library records on its stream
inside the timed region.

Prints one JSON line on stdout; progress goes to stderr.
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import sys
import time

METRIC = "MoE-layer tokens/sec (d=1024,E=64,top-2,bf16) + % MFMA peak / % HBM BW"
PEAK_BF16_FLOPS = 2.5e15      # MI355X dense bf16 MFMA
PEAK_HBM_BPS = 8.0e12         # MI355X HBM3E
GAMMA = 1e-3
PHASES = ("route", "gate_up", "down", "combine")
KERNEL_OF_PHASE = {
    "route": "route_topk + route_dispatch",
    "gate_up": "gemm256_kernel<true, false, 0> (routed + shared gate/up, one launch)",
    "down": "gemm256_kernel<false, false, 0> (routed down with gate scaling + shared down in two contraction halves, one launch)",
    "combine": "combine_kernel<bf16>",
}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def algorithmic_work(T, d, E, F, Fs, k, es=2):
    """Minimum FLOPs and HBM bytes of each phase: every weight and activation
    read once, every output written once; routed FLOPs over the T*k
    assignments only."""
    slots = T * k
    w = {}
    w["route"] = dict(flops=2.0 * T * d * E,
                      bytes=T * d * es + E * d * es + E * 4 + slots * 4 * 4 + (E * 2 + 1) * 4)
    w["gate_up"] = dict(flops=2.0 * slots * 2 * F * d + 2.0 * T * 2 * Fs * d,
                        bytes=E * 2 * F * d * es + 2 * Fs * d * es + T * d * es + slots * F * es
                        + T * Fs * es + slots * 4)
    w["down"] = dict(flops=2.0 * slots * d * F + 2.0 * T * d * Fs,
                     bytes=E * d * F * es + d * Fs * es + slots * F * es + T * Fs * es + slots * d * es
                     + T * d * es + slots * 8)
    w["combine"] = dict(flops=float(slots * d), bytes=T * d * es + slots * d * es + T * d * es + slots * 4)
    for v in w.values():
        t_mfma = v["flops"] / PEAK_BF16_FLOPS
        t_hbm = v["bytes"] / PEAK_HBM_BPS
        v["bound"] = "mfma" if t_mfma >= t_hbm else "hbm"
    return w


# Hardware byte counters of the dominant kernel (rocprofv3 --pmc FETCH_SIZE,
# then WRITE_SIZE, on this benchmark), kept under profiles/ with the hash of
# the sources they were taken on; reported only while those sources are
# unchanged.
TRAFFIC_FILE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "profiles",
                            "layer_t4096_gate_up_traffic.json")


def kernel_sources_hash(files):
    import hashlib
    root = os.path.dirname(os.path.abspath(__file__))
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(root, f), "rb") as fh:
            h.update(f.encode() + b"\0" + fh.read() + b"\0")
    return h.hexdigest()


def measured_traffic():
    """HBM bytes per launch of the gate/up GEMM from the committed counter
    summary: FETCH_SIZE and WRITE_SIZE (KiB per dispatch), each scaled by
    what the same counter reads for a plain 1 GiB device copy; None if the
    summary is missing or the kernel's sources changed since."""
    try:
        with open(TRAFFIC_FILE) as fh:
            t = json.load(fh)
        if kernel_sources_hash(t["sources"]) != t["sources_sha256"]:
            return None
        fetch = t["fetch_kib"] * 1024 * t["copy_bytes"] / (t["copy_fetch_kib"] * 1024)
        write = t["write_kib"] * 1024 * t["copy_bytes"] / (t["copy_write_kib"] * 1024)
        return fetch + write
    except (OSError, KeyError, ValueError, ZeroDivisionError):
        return None


HIP_EVENT_DISABLE_SYSTEM_FENCE = 0x20000000


class HipEvents:
    """hipEvent_t handles from the HIP runtime torch has loaded.

    Created with hipEventDisableSystemFence: a default event's record makes a
    system-scope release, which measured on MI355X adds about 3 us of idle GPU
    per record between two launches (14 us per step with five phase events);
    a device-scope event costs about 1 us."""

    def __init__(self):
        self.hip = ctypes.CDLL("libamdhip64.so.7")
        self.hip.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]

    def create(self):
        ev = ctypes.c_void_p()
        rc = self.hip.hipEventCreateWithFlags(ctypes.byref(ev), HIP_EVENT_DISABLE_SYSTEM_FENCE)
        if rc != 0:
            raise RuntimeError(f"hipEventCreate failed ({rc})")
        return ev.value

    def elapsed_ms(self, a, b):
        ms = ctypes.c_float()
        rc = self.hip.hipEventElapsedTime(ctypes.byref(ms), ctypes.c_void_p(a), ctypes.c_void_p(b))
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed ({rc})")
        return ms.value

    def destroy(self, e):
        self.hip.hipEventDestroy(ctypes.c_void_p(e))

    def record(self, e, stream):
        rc = self.hip.hipEventRecord(ctypes.c_void_p(e), ctypes.c_void_p(stream))
        if rc != 0:
            raise RuntimeError(f"hipEventRecord failed ({rc})")


def percentiles(us):
    """median / p10 / p90 of a list of per-step times (microseconds)."""
    import numpy as np
    a = np.asarray(us, dtype=np.float64)
    return dict(median=round(float(np.median(a)), 2), p10=round(float(np.percentile(a, 10)), 2),
                p90=round(float(np.percentile(a, 90)), 2), n=int(a.size))


def measured_peaks(torch):
    """Second denominators for the rooflines, measured on this GPU: the HBM
    rate of a plain 1 GiB device copy (read + write bytes over time) and the
    bf16 rate of the vendor GEMM library (torch.matmul -> hipBLASLt) on an
    8192^3 product, each the median of 10 event-timed runs."""
    import numpy as np
    out = {}
    src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    a = torch.randn(8192, 8192, device="cuda", dtype=torch.bfloat16)
    b = torch.randn(8192, 8192, device="cuda", dtype=torch.bfloat16)
    for name, fn, work in (("hbm_copy_gbps", lambda: dst.copy_(src), 2.0 * (1 << 30) / 1e9),
                           ("bf16_gemm_tflops", lambda: torch.matmul(a, b), 2.0 * 8192 ** 3 / 1e12)):
        for _ in range(3):
            fn()
        ts = []
        for _ in range(10):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1) * 1e-3)
        out[name] = round(work / float(np.median(ts)), 1)
    del src, dst, a, b
    out["how"] = ("hbm_copy_gbps: 1 GiB device-to-device copy, bytes read + written over time; "
                  "bf16_gemm_tflops: torch.matmul (hipBLASLt) 8192^3 bf16; medians of 10 runs")
    return out


def decode_bytes(T, d, E, F, Fs, unique_experts):
    """Algorithmic HBM bytes of one top-1 int4 serving forward: the router and
    the shared expert (bf16), each routed expert a token uses once (packed
    int4 + bf16 scales), activations in and out."""
    per_expert = 2 * F * d // 2 + 2 * F * (d // 128) * 2 + d * F // 2 + d * (F // 128) * 2
    return E * d * 2 + 3 * Fs * d * 2 + unique_experts * per_expert + 2 * T * d * 2


def bench_decode(moe, synth, torch, np, n_layers=23, iters=46, graph_reps=20):
    """Top-1 int4 serving forward at T = 1, 8, 64, cycling 23 distinct weight
    copies (one per MoE layer of the model) so every forward reads its
    weights from HBM.  Timed two ways: eager calls from Python (bound by the
    host's launch cost at small T), and the 23 forwards captured once in a
    HIP graph and replayed, as a serving loop would run them (`us`)."""
    E, d, F, Fs = 64, 1024, 512, 2048
    base = synth.make_layer(T=64, d=d, E=E, F=F, Fs=Fs, k=1, act="bf16", seed=11)
    qg, sg = synth.random_int4(E, 2 * F, d, seed=11)
    qd, sd = synth.random_int4(E, d, F, seed=12)
    bf = lambda a: torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(device="cuda", dtype=torch.bfloat16)
    w0 = dict(w_router=bf(base.w_router), w_gate_up=torch.from_numpy(qg).cuda(), s_gate_up=bf(sg),
              w_down=torch.from_numpy(qd).cuda(), s_down=bf(sd), w_sh_gate_up=bf(base.w_sh_gate_up),
              w_sh_down=bf(base.w_sh_down))
    layers = [w0] + [{n: t.clone() for n, t in w0.items()} for _ in range(n_layers - 1)]
    bias = torch.zeros(E, device="cuda")
    out = {}
    for T in (1, 8, 64):
        dims = moe.make_dims(T, d, E, F, Fs, 1, "bf16", w_routed="int4")
        x = bf(base.x[:T])
        y = torch.empty_like(x)
        r = moe.alloc_routing(dims)
        ws = moe.alloc_workspace(dims)
        for i in range(n_layers):
            moe.moe_forward(dims, x, layers[i], bias, y, r, ws)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for i in range(iters):
            moe.moe_forward(dims, x, layers[i % n_layers], bias, y, r, ws)
        e1.record()
        torch.cuda.synchronize()
        eager_us = e0.elapsed_time(e1) * 1e3 / iters
        # the same 23 forwards, captured once and replayed; then with each
        # layer naming the next (moe_weights.next, the last naming the first,
        # as a serving loop runs them token after token)
        def replay_us(ls):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                for i in range(n_layers):
                    moe.moe_forward(dims, x, ls[i], bias, y, r, ws)
            g.replay()
            torch.cuda.synchronize()
            e0.record()
            for _ in range(graph_reps):
                g.replay()
            e1.record()
            torch.cuda.synchronize()
            del g
            return e0.elapsed_time(e1) * 1e3 / (graph_reps * n_layers)

        us = replay_us(layers)
        us_hint = replay_us([dict(layers[i], next=layers[(i + 1) % n_layers]) for i in range(n_layers)])
        uniq = int((r["counts"] > 0).sum().item())
        nbytes = decode_bytes(T, d, E, F, Fs, uniq)
        gbps = nbytes / (us * 1e-6) / 1e9
        gbps_hint = nbytes / (us_hint * 1e-6) / 1e9
        out[f"T{T}"] = dict(us=round(us, 2), eager_us=round(eager_us, 2), unique_experts=uniq, bytes=nbytes,
                            gbps=round(gbps, 1), frac_hbm=round(gbps / (PEAK_HBM_BPS / 1e9), 4),
                            us_next_layer_hint=round(us_hint, 2),
                            frac_hbm_next_layer_hint=round(gbps_hint / (PEAK_HBM_BPS / 1e9), 4))
        log(f"decode T={T}: {us:.1f} us per forward (graph replay; eager {eager_us:.1f} us), {uniq} experts, "
            f"{gbps:.0f} GB/s ({gbps / 8000:.1%} of HBM); with the next-layer hint {us_hint:.1f} us "
            f"({gbps_hint / 8000:.1%})")
    # The floor the three dependent launches of a forward put under it: three
    # minimal dependent kernels (one-element adds) per forward, 23 forwards,
    # captured and replayed the same way.
    z = torch.zeros(1, device="cuda")
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(n_layers * 3):
            z.add_(1.0)
    g.replay()
    torch.cuda.synchronize()
    e0.record()
    for _ in range(graph_reps):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    out["launch_floor_us"] = round(e0.elapsed_time(e1) * 1e3 / (graph_reps * n_layers), 2)
    del g
    log(f"decode launch floor: {out['launch_floor_us']:.2f} us per forward (3 minimal dependent kernels, graph replay)")
    return out


def _pack_routed(moe, torch, dims, w):
    """w with its routed weights replaced by stage-major copies (moe_pack_routed_bf16)."""
    out = dict(w)
    out["w_gate_up"], out["w_down"] = torch.empty_like(w["w_gate_up"]), torch.empty_like(w["w_down"])
    moe.moe_pack_routed_bf16(dims, w["w_gate_up"], w["w_down"], out["w_gate_up"], out["w_down"])
    return out


def bench_stack(moe, synth, torch, np, n_layers=23, reps=10, graph_reps=20):
    """The model's 23 MoE layers chained through the residual stream with
    moe_forward_block (RMSNorm in, residual add out), distinct weights per
    layer so every layer reads its weights from HBM: bf16 at T = 4096 (eager
    launches), and the int4 top-1 serving path at T = 1, 8, 64 (the 23 blocks
    captured once in a HIP graph and replayed; the bf16 routed weights
    stage-major, packed before timing).  Weights are seeded N(0, 0.02)
    draws on the device (the same recipe as the one-layer workload; parity is
    the tests' business)."""
    E, d, F, Fs = 64, 1024, 512, 2048
    gen = torch.Generator(device="cuda")
    gen.manual_seed(1234)

    def randn(*shape, std=0.02, dtype=torch.bfloat16):
        return (torch.randn(*shape, generator=gen, device="cuda", dtype=torch.float32) * std).to(dtype)

    gamma = 1.0 + randn(d, std=0.1, dtype=torch.float32)
    out = {}
    # bf16 batch path, T = 4096
    T, k = 4096, 2
    dims = moe.make_dims(T, d, E, F, Fs, k, "bf16", w_routed="bf16_staged")   # routed weights stage-major
    layers = [_pack_routed(moe, torch, dims, dict(w_router=randn(E, d), w_gate_up=randn(E, 2 * F, d),
                                                  w_down=randn(E, d, F), w_sh_gate_up=randn(2 * Fs, d),
                                                  w_sh_down=randn(d, Fs))) for _ in range(n_layers)]
    biases = [torch.zeros(E, device="cuda") for _ in range(n_layers)]
    h = [randn(T, d, std=1.0), torch.empty(T, d, device="cuda", dtype=torch.bfloat16)]
    r = moe.alloc_routing(dims)
    ws = moe.alloc_workspace(dims)

    def stack():
        for i in range(n_layers):
            moe.moe_forward_block(dims, h[i % 2], gamma, 1e-6, layers[i], biases[i], h[(i + 1) % 2], r, ws)

    for _ in range(2):
        stack()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(reps):
        stack()
    torch.cuda.synchronize()
    el = (time.perf_counter() - t0) / reps
    out["bf16_t4096"] = dict(us_per_stack=round(el * 1e6, 1), us_per_layer=round(el * 1e6 / n_layers, 2),
                             tokens_per_s=T / el)
    log(f"stack bf16 T={T}: {el * 1e3:.3f} ms per {n_layers}-layer stack ({el * 1e6 / n_layers:.1f} us per layer), "
        f"{T / el / 1e6:.3f} M tokens/s")
    del layers, h, r, ws
    torch.cuda.empty_cache()
    # int4 top-1 serving path, T = 1, 8, 64
    base = synth.make_layer(T=64, d=d, E=E, F=F, Fs=Fs, k=1, act="bf16", seed=11)
    qg, sg = synth.random_int4(E, 2 * F, d, seed=11)
    qd, sd = synth.random_int4(E, d, F, seed=12)
    bf = lambda a: torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(device="cuda", dtype=torch.bfloat16)
    w0 = dict(w_router=bf(base.w_router), w_gate_up=torch.from_numpy(qg).cuda(), s_gate_up=bf(sg),
              w_down=torch.from_numpy(qd).cuda(), s_down=bf(sd), w_sh_gate_up=bf(base.w_sh_gate_up),
              w_sh_down=bf(base.w_sh_down))
    qlayers = [w0] + [{n: t.clone() for n, t in w0.items()} for _ in range(n_layers - 1)]
    # each layer names the one after it (moe_weights.next): its router and
    # shared gate/up rows are read into the caches during this layer's last
    # launch; the last layer names none
    hinted = [dict(qlayers[i], next=qlayers[i + 1]) for i in range(n_layers - 1)] + [qlayers[-1]]
    bias = torch.zeros(E, device="cuda")
    out["int4_top1"] = {}
    for T in (1, 8, 64):
        dims = moe.make_dims(T, d, E, F, Fs, 1, "bf16", w_routed="int4")
        h = [randn(T, d, std=1.0), torch.empty(T, d, device="cuda", dtype=torch.bfloat16)]
        r = moe.alloc_routing(dims)
        ws = moe.alloc_workspace(dims)

        def replay_us(layers):
            def qstack():
                for i in range(n_layers):
                    moe.moe_forward_block(dims, h[i % 2], gamma, 1e-6, layers[i], bias, h[(i + 1) % 2], r, ws)

            qstack()
            torch.cuda.synchronize()
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                qstack()
            g.replay()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(graph_reps):
                g.replay()
            e1.record()
            torch.cuda.synchronize()
            del g
            return e0.elapsed_time(e1) * 1e3 / graph_reps

        us_plain = replay_us(qlayers)
        us = replay_us(hinted)
        out["int4_top1"][f"T{T}"] = dict(us_per_stack=round(us, 1), us_per_layer=round(us / n_layers, 2),
                                         tokens_per_s=T / (us * 1e-6), us_per_stack_no_hint=round(us_plain, 1))
        log(f"stack int4 top-1 T={T}: {us:.1f} us per {n_layers}-layer stack (graph replay, next-layer hint; "
            f"{us / n_layers:.1f} us per layer), {T / (us * 1e-6):.0f} tokens/s; without the hint {us_plain:.1f} us")
    return out


def bench_zipf(moe, synth, torch, np, steps=50, warmup=5, calib=400):
    """Skewed routing: the layer at T = 16384 with the router bias preset so
    the expected expert loads follow Zipf(1) over the 64 experts (expert 0
    hottest, ~21% of assignments; several near-dead experts).  The preset is
    found with the library's own router: b_e += eta * sign(T*k*p_e - load_e),
    eta = 0.02 * 2^-(it // 100), 400 iterations on this batch.  Then forward +
    bias step with telemetry, timed like the headline (8 weight sets)."""
    inp = synth.make_workload("zipf_t16384", seed=0)
    T, d, E, F, Fs, k = inp.T, inp.d, inp.E, inp.F, inp.Fs, inp.k
    dims = moe.make_dims(T, d, E, F, Fs, k, "bf16", w_routed="bf16_staged")   # routed weights stage-major
    bf = lambda a: torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(device="cuda", dtype=torch.bfloat16)
    base = _pack_routed(moe, torch, dims, dict(w_router=bf(inp.w_router), w_gate_up=bf(inp.w_gate_up),
                                               w_down=bf(inp.w_down), w_sh_gate_up=bf(inp.w_sh_gate_up),
                                               w_sh_down=bf(inp.w_sh_down)))
    sets = [base] + [{n: t.clone() for n, t in base.items()} for _ in range(7)]
    x = bf(inp.x)
    y = torch.empty_like(x)
    r = moe.alloc_routing(dims)
    ws = moe.alloc_workspace(dims)
    pz = 1.0 / np.arange(1, E + 1)
    target = T * k * pz / pz.sum()
    b = np.zeros(E, np.float32)
    bt = torch.zeros(E, device="cuda")
    for it in range(calib):
        bt.copy_(torch.from_numpy(b))
        moe.moe_route(dims, x, base["w_router"], bt, r, ws)
        load = r["counts"].cpu().numpy()
        b = (b + np.float32(0.02 * 2.0 ** -(it // 100)) * np.sign(target - load).astype(np.float32)).astype(np.float32)
    bt.copy_(torch.from_numpy(b))
    stats = torch.zeros(steps, 4, device="cuda")
    bias = bt.clone()
    for i in range(warmup):
        moe.moe_forward(dims, x, sets[i % 8], bias, y, r, ws)
    ev = HipEvents()
    e_g = [[ev.create() for _ in range(len(PHASES) + 1)] for _ in range(steps)]
    bias.copy_(bt)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        moe.moe_forward_events(dims, x, sets[i % 8], bias, y, r, ws, e_g[i], bias_step=True, gamma=GAMMA,
                               stats=stats[i])
    torch.cuda.synchronize()
    el = (time.perf_counter() - t0) / steps
    # phase j spans events j -> j + 1 (PHASES: route, gate_up, down, combine)
    ph_us = {p: sum(ev.elapsed_ms(e_g[i][j], e_g[i][j + 1]) for i in range(steps)) / steps * 1e3
             for j, p in enumerate(PHASES)}
    gate_up_us = ph_us["gate_up"]
    for row in e_g:
        for e_ in row:
            ev.destroy(e_)
    st0 = stats[0].cpu().tolist()
    work = algorithmic_work(T, d, E, F, Fs, k)
    out = dict(T=T, us_per_step=round(el * 1e6, 1), tokens_per_s=T / el,
               phases_us={p: round(v, 1) for p, v in ph_us.items()}, gate_up_us=round(gate_up_us, 1),
               gate_up_tflops=round(work["gate_up"]["flops"] / (gate_up_us * 1e-6) / 1e12, 1),
               down_tflops=round(work["down"]["flops"] / (ph_us["down"] * 1e-6) / 1e12, 1),
               max_over_mean_load=round(st0[1], 3), dead_fraction=round(st0[0], 4))
    log(f"zipf T={T}: {el * 1e6:.1f} us/step, {T / el / 1e6:.2f} M tokens/s; phases (us): "
        + ", ".join(f"{p}={v:.1f}" for p, v in ph_us.items())
        + f"; gate/up {out['gate_up_tflops']:.0f} TFLOP/s, down {out['down_tflops']:.0f} TFLOP/s; "
        f"hottest expert {st0[1]:.2f} x the mean load")
    return out


def bench_int4(moe, synth, torch, np, reps=20, steps=50, warmup=5, n_sets=8):
    """int4 export and prefill.  Export: moe_quantize_int4 over one layer's
    routed weights (bf16 [64, 1024, 1024] gate/up and [64, 1024, 512] down,
    N(0, 0.02)); algorithmic bytes = 2 read + 0.5 written per element + 2 per
    128 (scales).  Prefill: the int4 top-1 layer at T = 4096 (x RMS-normalised
    N(0, 1)) on those exported weights, 8 weight sets rotated (cold), phases
    from the library's events (the grouped GEMMs read the packed experts
    directly, so the phases are those of the bf16 layer)."""
    E, d, F, Fs = 64, 1024, 512, 2048
    inp = synth.make_layer(T=4096, d=d, E=E, F=F, Fs=Fs, k=1, act="bf16", seed=5)
    bf = lambda a: torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(device="cuda", dtype=torch.bfloat16)
    wgu, wd = bf(inp.w_gate_up), bf(inp.w_down)
    pg = torch.empty(E, 2 * F, d // 2, dtype=torch.uint8, device="cuda")
    sg = torch.empty(E, 2 * F, d // 128, dtype=torch.bfloat16, device="cuda")
    pd = torch.empty(E, d, F // 2, dtype=torch.uint8, device="cuda")
    sd = torch.empty(E, d, F // 128, dtype=torch.bfloat16, device="cuda")

    def export():
        moe.moe_quantize_int4(wgu, pg, sg)
        moe.moe_quantize_int4(wd, pd, sd)

    for _ in range(3):
        export()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        export()
    e1.record()
    torch.cuda.synchronize()
    us_x = e0.elapsed_time(e1) * 1e3 / reps
    n_el = E * 2 * F * d + E * d * F
    xbytes = n_el * (2 + 0.5) + n_el // 128 * 2
    out = dict(export=dict(us=round(us_x, 1), gbps=round(xbytes / (us_x * 1e-6) / 1e9, 1),
                           frac_hbm=round(xbytes / (us_x * 1e-6) / PEAK_HBM_BPS, 3), bytes=int(xbytes)))
    log(f"int4 export: {us_x:.1f} us for one layer's routed weights ({xbytes / 1e6:.1f} MB), "
        f"{xbytes / (us_x * 1e-6) / 1e9:.0f} GB/s")
    del wgu, wd
    # prefill on the exported weights
    T = inp.T
    dims = moe.make_dims(T, d, E, F, Fs, 1, "bf16", w_routed="int4")
    base = dict(w_router=bf(inp.w_router), w_gate_up=pg, s_gate_up=sg, w_down=pd, s_down=sd,
                w_sh_gate_up=bf(inp.w_sh_gate_up), w_sh_down=bf(inp.w_sh_down))
    sets = [base] + [{n: t.clone() for n, t in base.items()} for _ in range(n_sets - 1)]
    x = bf(inp.x)
    y = torch.empty_like(x)
    r = moe.alloc_routing(dims)
    ws = moe.alloc_workspace(dims)
    bias = torch.zeros(E, device="cuda")
    for i in range(warmup):
        moe.moe_forward(dims, x, sets[i % n_sets], bias, y, r, ws)
    ev = HipEvents()
    e_g = [[ev.create() for _ in range(len(PHASES) + 1)] for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        moe.moe_forward_events(dims, x, sets[i % n_sets], bias, y, r, ws, e_g[i])
    torch.cuda.synchronize()
    el = (time.perf_counter() - t0) / steps
    ph_us = {p: sum(ev.elapsed_ms(e_g[i][j], e_g[i][j + 1]) for i in range(steps)) / steps * 1e3
             for j, p in enumerate(PHASES)}
    for row in e_g:
        for e_ in row:
            ev.destroy(e_)
    active = int(np.count_nonzero(r["counts"].cpu().numpy()))
    work = algorithmic_work(T, d, E, F, Fs, 1)
    out["prefill"] = dict(T=T, us_per_forward=round(el * 1e6, 1), tokens_per_s=T / el, active_experts=active,
                          phases_us={p: round(v, 1) for p, v in ph_us.items()},
                          gate_up_tflops=round(work["gate_up"]["flops"] / (ph_us["gate_up"] * 1e-6) / 1e12, 1))
    log(f"int4 prefill T={T}: {el * 1e6:.1f} us/forward, {T / el / 1e6:.2f} M tokens/s; phases (us): "
        + ", ".join(f"{p}={v:.1f}" for p, v in ph_us.items()) + ", "
        f"{active} experts loaded")
    return out


def bench_stream(moe, synth, torch, np, steps=200, warmup=30):
    """Expert streaming for int4 top-1 serving: the LRU expert cache over a few
    HBM slots, filled from pinned host memory, against all experts resident.
    A step serves one batch of fresh tokens: moe_route, the loads copied to the
    host, moe_cache_prepare (the misses' int4 arrays copied host -> slot), then
    moe_forward_cached; eager launches, timed on the host clock.  Routing:
    uniform (no bias) and skewed (bias_e = -0.1 ln(1 + e), favouring the low
    experts).  Weights: N(0, 0.02) draws, int4-encoded by the library."""
    E, d, F, Fs = 64, 1024, 512, 2048
    inp = synth.make_layer(T=1, d=d, E=E, F=F, Fs=Fs, k=1, act="bf16", seed=9)
    bf = lambda a: torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(device="cuda", dtype=torch.bfloat16)
    wgu, wd = bf(inp.w_gate_up), bf(inp.w_down)
    full = dict(w_router=bf(inp.w_router), w_sh_gate_up=bf(inp.w_sh_gate_up), w_sh_down=bf(inp.w_sh_down),
                w_gate_up=torch.empty(E, 2 * F, d // 2, dtype=torch.uint8, device="cuda"),
                s_gate_up=torch.empty(E, 2 * F, d // 128, dtype=torch.bfloat16, device="cuda"),
                w_down=torch.empty(E, d, F // 2, dtype=torch.uint8, device="cuda"),
                s_down=torch.empty(E, d, F // 128, dtype=torch.bfloat16, device="cuda"))
    moe.moe_quantize_int4(wgu, full["w_gate_up"], full["s_gate_up"])
    moe.moe_quantize_int4(wd, full["w_down"], full["s_down"])
    del wgu, wd
    int4 = ("w_gate_up", "s_gate_up", "w_down", "s_down")
    pinned = {n: full[n].cpu().pin_memory() for n in int4}
    per_expert = sum(pinned[n][0].numel() * pinned[n].element_size() for n in int4)
    out = dict(bytes_per_expert=per_expert, cases=[])
    gen = torch.Generator(device="cuda")
    gen.manual_seed(77)
    for T in (1, 8):
        dims = moe.make_dims(T, d, E, F, Fs, 1, "bf16", w_routed="int4")
        xs = (torch.randn(warmup + steps, T, d, generator=gen, device="cuda")).to(torch.bfloat16)
        r = moe.alloc_routing(dims)
        ws = moe.alloc_workspace(dims)
        y = torch.empty(T, d, dtype=torch.bfloat16, device="cuda")
        for skew in (0.0, 0.1):
            bias = (-skew * torch.log1p(torch.arange(E, dtype=torch.float32, device="cuda"))).contiguous()
            # all experts resident
            for i in range(warmup):
                moe.moe_forward(dims, xs[i], full, bias, y, r, ws)
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            for i in range(steps):
                moe.moe_forward(dims, xs[warmup + i], full, bias, y, r, ws)
            torch.cuda.synchronize()
            us_res = (time.perf_counter() - t0) / steps * 1e6
            for n_slots in (8, 16, 32, 64):
                dev = {n: torch.zeros((n_slots,) + tuple(pinned[n].shape[1:]), dtype=pinned[n].dtype,
                                      device="cuda") for n in int4}
                slot = torch.full((E,), -1, dtype=torch.int32, device="cuda")
                cache = moe.ExpertCache(dims, n_slots, host=pinned, dev=dev, slot=slot)
                cache.state()
                out["fill"] = "one launch reading the pinned host copy" if cache.zero_copy else "hipMemcpyAsync per array"
                w = dict(full)
                w.update(dev)
                nmiss, active = 0, 0
                t0 = 0.0
                for i in range(warmup + steps):
                    if i == warmup:
                        torch.cuda.synchronize()
                        t0 = time.perf_counter()
                        nmiss, active = 0, 0
                    moe.moe_route(dims, xs[i], full["w_router"], bias, r, ws)
                    counts = r["counts"].cpu().numpy()
                    nmiss += cache.prepare(counts)
                    active += int(np.count_nonzero(counts))
                    moe.moe_forward_cached(dims, xs[i], w, slot, n_slots, bias, y, r, ws)
                torch.cuda.synchronize()
                us = (time.perf_counter() - t0) / steps * 1e6
                cache.close()
                case = dict(T=T, skew=skew, n_slots=n_slots, us_per_step=round(us, 1), us_all_resident=round(us_res, 1),
                            misses_per_step=round(nmiss / steps, 3), miss_rate=round(nmiss / max(active, 1), 4),
                            h2d_mb_per_step=round(nmiss * per_expert / steps / 1e6, 3), tokens_per_s=T / (us * 1e-6))
                out["cases"].append(case)
                log(f"stream T={T} skew={skew} slots={n_slots}: {us:.1f} us/step (all resident {us_res:.1f}), "
                    f"{nmiss / steps:.2f} misses/step ({100 * nmiss / max(active, 1):.1f}% of active experts), "
                    f"{nmiss * per_expert / steps / 1e6:.2f} MB/step host->device")
                del dev, slot, w
    return out


def bench_train(moe, synth, torch, np, steps=10, warmup=3):
    """One training step of the layer at T = 32768 (16 x 2048): forward with
    saved activations, backward (dx and every weight gradient), bias step."""
    inp = synth.make_workload("train_t32768", with_dy=True)
    T, d, E, F, Fs, k = inp.T, inp.d, inp.E, inp.F, inp.Fs, inp.k
    dims = moe.make_dims(T, d, E, F, Fs, k, "bf16")
    bf = lambda a: torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(device="cuda", dtype=torch.bfloat16)
    w = dict(w_router=bf(inp.w_router), w_gate_up=bf(inp.w_gate_up), w_down=bf(inp.w_down),
             w_sh_gate_up=bf(inp.w_sh_gate_up), w_sh_down=bf(inp.w_sh_down))
    x, dy = bf(inp.x), bf(inp.dy)
    y, dx = torch.empty_like(x), torch.empty_like(x)
    bias = torch.zeros(E, device="cuda")
    r = moe.alloc_routing(dims)
    ws = moe.alloc_workspace(dims, training=True)
    g = moe.alloc_grads(dims)

    def step():
        moe.moe_forward(dims, x, w, bias, y, r, ws, training=True)
        moe.moe_backward(dims, x, w, r, dy, dx, g, ws)
        moe.moe_bias_update(E, T * k, r["counts"], GAMMA, bias)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    el = (time.perf_counter() - t0) / steps
    flops = 3 * (2.0 * T * k * 3 * d * F + 2.0 * T * 3 * d * Fs + 2.0 * T * d * E)
    out = dict(T=T, ms_per_step=round(el * 1e3, 3), tokens_per_s=T / el, algorithmic_tflop=round(flops / 1e12, 3),
               tflops=round(flops / el / 1e12, 1), frac_mfma=round(flops / el / PEAK_BF16_FLOPS, 4))
    log(f"train T={T}: {el * 1e3:.2f} ms/step, {T / el / 1e6:.2f} M tokens/s, {flops / el / 1e12:.0f} TFLOP/s")
    return out


def cpu_baseline(inp, seconds: float):
    """The CPU oracle as it stands, on this host's cores, over a bounded sample:
    whole copies of the benchmark batch until `seconds` have passed."""
    import numpy as np
    from oracle import moe_oracle as om
    cores = len(os.sched_getaffinity(0))          # the host cores this process may run on
    try:
        from threadpoolctl import threadpool_info
        threads = max((i.get("num_threads", 1) for i in threadpool_info()), default=1)
    except Exception:
        threads = None
    model = None
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    t0 = time.perf_counter()
    n = 0
    while True:
        om.forward(inp.x, inp.w_router, inp.w_gate_up, inp.w_down, inp.w_sh_gate_up, inp.w_sh_down, inp.bias, inp.k)
        n += 1
        el = time.perf_counter() - t0
        if el >= seconds:
            break
    return dict(value=n * inp.T / el, unit="tokens/s", cores=int(cores), kind="oracle",
                impl="NumPy float64, BLAS matmuls as steps", blas_threads=threads, cpu_model=model,
                sample=f"{n} x the {inp.T}-token benchmark batch (float64 oracle forward incl. routing), "
                       f"{el:.1f} s wall")


GATE_UP_KERNEL = "gemm256_kernel<true, false, 0>"   # the bf16 gate/up instantiation
TRAFFIC_SOURCES = ["fine_grained_moe_amd/csrc/gemm_fwd.hip", "fine_grained_moe_amd/csrc/gemm_tile.h",
                   "fine_grained_moe_amd/csrc/common.h", "fine_grained_moe_amd/csrc/kernels.h",
                   "fine_grained_moe_amd/csrc/api.hip"]


def traffic_summary(fetch_csv, write_csv):
    """Reduce two rocprofv3 --pmc counter files of a `--copy-calibration` run
    (FETCH_SIZE, then WRITE_SIZE) to the figures bench.py reports: the mean
    per-dispatch KiB of the gate/up GEMM, and the counter readings of the
    1 GiB device copy that scale them to bytes."""
    import csv

    def read(path, counter):
        gemm, copy = [], []
        with open(path) as fh:
            for r in csv.DictReader(fh):
                if r["Counter_Name"] != counter:
                    continue
                v = float(r["Counter_Value"])
                if GATE_UP_KERNEL in r["Kernel_Name"]:
                    gemm.append(v)
                elif "copyBuffer" in r["Kernel_Name"] and v >= 256 * 1024:   # the 1 GiB copies
                    copy.append(v)
        if not gemm or not copy:
            raise SystemExit(f"{path}: no {counter} readings of the gate/up GEMM or of the 1 GiB copy")
        return sum(gemm) / len(gemm), len(gemm), max(copy)

    f_kib, nf, f_copy = read(fetch_csv, "FETCH_SIZE")
    w_kib, nw, w_copy = read(write_csv, "WRITE_SIZE")
    out = dict(kernel=GATE_UP_KERNEL, workload="layer_t4096", fetch_kib=round(f_kib, 1), write_kib=round(w_kib, 1),
               dispatches=[nf, nw], copy_bytes=1 << 30, copy_fetch_kib=round(f_copy, 1),
               copy_write_kib=round(w_copy, 1), sources=TRAFFIC_SOURCES,
               sources_sha256=kernel_sources_hash(TRAFFIC_SOURCES))
    with open(TRAFFIC_FILE, "w") as fh:
        json.dump(out, fh, indent=1)
        fh.write("\n")
    print(json.dumps(out))


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--routed-layout", choices=("staged", "row-major"), default="staged",
                    help="layout of the routed expert weights in the headline step")
    ap.add_argument("--weight-sets", type=int, default=8, help="distinct expert-weight copies rotated per step")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-warm", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-train", action="store_true")
    ap.add_argument("--no-stack", action="store_true")
    ap.add_argument("--no-zipf", action="store_true")
    ap.add_argument("--no-int4", action="store_true")
    ap.add_argument("--no-stream", action="store_true")
    ap.add_argument("--no-row-major", action="store_true")
    ap.add_argument("--leg", choices=("decode", "train", "stack", "zipf", "int4", "stream"),
                    help="run only this extra leg and print its result (for kernel traces of it)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 1 GiB device copy (for scaling hardware byte counters)")
    ap.add_argument("--traffic-summary", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="write the gate/up GEMM's counter summary from two rocprofv3 --pmc runs and exit")
    args = ap.parse_args()
    if args.traffic_summary:
        traffic_summary(*args.traffic_summary)
        return 0

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        return 2

    import numpy as np
    import torch
    from fine_grained_moe_amd import moe, synth

    torch.cuda.set_device(0)
    if args.leg is not None:
        fn = {"decode": bench_decode, "train": bench_train, "stack": bench_stack, "zipf": bench_zipf,
              "int4": bench_int4, "stream": bench_stream}[args.leg]
        print(json.dumps({args.leg: fn(moe, synth, torch, np)}), flush=True)
        return 0
    inp = synth.make_workload("layer_t4096", seed=0)
    T, d, E, F, Fs, k = inp.T, inp.d, inp.E, inp.F, inp.Fs, inp.k
    log(f"workload layer_t4096: T={T} d={d} E={E} F={F} Fs={Fs} k={k} bf16")
    # routed weights in the stage-major layout (packed once, as at model load)
    staged = args.routed_layout == "staged"
    dims = moe.make_dims(T, d, E, F, Fs, k, "bf16", w_routed="bf16_staged" if staged else None)

    def up(a):
        return torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(device="cuda", dtype=torch.bfloat16)

    base = dict(w_router=up(inp.w_router), w_gate_up=up(inp.w_gate_up), w_down=up(inp.w_down),
                w_sh_gate_up=up(inp.w_sh_gate_up), w_sh_down=up(inp.w_sh_down))
    if staged:
        packed_gu, packed_d = torch.empty_like(base["w_gate_up"]), torch.empty_like(base["w_down"])
        moe.moe_pack_routed_bf16(dims, base["w_gate_up"], base["w_down"], packed_gu, packed_d)
        base["w_gate_up"], base["w_down"] = packed_gu, packed_d
    sets = [base] + [{n: t.clone() for n, t in base.items()} for _ in range(max(0, args.weight_sets - 1))]
    x = up(inp.x)
    y = torch.empty_like(x)
    bias0 = torch.zeros(E, dtype=torch.float32, device="cuda")
    bias = bias0.clone()
    r = moe.alloc_routing(dims)
    ws = moe.alloc_workspace(dims)
    torch.cuda.synchronize()

    if args.copy_calibration:
        src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        log("copy calibration: 3 x 1 GiB device copies done")
        del src, dst

    ev = HipEvents()
    nph = len(PHASES) + 1
    stream = torch.cuda.current_stream().cuda_stream

    # expert-balance telemetry of every step, one row each, read after timing
    stats = torch.zeros(max(args.steps, 100, 1), 4, dtype=torch.float32, device="cuda")

    def run(wsets, steps, warmup):
        """`steps` timed steps on the host clock, bracketed by synchronisations;
        one HIP event between consecutive steps gives each step's GPU time."""
        n_sets = len(wsets)
        bias.copy_(bias0)
        for i in range(warmup):
            moe.moe_forward_bias_step(dims, x, wsets[i % n_sets], bias, GAMMA, stats[0], y, r, ws)
        marks = [ev.create() for _ in range(steps + 1)]
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(steps):
            ev.record(marks[i], stream)
            moe.moe_forward_bias_step(dims, x, wsets[(warmup + i) % n_sets], bias, GAMMA, stats[i], y, r, ws)
        ev.record(marks[steps], stream)
        torch.cuda.synchronize()
        el = time.perf_counter() - t0
        step_us = [ev.elapsed_ms(marks[i], marks[i + 1]) * 1e3 for i in range(steps)]
        for e_ in marks:
            ev.destroy(e_)
        return el, step_us

    def run_phases(wsets, steps, warmup):
        """The phase split, from a run of its own: the instrumented entry point
        records an event at every phase boundary of every step."""
        n_sets = len(wsets)
        bias.copy_(bias0)
        for i in range(warmup):
            moe.moe_forward_bias_step(dims, x, wsets[i % n_sets], bias, GAMMA, stats[0], y, r, ws)
        events = [[ev.create() for _ in range(nph)] for _ in range(steps)]
        torch.cuda.synchronize()
        for i in range(steps):
            moe.moe_forward_events(dims, x, wsets[(warmup + i) % n_sets], bias, y, r, ws, events[i],
                                   bias_step=True, gamma=GAMMA, stats=stats[i])
        torch.cuda.synchronize()
        ph = {p: [ev.elapsed_ms(events[i][j], events[i][j + 1]) * 1e3 for i in range(steps)]
              for j, p in enumerate(PHASES)}
        for row in events:
            for e_ in row:
                ev.destroy(e_)
        return {p: sum(v) / len(v) for p, v in ph.items()}, {p: percentiles(v) for p, v in ph.items()}

    n_dist = max(args.steps, 100)
    log(f"timing {args.steps} steps (+{args.warmup} warm-up) over {args.weight_sets} weight sets")
    el, step_us = run(sets, args.steps, args.warmup)
    value = T * args.steps / el
    last = stats[args.steps - 1].cpu().tolist()
    if n_dist > args.steps:
        log(f"per-step distribution: {n_dist} more steps")
        _, step_us = run(sets, n_dist, args.warmup)
    dist = percentiles(step_us)
    phases, phase_dist = run_phases(sets, n_dist, args.warmup)
    log(f"cold: {value / 1e6:.2f} M tokens/s, {el / args.steps * 1e6:.1f} us/step (host clock); per-step GPU "
        f"median {dist['median']} us (p10 {dist['p10']}, p90 {dist['p90']}); phases (us, mean): "
        + ", ".join(f"{p}={v:.1f}" for p, v in phases.items()))
    balance = dict(dead_fraction=last[0], max_over_mean=last[1], entropy=last[2], entropy_normalized=last[3])

    work = algorithmic_work(T, d, E, F, Fs, k)
    dom = max(phases, key=lambda p: phases[p])
    wd = work[dom]
    t = phases[dom] * 1e-6
    if wd["bound"] == "mfma":
        roof = dict(bound="mfma", achieved=wd["flops"] / t / 1e12, peak=PEAK_BF16_FLOPS / 1e12, unit="TFLOP/s")
    else:
        roof = dict(bound="hbm", achieved=wd["bytes"] / t / 1e9, peak=PEAK_HBM_BPS / 1e9, unit="GB/s")
    roof["frac"] = roof["achieved"] / roof["peak"]
    # hardware HBM bytes per launch of the dominant kernel (the gate/up GEMM)
    traffic = measured_traffic() if dom == "gate_up" else None
    roof["traffic"] = None if traffic is None else int(round(traffic))   # bytes per launch
    roof["algorithmic_bytes"] = wd["bytes"]
    roof["algorithmic_flops"] = wd["flops"]
    roof["kernel"] = KERNEL_OF_PHASE[dom]
    roof["avg_us"] = phases[dom]
    roof["mfma_frac"] = wd["flops"] / t / PEAK_BF16_FLOPS
    roof["hbm_frac"] = wd["bytes"] / t / PEAK_HBM_BPS

    out = {
        "metric": METRIC, "value": value, "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": el / args.steps * 1e3, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "layer_t4096", "T": T, "d": d, "E": E, "F": F, "Fs": Fs, "k": k,
                   "weight_sets": args.weight_sets, "bias_update_every_step": True,
                   "routed_weights": ("bf16, stage-major (packed once before timing)" if staged
                                      else "bf16, row-major")},
        "roofline": roof,
        "step_us": dist,
    }
    phase_report = {}
    for p, us in phases.items():
        wp = work[p]
        phase_report[p] = dict(us=round(us, 2), tflops=round(wp["flops"] / (us * 1e-6) / 1e12, 1),
                               gbps=round(wp["bytes"] / (us * 1e-6) / 1e9, 1), bound=wp["bound"],
                               dist_us=phase_dist[p])
    out["phases"] = phase_report
    out["balance"] = balance      # the last timed step's loads (the fused bias step's figures)

    if not args.no_warm:
        el_w, us_w = run(sets[:1], n_dist, args.warmup)
        out["warm"] = dict(value=T * n_dist / el_w, ms_per_step=el_w / n_dist * 1e3, step_us=percentiles(us_w))
        log(f"warm: {out['warm']['value'] / 1e6:.2f} M tokens/s, per-step median {out['warm']['step_us']['median']} us")

    if staged and not args.no_row_major:
        # the same step on row-major routed weights (what a training forward reads)
        dims_rm = moe.make_dims(T, d, E, F, Fs, k, "bf16")
        rm = dict(base)
        rm["w_gate_up"], rm["w_down"] = up(inp.w_gate_up), up(inp.w_down)
        sets_rm = [rm] + [{n: t.clone() for n, t in rm.items()} for _ in range(max(0, args.weight_sets - 1))]
        dims_save, dims = dims, dims_rm
        el_r, us_r = run(sets_rm, n_dist, args.warmup)
        dims = dims_save
        out["row_major"] = dict(value=T * n_dist / el_r, ms_per_step=el_r / n_dist * 1e3, step_us=percentiles(us_r))
        log(f"row-major routed weights: {out['row_major']['value'] / 1e6:.2f} M tokens/s, per-step median "
            f"{out['row_major']['step_us']['median']} us")
        del sets_rm, rm

    out["measured_peaks"] = measured_peaks(torch)
    mp = out["measured_peaks"]
    roof["frac_of_measured"] = (wd["flops"] / t / 1e12 / mp["bf16_gemm_tflops"] if roof["bound"] == "mfma"
                                else wd["bytes"] / t / 1e9 / mp["hbm_copy_gbps"])
    log(f"measured peaks: copy {mp['hbm_copy_gbps']} GB/s, hipBLASLt bf16 {mp['bf16_gemm_tflops']} TFLOP/s")

    if not args.no_decode:
        out["decode"] = bench_decode(moe, synth, torch, np)
    if not args.no_train:
        out["train"] = bench_train(moe, synth, torch, np)
    if not args.no_stack:
        out["stack"] = bench_stack(moe, synth, torch, np)
    if not args.no_zipf:
        out["zipf"] = bench_zipf(moe, synth, torch, np)
    if not args.no_int4:
        out["int4"] = bench_int4(moe, synth, torch, np)
    if not args.no_stream:
        out["stream"] = bench_stream(moe, synth, torch, np)

    if not args.no_cpu_baseline:
        log(f"CPU oracle baseline (~{args.cpu_seconds:.0f} s)")
        out["cpu_baseline"] = cpu_baseline(inp, args.cpu_seconds)
        log(f"CPU oracle: {out['cpu_baseline']['value']:.0f} tokens/s on {out['cpu_baseline']['cores']} threads")

    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
