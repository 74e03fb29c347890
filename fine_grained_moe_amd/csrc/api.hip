// C ABI of the MoE layer (declared in include/moe.h): argument checks on the
// host, workspace layout, and the order of kernel launches on the caller's
// stream.  Nothing here allocates, synchronises or copies.
#include <stddef.h>
#include <stdint.h>

#include <algorithm>
#include <mutex>
#include <vector>

#include "kernels.h"
#include "moe.h"

using namespace fgmoe;

namespace {

constexpr size_t kAlign = 256;
size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

size_t act_bytes(int act) { return act == MOE_BF16 ? 2 : 4; }

// Workspace regions (byte offsets from the workspace base).
struct Layout {
  size_t block_counts, rank, tile_e, tile_m0, tile_count, tile2_e, tile2_m0, tile2_count;
  size_t xb;              // moe_forward_block: x = RMSNorm(h)
  size_t H, O, Hs, S;     // forward intermediates
  size_t AU, Ou, AUs;     // training: routed pre-activations, ungated expert rows, shared pre-activations
  // backward scratch (training): padded contraction tables and transposed
  // operands (fp32; bf16 reads the activations K-major: the token of each
  // dispatch-order row, a zero row and the gate-scaled routed activations)
  size_t kofs, klen, ksh, pcol, dwr_part, dwpart, dl, dAU, dAUT, XpT, dOT, HT, dXp, WdT, WguT, WsdT, WsguT, dAUs, dAUsT, xT, dyT, HsT,
      dXs, krow, zrow, Hg;
  long long P, Tp;        // padded column counts of the routed and shared transposes
  size_t active, n_active, rkey, rscore, part_sh;   // int4 serving path: active experts, router tile maxima, fp32 shared-down partials
  size_t wdq_gu, wdq_d;   // int4 prefill: the experts' weights dequantised to bf16
  size_t total;
};

moe_status check_dims(const moe_dims* d) {
  if (!d) return MOE_E_ARG;
  if (d->T < 0 || d->d < 1 || d->E < 1 || d->F < 1 || d->Fs < 1 || d->k < 1) return MOE_E_ARG;
  if (d->act != MOE_F32 && d->act != MOE_BF16) return MOE_E_UNSUPPORTED;
  if (d->w_routed != d->act && d->w_routed != MOE_INT4_G128 && d->w_routed != MOE_BF16_STAGED)
    return MOE_E_UNSUPPORTED;
  // stage-major bf16 routed weights: whole 256-row tiles of the gate/up and
  // down launches
  if (d->w_routed == MOE_BF16_STAGED && (d->act != MOE_BF16 || d->d % 256 || d->F % 128)) return MOE_E_UNSUPPORTED;
  if (d->E > 64 || d->k > d->E || d->k > 8) return MOE_E_UNSUPPORTED;
  if (d->d % 128 || d->F % 64 || d->Fs % 64) return MOE_E_UNSUPPORTED;
  if (d->w_routed == MOE_INT4_G128) {
    // top-1 serving: bf16 activations, one expert per token, groups of 128
    // along d and F (int4_decode picks the kernels)
    if (d->act != MOE_BF16 || d->k != 1 || d->F % 128 != 0) return MOE_E_UNSUPPORTED;
  }
  const long long slots = (long long)d->T * d->k;
  const long long wide = std::max<long long>(d->d, 2LL * d->F);
  if (slots * wide >= (1LL << 31)) return MOE_E_UNSUPPORTED;
  if ((long long)d->T * std::max<long long>(d->d, 2LL * d->Fs) >= (1LL << 31)) return MOE_E_UNSUPPORTED;
  return MOE_OK;
}

// int4 top-1 batches the decode kernels take: up to kDecodeMaxT tokens at the
// layer shape they are built for.  Every other int4 batch runs the prefill
// path (route, the grouped GEMMs on the packed experts, combine), which
// serves any shape with F a multiple of 128 and any T.
bool int4_decode(const moe_dims& d) { return d.T <= kDecodeMaxT && decode_shape_supported(d.d, d.F, d.Fs); }

// Training needs the backward GEMM tiles (128 output columns over F and Fs)
// and the bf16/fp32 routed experts.
moe_status check_training(const moe_dims& d) {
  if (d.w_routed == MOE_INT4_G128 || d.w_routed == MOE_BF16_STAGED || d.F % 128 || d.Fs % 128)
    return MOE_E_UNSUPPORTED;
  return MOE_OK;
}

// The int4 prefill reads the packed experts straight into the grouped GEMMs
// (dequantised per operand fragment) when a tile's scales fit in LDS;
// otherwise the experts that received tokens are dequantised to bf16 in the
// workspace first.
bool int4_prefill_fused(const moe_dims& d) { return d.d / 128 <= kInt4MaxGroups && d.F / 128 <= kInt4MaxGroups; }

// Contraction slices of the shared down GEMM (bf16 forward): at 4096 tokens
// 256 x 256 tiles over the whole 2048-long contraction would be 64 tiles
// holding a quarter of the chip for the whole launch.  Two halves measured
// best there (four: more combine traffic, no shorter launch).  From 16384
// tokens there are tiles enough for the whole contraction, and one slice
// writes S once and the combine reads it once (skewed routing at 16384
// tokens: 436 -> 424 us per step; training at 32768: 2.69 -> 2.65 ms).
int shared_down_slices(const moe_dims& d) { return d.act == MOE_BF16 && d.T < 16384 ? 2 : 1; }

Layout make_layout(const moe_dims& d, int training) {
  Layout L{};
  const size_t es = act_bytes(d.act);
  const size_t nblk = (size_t)route_blocks(d.T, 16);   // the most router blocks of any block size
  const size_t slots = (size_t)d.T * d.k;
  const size_t tiles = (size_t)max_group_tiles((long long)slots, d.E);
  size_t o = 0;
  auto take = [&](size_t bytes) { const size_t at = o; o = align_up(o + std::max<size_t>(bytes, 1)); return at; };
  L.block_counts = take(nblk * d.E * 4);
  L.rank = take(slots * 4);
  L.tile_e = take(tiles * 4);
  L.tile_m0 = take(tiles * 4);
  L.tile_count = take(4);
  const size_t tiles2 = (size_t)max_group_tiles((long long)slots, d.E, kTileMFwd);
  L.tile2_e = take(tiles2 * 4);
  L.tile2_m0 = take(tiles2 * 4);
  L.tile2_count = take(4);
  L.xb = take((size_t)d.T * d.d * es);           // the MoE block's normalised input
  L.H = take(slots * d.F * es);
  L.Hs = take((size_t)d.T * d.Fs * es);
  if (d.w_routed == MOE_INT4_G128 && int4_decode(d)) {
    L.active = take((size_t)d.E * 3 * 4);
    L.n_active = take(4);
    L.rkey = take(4 * 64 * 8);
    L.rscore = take(4 * 64 * 4);
    L.part_sh = take((size_t)4 * d.T * d.d * 4);
    L.total = o;
    return L;
  }
  L.O = take(slots * d.d * es);
  // bf16: the shared down is split over contraction slices, each written as
  // its own [T, d] block that the combine adds
  L.S = take((size_t)d.T * d.d * es * shared_down_slices(d));
  if (d.w_routed == MOE_INT4_G128 && !int4_prefill_fused(d)) {
    L.wdq_gu = take((size_t)d.E * 2 * d.F * d.d * 2);
    L.wdq_d = take((size_t)d.E * d.d * d.F * 2);
  }
  if (training) {
    L.AU = take(slots * 2 * d.F * es);
    L.Ou = take(slots * d.d * es);
    L.AUs = take((size_t)d.T * 2 * d.Fs * es);
    const size_t E = d.E, D = d.d, F = d.F, Fs = d.Fs, T = d.T;
    L.P = pad_k((long long)slots + (long long)E * (kPadK - 1));   // whole 8-element vectors for the transposes
    L.Tp = pad_k(d.T);
    const size_t P = (size_t)L.P, Tp = (size_t)L.Tp;
    L.kofs = take(E * 4);
    L.klen = take(E * 4);
    L.ksh = take(2 * kMaxSplitK * 4);
    L.pcol = take(P * 4);
    L.dwr_part = take(P / kPadK * D * 4);
    const int S = splitk_count((long long)Tp);
    L.dwpart = take(S > 1 ? (size_t)S * std::max(2 * Fs * D, D * Fs) * 4 : 0);
    L.dl = take(slots * 4);
    const bool kmaj = d.act == MOE_BF16;
    L.dAU = take(slots * 2 * F * es);
    L.dXp = take(slots * D * es);
    if (!kmaj) {
      L.WdT = take(E * F * D * es);
      L.WguT = take(E * D * 2 * F * es);
      L.WsdT = take(Fs * D * es);
      L.WsguT = take(D * 2 * Fs * es);
    }
    L.dAUs = take(T * 2 * Fs * es);
    L.dXs = take(T * D * es);
    if (kmaj) {
      L.krow = take((slots + 32) * 4);
      L.zrow = take(512);
      L.Hg = take(slots * F * es);
    } else {
      L.dAUT = take(2 * F * P * es);
      L.XpT = take(D * P * es);
      L.dOT = take(D * P * es);
      L.HT = take(F * P * es);
      L.dAUsT = take(2 * Fs * Tp * es);
      L.xT = take(D * Tp * es);
      L.dyT = take(D * Tp * es);
      L.HsT = take(Fs * Tp * es);
    }
  }
  L.total = o;
  return L;
}

struct Range {
  const void* p;
  size_t n;
  bool out;
};

bool overlaps(const Range& a, const Range& b) {
  if (!a.p || !b.p || a.n == 0 || b.n == 0) return false;
  const uintptr_t a0 = (uintptr_t)a.p, a1 = a0 + a.n, b0 = (uintptr_t)b.p, b1 = b0 + b.n;
  return a0 < b1 && b0 < a1;
}

// Outputs may overlap nothing; inputs may overlap each other.
bool any_alias(const std::vector<Range>& rs) {
  for (size_t i = 0; i < rs.size(); ++i)
    for (size_t j = i + 1; j < rs.size(); ++j)
      if ((rs[i].out || rs[j].out) && overlaps(rs[i], rs[j])) return true;
  return false;
}

bool null_with_size(const std::vector<Range>& rs) {
  for (const Range& r : rs)
    if (!r.p && r.n) return true;
  return false;
}

void add_routing_ranges(std::vector<Range>& rs, const moe_dims& d, const moe_routing* r) {
  const size_t tk = (size_t)d.T * d.k;
  rs.push_back({r->idx, tk * 4, true});
  rs.push_back({r->gate, tk * 4, true});
  rs.push_back({r->counts, (size_t)d.E * 4, true});
  rs.push_back({r->offsets, (size_t)(d.E + 1) * 4, true});
  rs.push_back({r->perm, tk * 4, true});
  rs.push_back({r->pos, tk * 4, true});
}

template <typename P>
P* at(void* ws, size_t off) {
  return reinterpret_cast<P*>(reinterpret_cast<char*>(ws) + off);
}

// The bias step fused into a forward (moe_forward_bias_step).
struct BiasStep {
  float gamma;
  float* bias;
  float* stats;
};

// Router + loads + dispatch order; the routing outputs are complete afterwards.
// bs (may be null): the bias step, taken by the dispatch launch.
void enqueue_route(const moe_dims& d, const Layout& L, const void* x, const void* w_router, const float* bias,
                   const moe_routing* r, void* ws, hipStream_t s, const BiasStep* bs = nullptr) {
  launch_route_topk(d.act, x, w_router, bias, d.T, d.d, d.E, d.k, r->idx, r->gate, at<int32_t>(ws, L.block_counts),
                    at<int32_t>(ws, L.rank), s);
  const TileTable tiles{at<int32_t>(ws, L.tile_e), at<int32_t>(ws, L.tile_m0), at<int32_t>(ws, L.tile_count)};
  const TileTable tiles_fwd{at<int32_t>(ws, L.tile2_e), at<int32_t>(ws, L.tile2_m0), at<int32_t>(ws, L.tile2_count)};
  launch_route_dispatch(at<int32_t>(ws, L.block_counts), r->idx, at<int32_t>(ws, L.rank), route_tpb(d.T, d.act, d.d),
                        d.T, d.E, d.k,
                        r->counts, r->offsets, tiles, tiles_fwd, r->perm, r->pos, bs ? bs->gamma : 0.f,
                        bs ? bs->bias : nullptr, bs ? bs->stats : nullptr, s);
}

// Column groups of the XCD grid of a dense job with M x K and N x K operands
// (launch_gemm_fwd256): the gc in {1, 2, 4, 8} with the fewest L2 misses,
// (M * gc + N * 8 / gc) rows, at most the job's N tiles of 256.
int dense_xcd_cols(long long M, long long N) {
  int best = 1;
  long long best_rows = M + 8 * N;
  for (int gc = 2; gc <= 8; gc *= 2) {
    if ((N + 255) / 256 < gc) break;
    const long long rows = M * gc + N * (8 / gc);
    if (rows < best_rows) {
      best = gc;
      best_rows = rows;
    }
  }
  return best;
}

// From 16384 rows a dense job whose B fits an XCD's L2 runs each row item's
// N tiles back to back on one XCD (as grouped jobs do): one XCD's share of
// the A rows no longer fits its 4 MB L2, so taking the N tiles outer re-read
// them once per N tile.  Measured: the training step (32768 tokens, shared
// down, dH and dX shared jobs) 2.67 -> 2.62 ms; the skewed-routing step's
// shared down (16384) 145 -> 138 us.  The shared gate/up (8 MB of weights)
// keeps the grid (216 against 209 us), as does the 4096-token layer (no
// gain).
int dense_order(long long M, long long N) { return M >= 16384 ? -1 : dense_xcd_cols(M, N); }

moe_status device_status() { return hipGetLastError() == hipSuccess ? MOE_OK : MOE_E_DEVICE; }

// Phase-boundary events of one instrumented call (moe_forward_events): the
// caller's hipEvent_t handles, recorded on the call's stream.  Held for the
// duration of the call only; null for every other entry point.
constexpr int kMaxPhaseEvents = 8;
struct Phases {
  hipEvent_t ev[kMaxPhaseEvents];
  int n;
};

void mark_phase(const Phases* ph, int i, hipStream_t s) {
  if (ph && i < ph->n) (void)hipEventRecord(ph->ev[i], s);
}

}  // namespace

extern "C" {

const char* moe_status_str(moe_status s) {
  switch (s) {
    case MOE_OK: return "ok";
    case MOE_E_ARG: return "invalid argument (null pointer or inconsistent size)";
    case MOE_E_UNSUPPORTED: return "unsupported shape or dtype";
    case MOE_E_WORKSPACE: return "workspace missing or too small";
    case MOE_E_ALIAS: return "an output overlaps an input or another output";
    case MOE_E_DEVICE: return "the HIP runtime rejected a launch";
  }
  return "unknown status";
}

size_t moe_workspace_bytes(const moe_dims* dims, int training) {
  if (check_dims(dims) != MOE_OK) return 0;
  if (training && check_training(*dims) != MOE_OK) return 0;
  return make_layout(*dims, training ? 1 : 0).total;
}

moe_status moe_route(const moe_dims* dims, const void* x, const void* w_router, const float* bias,
                     const moe_routing* out, void* ws, size_t ws_bytes, void* stream) {
  moe_status st = check_dims(dims);
  if (st != MOE_OK) return st;
  if (!out) return MOE_E_ARG;
  const moe_dims& d = *dims;
  const size_t es = act_bytes(d.act);
  std::vector<Range> rs = {{x, (size_t)d.T * d.d * es, false},
                           {w_router, (size_t)d.E * d.d * es, false},
                           {bias, (size_t)d.E * 4, false}};
  add_routing_ranges(rs, d, out);
  if (null_with_size(rs)) return MOE_E_ARG;
  const Layout L = make_layout(d, 0);
  if (!ws || ws_bytes < L.total) return MOE_E_WORKSPACE;
  rs.push_back({ws, L.total, true});
  if (any_alias(rs)) return MOE_E_ALIAS;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  enqueue_route(d, L, x, w_router, bias, out, ws, s);
  return device_status();
}

}  // extern "C"

namespace {

// The expert GEMMs and the combine, once routing (and the dispatch tables)
// are in place: gate/up (routed + shared), down (routed + shared), combine.
// w's routed weights are act-typed (the bf16/fp32 layer, or the int4
// prefill's dequantised copies).
// routed_int4: w's routed weights are the packed int4 experts with their
// scales (the int4 prefill), read by the GEMMs directly.
moe_status enqueue_expert_gemms(const moe_dims& d, const Layout& L, const void* x, const moe_weights* w, void* y,
                                const moe_routing* routing, int training, void* ws, hipStream_t s,
                                const void* resid, const Phases* ph, bool routed_int4 = false) {
  const size_t D = d.d, F = d.F, Fs = d.Fs;
  const long long slots = (long long)d.T * d.k;
  // bf16 runs on the 256 x 256 tiles of gemm_fwd.hip (grouped jobs index the
  // 256-row tile table), fp32 on gemm.hip's 128 x 256 tiles.
  const bool big = d.act == MOE_BF16;
  const int tm = big ? kTileMFwd : kTileM;
  const int max_tiles = (int)max_group_tiles(slots, d.E, tm);
  auto gemm = big ? launch_gemm_fwd256 : launch_gemm;
  void* H = at<char>(ws, L.H);
  void* O = at<char>(ws, L.O);
  void* Hs = at<char>(ws, L.Hs);
  void* S = at<char>(ws, L.S);

  // Launch 1: routed gate/up + SwiGLU (H[slot] = silu(x_t Wg^T) * (x_t Wu^T),
  // x_t gathered by perm) and shared gate/up + SwiGLU over every token.
  GemmJob g{};
  g.epi = EPI_SWIGLU;
  g.A = x;
  g.lda = D;
  g.a_rows = routing->perm;
  g.a_div = d.k;
  g.B = w->w_gate_up;
  g.ldb = D;
  g.b_estride = 2LL * F * D;
  g.b_staged = d.w_routed == MOE_BF16_STAGED;
  g.K = d.d;
  g.N = d.F;
  g.up_off = d.F;
  g.grouped = 1;
  g.tile_e = at<int32_t>(ws, big ? L.tile2_e : L.tile_e);
  g.tile_m0 = at<int32_t>(ws, big ? L.tile2_m0 : L.tile_m0);
  g.tile_count = at<int32_t>(ws, big ? L.tile2_count : L.tile_count);
  g.offsets = routing->offsets;
  g.counts = routing->counts;
  g.max_items = max_tiles;
  g.C = H;
  g.ldc = F;
  g.aux = training ? at<char>(ws, L.AU) : nullptr;
  g.ldaux = 2LL * F;
  if (routed_int4) {
    g.b_int4 = 1;
    g.b_staged = 0;
    g.ldb = D / 2;                                   // bytes per packed row
    g.b_estride = 2LL * F * (D / 2);                 // bytes per expert
    g.b_scales = w->s_gate_up;
    g.b_sestride = 2LL * F * (D / 128);              // scales per expert
  }

  GemmJob sg{};
  sg.epi = EPI_SWIGLU;
  sg.A = x;
  sg.lda = D;
  sg.a_div = 1;
  sg.B = w->w_sh_gate_up;
  sg.ldb = D;
  sg.K = d.d;
  sg.N = d.Fs;
  sg.up_off = d.Fs;
  sg.grouped = 0;
  sg.M = d.T;
  sg.max_items = (d.T + tm - 1) / tm;
  sg.C = Hs;
  sg.ldc = Fs;
  sg.xcd_cols = dense_xcd_cols(d.T, 2LL * Fs);
  sg.aux = training ? at<char>(ws, L.AUs) : nullptr;
  sg.ldaux = 2LL * Fs;

  // int4 experts: tiles of few rows spread them over all eight waves, which
  // then share the in-register dequantisation (measured on the int4 prefill
  // at 4096 tokens, about 64 rows per expert: gate/up 78 -> 74 us, down 53 ->
  // 49 us; no change on the bf16 layer, whose loop does not wait for the
  // MFMAs of the active waves)
  GemmArgs ga{};
  ga.small_layouts = routed_int4 ? 1 : 0;
  ga.act = d.act;
  ga.njobs = 2;
  ga.order = 1;                                      // routed tiles first: they run longest
  ga.job[0] = g;
  ga.job[1] = sg;
  gemm(ga, s);
  mark_phase(ph, 2, s);

  // Launch 2: routed down, rows scaled by their routing weight
  // (O[slot] = g * (H[slot] Wd^T)), and shared down (S = Hs Wsd^T).
  GemmJob dn = g;
  dn.epi = EPI_ROWSCALE;
  dn.A = H;
  dn.lda = F;
  dn.a_rows = nullptr;
  dn.a_div = 1;
  dn.B = w->w_down;
  dn.ldb = F;
  dn.b_estride = (long long)D * F;
  dn.K = d.F;
  dn.N = d.d;
  dn.up_off = 0;
  dn.C = O;
  dn.ldc = D;
  dn.aux = training ? at<char>(ws, L.Ou) : nullptr;
  dn.ldaux = D;
  dn.gate = routing->gate;
  dn.perm = routing->perm;
  if (routed_int4) {
    dn.ldb = F / 2;
    dn.b_estride = (long long)D * (F / 2);
    dn.b_scales = w->s_down;
    dn.b_sestride = (long long)D * (F / 128);
  }

  GemmJob sd = sg;
  sd.epi = EPI_STORE;
  sd.A = Hs;
  sd.lda = Fs;
  sd.B = w->w_sh_down;
  sd.ldb = Fs;
  sd.K = d.Fs;
  sd.N = d.d;
  sd.up_off = 0;
  sd.C = S;
  sd.ldc = D;
  sd.aux = nullptr;
  const int nsd = shared_down_slices(d);
  sd.ksplit = nsd;
  sd.c_kstride = (long long)d.T * D;
  sd.xcd_cols = dense_order(d.T, D);

  GemmArgs da{};
  da.small_layouts = routed_int4 ? 1 : 0;
  da.act = d.act;
  da.njobs = 2;
  da.order = 2;                                      // shared tiles first: twice the contraction of a routed tile
  da.job[0] = dn;
  da.job[1] = sd;
  gemm(da, s);
  mark_phase(ph, 3, s);

  // combine: y[t] = S[t] + sum_j O[pos[t, j]]
  launch_combine(d.act, S, nsd, O, routing->pos, d.T, d.d, d.k, resid, y, s);
  mark_phase(ph, 4, s);
  return device_status();
}

// Top-1 serving with int4 routed experts.
// gamma (the MoE block): x is the block input h; stage 1 normalises it.
moe_status forward_int4(const moe_dims& d, const void* x, const moe_weights* w, const float* bias, void* y,
                        const moe_routing* routing, int training, void* ws, size_t ws_bytes, hipStream_t s,
                        const void* resid = nullptr, bool x_in_ws = false, const float* gamma = nullptr,
                        float eps = 0.f, const BiasStep* bs = nullptr, const int32_t* slot = nullptr,
                        int n_slots = 0, const Phases* ph = nullptr) {
  if (training) return MOE_E_UNSUPPORTED;
  // expert streaming (slot table): the decode path only
  if (slot && !int4_decode(d)) return MOE_E_UNSUPPORTED;
  const size_t E = d.E, D = d.d, F = d.F, Fs = d.Fs;
  const size_t EW = slot ? (size_t)n_slots : E;   // expert weight blocks held
  std::vector<Range> rs = {{x, (size_t)d.T * D * 2, false},
                           {w->w_router, E * D * 2, false},
                           {w->w_gate_up, EW * 2 * F * D / 2, false},
                           {w->s_gate_up, EW * 2 * F * (D / 128) * 2, false},
                           {w->w_down, EW * D * F / 2, false},
                           {w->s_down, EW * D * (F / 128) * 2, false},
                           {w->w_sh_gate_up, 2 * Fs * D * 2, false},
                           {w->w_sh_down, D * Fs * 2, false},
                           {bias, E * 4, bs != nullptr},
                           {y, (size_t)d.T * D * 2, true}};
  if (resid) rs.push_back({resid, (size_t)d.T * D * 2, false});
  if (bs && bs->stats) rs.push_back({bs->stats, 4 * 4, true});
  if (slot) rs.push_back({slot, E * 4, false});
  if (x_in_ws) rs.erase(rs.begin());             // x lives in the workspace (the block's normalised input)
  add_routing_ranges(rs, d, routing);
  if (null_with_size(rs)) return MOE_E_ARG;
  const Layout L = make_layout(d, 0);
  if (!ws || ws_bytes < L.total) return MOE_E_WORKSPACE;
  rs.push_back({ws, L.total, true});
  if (any_alias(rs)) return MOE_E_ALIAS;
  if (!int4_decode(d) && int4_prefill_fused(d)) {
    // Prefill: route, then the grouped GEMMs read the int4 experts directly
    // (each operand fragment expanded to bf16(q * scale) in registers).
    mark_phase(ph, 0, s);
    enqueue_route(d, L, x, w->w_router, bias, routing, ws, s, bs);
    mark_phase(ph, 1, s);
    return enqueue_expert_gemms(d, L, x, w, y, routing, 0, ws, s, resid, ph, true);
  }
  if (!int4_decode(d)) {
    // Prefill with contractions too long for a tile's scales in LDS: route,
    // dequantise every expert that received tokens into the workspace (bf16,
    // one rounding of q * scale), then the bf16 expert GEMMs.
    char* wgu = at<char>(ws, L.wdq_gu);
    char* wd = at<char>(ws, L.wdq_d);
    moe_weights wb = *w;
    wb.w_gate_up = wgu;
    wb.w_down = wd;
    mark_phase(ph, 0, s);
    enqueue_route(d, L, x, w->w_router, bias, routing, ws, s, bs);
    launch_dequant_int4(w->w_gate_up, w->s_gate_up, d.E, 2 * d.F, d.d, routing->counts, wgu, s);
    launch_dequant_int4(w->w_down, w->s_down, d.E, d.d, d.F, routing->counts, wd, s);
    mark_phase(ph, 1, s);
    return enqueue_expert_gemms(d, L, x, &wb, y, routing, 0, ws, s, resid, ph);
  }
  DecodeArgs a{};
  a.T = d.T;
  a.d = d.d;
  a.E = d.E;
  a.F = d.F;
  a.Fs = d.Fs;
  a.k = d.k;
  a.x = (const uint16_t*)x;
  a.w_router = (const uint16_t*)w->w_router;
  a.bias = bias;
  a.w_sh_gate_up = (const uint16_t*)w->w_sh_gate_up;
  a.w_sh_down = (const uint16_t*)w->w_sh_down;
  a.q_gate_up = (const uint8_t*)w->w_gate_up;
  a.s_gate_up = (const uint16_t*)w->s_gate_up;
  a.q_down = (const uint8_t*)w->w_down;
  a.s_down = (const uint16_t*)w->s_down;
  a.idx = routing->idx;
  a.gate = routing->gate;
  a.counts = routing->counts;
  a.offsets = routing->offsets;
  a.perm = routing->perm;
  a.pos = routing->pos;
  a.active = at<int32_t>(ws, L.active);
  a.n_active = at<int32_t>(ws, L.n_active);
  a.rkey = at<uint64_t>(ws, L.rkey);
  a.rscore = at<float>(ws, L.rscore);
  a.Hs = at<uint16_t>(ws, L.Hs);
  a.H = at<uint16_t>(ws, L.H);
  a.part_sh = at<float>(ws, L.part_sh);
  a.y = (uint16_t*)y;
  a.resid = (const uint16_t*)resid;
  a.gamma = gamma;
  a.eps = eps;
  a.xn = at<uint16_t>(ws, L.xb);
  a.slot = slot;
  a.n_slots = n_slots;
  // the next layer's router and shared gate/up, read into the caches by stage 3
  if (w->next && w->next->w_router && w->next->w_sh_gate_up) {
    a.pf_router = (const uint16_t*)w->next->w_router;
    a.pf_sh_gate_up = (const uint16_t*)w->next->w_sh_gate_up;
  }
  // the bias step: stage 2's first workgroup takes it once the loads are
  // known (the router in stage 1 is the bias's only reader)
  a.step_bias = bs ? bs->bias : nullptr;
  a.step_gamma = bs ? bs->gamma : 0.f;
  a.step_stats = bs ? bs->stats : nullptr;
  mark_phase(ph, 0, s);
  launch_decode(a, s);
  mark_phase(ph, 1, s);
  return device_status();
}

// The forward of the layer; resid (the MoE block's input h, or null) is
// added to y in the combine.  x_in_ws: x is the workspace's normalised block
// input (not checked against the workspace for overlap).
moe_status forward_core(const moe_dims* dims, const void* x, const moe_weights* w, const float* bias, void* y,
                        const moe_routing* routing, int training, void* ws, size_t ws_bytes, hipStream_t s,
                        const void* resid, bool x_in_ws, const BiasStep* bs = nullptr,
                        const Phases* ph = nullptr) {
  moe_status st = check_dims(dims);
  if (st != MOE_OK) return st;
  if (!w || !routing) return MOE_E_ARG;
  if (dims->w_routed == MOE_INT4_G128)
    return forward_int4(*dims, x, w, bias, y, routing, training, ws, ws_bytes, s, resid, x_in_ws, nullptr, 0.f, bs,
                        nullptr, 0, ph);
  const moe_dims& d = *dims;
  if (training && check_training(d) != MOE_OK) return MOE_E_UNSUPPORTED;
  const size_t es = act_bytes(d.act);
  const size_t E = d.E, D = d.d, F = d.F, Fs = d.Fs;
  std::vector<Range> rs = {{x, (size_t)d.T * D * es, false},
                           {w->w_router, E * D * es, false},
                           {w->w_gate_up, E * 2 * F * D * es, false},
                           {w->w_down, E * D * F * es, false},
                           {w->w_sh_gate_up, 2 * Fs * D * es, false},
                           {w->w_sh_down, D * Fs * es, false},
                           {bias, E * 4, bs != nullptr},
                           {y, (size_t)d.T * D * es, true}};
  if (resid) rs.push_back({resid, (size_t)d.T * D * es, false});
  if (bs && bs->stats) rs.push_back({bs->stats, 4 * 4, true});
  if (x_in_ws) rs.erase(rs.begin());
  add_routing_ranges(rs, d, routing);
  if (null_with_size(rs)) return MOE_E_ARG;
  const Layout L = make_layout(d, training ? 1 : 0);
  if (!ws || ws_bytes < L.total) return MOE_E_WORKSPACE;
  rs.push_back({ws, L.total, true});
  if (any_alias(rs)) return MOE_E_ALIAS;

  mark_phase(ph, 0, s);
  enqueue_route(d, L, x, w->w_router, bias, routing, ws, s, bs);
  mark_phase(ph, 1, s);
  if (d.T == 0) return device_status();

  return enqueue_expert_gemms(d, L, x, w, y, routing, training, ws, s, resid, ph);
}

}  // namespace

extern "C" {

}  // extern "C"

namespace {

// The workspace of moe_forward_noalloc: a static device array, one copy per
// GPU the library runs on, held until the process ends.  In host code the
// array's name is only a host-side stand-in: its device address on the
// current GPU comes from hipGetSymbolAddress, taken once per device on the
// first call there and kept in scratch_dev.
constexpr size_t kNoAllocScratchBytes = (size_t)MOE_NOALLOC_SCRATCH_BYTES;
__device__ __align__(256) char scratch[kNoAllocScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex scratch_mu;
void* scratch_dev[kMaxDevices];

// This GPU's address of `scratch`, or null if the runtime refuses it.
void* scratch_on_current_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(scratch_mu);
  if (!scratch_dev[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) {
      (void)hipGetLastError();
      return nullptr;
    }
    scratch_dev[dev] = p;
  }
  return scratch_dev[dev];
}

}  // namespace

extern "C" {

moe_status moe_forward_noalloc(const moe_dims* dims, const void* x, const moe_weights* w, const float* bias, void* y,
                               const moe_routing* routing, void* stream) {
  moe_status st = check_dims(dims);
  if (st != MOE_OK) return st;
  // the size check comes first: a refused request touches no device state
  if (make_layout(*dims, 0).total > kNoAllocScratchBytes) return MOE_E_WORKSPACE;
  void* ws = scratch_on_current_device();
  if (!ws) return MOE_E_DEVICE;
  return forward_core(dims, x, w, bias, y, routing, 0, ws, kNoAllocScratchBytes,
                      reinterpret_cast<hipStream_t>(stream), nullptr, false);
}

moe_status moe_forward(const moe_dims* dims, const void* x, const moe_weights* w, const float* bias, void* y,
                       const moe_routing* routing, int training, void* ws, size_t ws_bytes, void* stream) {
  return forward_core(dims, x, w, bias, y, routing, training, ws, ws_bytes, reinterpret_cast<hipStream_t>(stream),
                      nullptr, false);
}

moe_status moe_forward_bias_step(const moe_dims* dims, const void* x, const moe_weights* w, float* bias, float gamma,
                                 float* stats, void* y, const moe_routing* routing, int training, void* ws,
                                 size_t ws_bytes, void* stream) {
  if (!bias) return MOE_E_ARG;
  const BiasStep bs{gamma, bias, stats};
  return forward_core(dims, x, w, bias, y, routing, training, ws, ws_bytes, reinterpret_cast<hipStream_t>(stream),
                      nullptr, false, &bs);
}

moe_status moe_forward_events(const moe_dims* dims, const void* x, const moe_weights* w, float* bias, int32_t bias_step,
                              float gamma, float* stats, void* y, const moe_routing* routing, int training, void* ws,
                              size_t ws_bytes, void* stream, void* const* events, int32_t n_events) {
  if (n_events < 0 || n_events > kMaxPhaseEvents || (n_events > 0 && !events)) return MOE_E_ARG;
  if (bias_step != 0 && bias_step != 1) return MOE_E_ARG;
  Phases ph{};
  ph.n = n_events;
  for (int i = 0; i < n_events; ++i) {
    if (!events[i]) return MOE_E_ARG;
    ph.ev[i] = reinterpret_cast<hipEvent_t>(events[i]);
  }
  if (bias_step && !bias) return MOE_E_ARG;
  const BiasStep bs{gamma, bias, stats};
  return forward_core(dims, x, w, bias, y, routing, training, ws, ws_bytes, reinterpret_cast<hipStream_t>(stream),
                      nullptr, false, bias_step ? &bs : nullptr, &ph);
}

moe_status moe_forward_cached(const moe_dims* dims, const void* x, const moe_weights* w, const int32_t* slot,
                              int32_t n_slots, const float* bias, void* y, const moe_routing* routing, void* ws,
                              size_t ws_bytes, void* stream) {
  moe_status st = check_dims(dims);
  if (st != MOE_OK) return st;
  if (!w || !routing || !slot) return MOE_E_ARG;
  if (n_slots < 1 || n_slots > dims->E) return MOE_E_ARG;
  if (dims->w_routed != MOE_INT4_G128 || !int4_decode(*dims)) return MOE_E_UNSUPPORTED;
  return forward_int4(*dims, x, w, bias, y, routing, 0, ws, ws_bytes, reinterpret_cast<hipStream_t>(stream),
                      nullptr, false, nullptr, 0.f, nullptr, slot, n_slots);
}

moe_status moe_forward_block(const moe_dims* dims, const void* h, const float* norm_weight, float eps,
                             const moe_weights* w, const float* bias, void* h_out, const moe_routing* routing,
                             void* ws, size_t ws_bytes, void* stream) {
  moe_status st = check_dims(dims);
  if (st != MOE_OK) return st;
  const moe_dims& d = *dims;
  if (d.act != MOE_BF16 || d.d > 8 * 64 * kNormMaxVec) return MOE_E_UNSUPPORTED;
  if (!(eps >= 0.f) || !w || !routing) return MOE_E_ARG;
  const size_t n = (size_t)d.T * d.d * 2;
  std::vector<Range> rs = {{h, n, false}, {norm_weight, (size_t)d.d * 4, false}, {h_out, n, true}};
  if (null_with_size(rs) || !norm_weight) return MOE_E_ARG;
  const Layout L = make_layout(d, 0);
  if (!ws || ws_bytes < L.total) return MOE_E_WORKSPACE;
  rs.push_back({ws, L.total, true});
  if (any_alias(rs)) return MOE_E_ALIAS;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  // The serving path normalises h inside its first launch for one tile of
  // up to 16 tokens (measured: 18.5 -> 16.8 us per layer at T = 1); above
  // that every stage-1 workgroup would redo the norm of its token tiles (with
  // one tile per workgroup, 1040 of them at T = 64: 39.4 -> 42.9 us), and the
  // norm is a launch of its own.
  if (d.w_routed == MOE_INT4_G128 && d.T <= 16 && int4_decode(d))
    return forward_int4(d, h, w, bias, h_out, routing, 0, ws, ws_bytes, s, h, false, norm_weight, eps);
  void* x = at<char>(ws, L.xb);
  launch_rmsnorm(h, norm_weight, eps, d.T, d.d, x, s);
  if (d.w_routed == MOE_INT4_G128)
    return forward_int4(d, x, w, bias, h_out, routing, 0, ws, ws_bytes, s, h, true);
  return forward_core(dims, x, w, bias, h_out, routing, 0, ws, ws_bytes, s, h, true, nullptr, nullptr);
}

moe_status moe_bias_update(int32_t E, int64_t total_assignments, const int32_t* counts, float gamma, float* bias,
                           void* stream) {
  if (E < 1 || total_assignments < 0 || !counts || !bias) return MOE_E_ARG;
  if (E > 64) return MOE_E_UNSUPPORTED;
  std::vector<Range> rs = {{counts, (size_t)E * 4, false}, {bias, (size_t)E * 4, true}};
  if (any_alias(rs)) return MOE_E_ALIAS;
  launch_bias_update(E, (long long)total_assignments, counts, gamma, bias, nullptr,
                     reinterpret_cast<hipStream_t>(stream));
  return device_status();
}

moe_status moe_bias_update_stats(int32_t E, int64_t total_assignments, const int32_t* counts, float gamma,
                                 float* bias, float* stats, void* stream) {
  if (E < 1 || total_assignments < 0 || !counts || !bias || !stats) return MOE_E_ARG;
  if (E > 64) return MOE_E_UNSUPPORTED;
  std::vector<Range> rs = {{counts, (size_t)E * 4, false}, {bias, (size_t)E * 4, true}, {stats, 4 * 4, true}};
  if (any_alias(rs)) return MOE_E_ALIAS;
  launch_bias_update(E, (long long)total_assignments, counts, gamma, bias, stats,
                     reinterpret_cast<hipStream_t>(stream));
  return device_status();
}

moe_status moe_pack_routed_bf16(const moe_dims* dims, const void* w_gate_up, const void* w_down, void* out_gate_up,
                                void* out_down, void* stream) {
  if (!dims) return MOE_E_ARG;
  moe_dims d = *dims;
  d.w_routed = MOE_BF16_STAGED;
  d.T = 0;
  moe_status st = check_dims(&d);
  if (st != MOE_OK) return st;
  const size_t gu = (size_t)d.E * 2 * d.F * d.d * 2, dn = (size_t)d.E * d.d * d.F * 2;
  std::vector<Range> rs = {{w_gate_up, gu, false}, {w_down, dn, false}, {out_gate_up, gu, true}, {out_down, dn, true}};
  if (null_with_size(rs)) return MOE_E_ARG;
  if (any_alias(rs)) return MOE_E_ALIAS;
  launch_pack_routed(w_gate_up, w_down, d.E, d.d, d.F, out_gate_up, out_down, reinterpret_cast<hipStream_t>(stream));
  return device_status();
}

moe_status moe_quantize_int4(int32_t dtype, const void* w, int64_t rows, int32_t K, uint8_t* packed, void* scales,
                             void* stream) {
  if (rows < 0 || K < 1) return MOE_E_ARG;
  if (dtype != MOE_BF16 && dtype != MOE_F32) return MOE_E_UNSUPPORTED;
  if (K % 128 || rows * (K / 128) >= (1LL << 33)) return MOE_E_UNSUPPORTED;
  if (rows == 0) return MOE_OK;
  if (!w || !packed || !scales) return MOE_E_ARG;
  const size_t n = (size_t)rows * (size_t)K;
  std::vector<Range> rs = {{w, n * act_bytes(dtype), false}, {packed, n / 2, true}, {scales, n / 128 * 2, true}};
  if (any_alias(rs)) return MOE_E_ALIAS;
  launch_quant_int4(dtype, w, rows, K, packed, scales, reinterpret_cast<hipStream_t>(stream));
  return device_status();
}

moe_status moe_backward(const moe_dims* dims, const void* x, const moe_weights* w, const moe_routing* routing,
                        const void* dy, void* dx, const moe_grads* dw, void* ws, size_t ws_bytes, void* stream) {
  moe_status st = check_dims(dims);
  if (st != MOE_OK) return st;
  if (!w || !routing || !dw) return MOE_E_ARG;
  const moe_dims& d = *dims;
  if (check_training(d) != MOE_OK) return MOE_E_UNSUPPORTED;
  const size_t es = act_bytes(d.act);
  const size_t E = d.E, D = d.d, F = d.F, Fs = d.Fs, T = d.T;
  std::vector<Range> rs = {{x, T * D * es, false},
                           {w->w_router, E * D * es, false},
                           {w->w_gate_up, E * 2 * F * D * es, false},
                           {w->w_down, E * D * F * es, false},
                           {w->w_sh_gate_up, 2 * Fs * D * es, false},
                           {w->w_sh_down, D * Fs * es, false},
                           {dy, T * D * es, false},
                           {dx, T * D * es, true},
                           {dw->dw_router, E * D * 4, true},
                           {dw->dw_gate_up, E * 2 * F * D * 4, true},
                           {dw->dw_down, E * D * F * 4, true},
                           {dw->dw_sh_gate_up, 2 * Fs * D * 4, true},
                           {dw->dw_sh_down, D * Fs * 4, true}};
  const size_t tk = T * d.k;
  rs.push_back({routing->idx, tk * 4, false});
  rs.push_back({routing->gate, tk * 4, false});
  rs.push_back({routing->counts, E * 4, false});
  rs.push_back({routing->offsets, (E + 1) * 4, false});
  rs.push_back({routing->perm, tk * 4, false});
  rs.push_back({routing->pos, tk * 4, false});
  if (null_with_size(rs)) return MOE_E_ARG;
  const Layout L = make_layout(d, 1);
  if (!ws || ws_bytes < L.total) return MOE_E_WORKSPACE;
  rs.push_back({ws, L.total, true});
  if (any_alias(rs)) return MOE_E_ALIAS;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (T == 0) {
    // no tokens: every gradient is zero
    launch_fill_zero(dw->dw_router, E * D * 4, s);
    launch_fill_zero(dw->dw_gate_up, E * 2 * F * D * 4, s);
    launch_fill_zero(dw->dw_down, E * D * F * 4, s);
    launch_fill_zero(dw->dw_sh_gate_up, 2 * Fs * D * 4, s);
    launch_fill_zero(dw->dw_sh_down, D * Fs * 4, s);
    return device_status();
  }

  const int act = d.act;
  const int P = (int)L.P, Tp = (int)L.Tp;
  int32_t* kofs = at<int32_t>(ws, L.kofs);
  int32_t* klen = at<int32_t>(ws, L.klen);
  int32_t* ksh = at<int32_t>(ws, L.ksh);
  int32_t* pcol = at<int32_t>(ws, L.pcol);
  float* dl = at<float>(ws, L.dl);
  void* dAU = at<char>(ws, L.dAU);
  void* dAUT = at<char>(ws, L.dAUT);
  void* XpT = at<char>(ws, L.XpT);
  void* dOT = at<char>(ws, L.dOT);
  void* HT = at<char>(ws, L.HT);
  void* dXp = at<char>(ws, L.dXp);
  void* WdT = at<char>(ws, L.WdT);
  void* WguT = at<char>(ws, L.WguT);
  void* WsdT = at<char>(ws, L.WsdT);
  void* WsguT = at<char>(ws, L.WsguT);
  void* dAUs = at<char>(ws, L.dAUs);
  void* dAUsT = at<char>(ws, L.dAUsT);
  void* xT = at<char>(ws, L.xT);
  void* dyT = at<char>(ws, L.dyT);
  void* HsT = at<char>(ws, L.HsT);
  void* dXs = at<char>(ws, L.dXs);

  // bf16: the weight gradients read the activations K-major (no transposes)
  const bool kmaj = act == MOE_BF16;
  int32_t* krow = kmaj ? at<int32_t>(ws, L.krow) : nullptr;
  void* Hg = kmaj ? at<char>(ws, L.Hg) : nullptr;
  const long long slots = (long long)d.T * d.k;

  // 1. padded per-expert contraction ranges
  const int S = splitk_count(Tp), step = (int)splitk_step(Tp);
  launch_bwd_prep(routing->counts, routing->offsets, d.E, P, Tp, S, step, kofs, klen, ksh, pcol,
                  kmaj ? krow + slots : nullptr, kmaj ? at<int32_t>(ws, L.zrow) : nullptr, s);

  // 2. fp32: transposed weights W_d^T [E][F][d], W_gu^T [E][d][2F], W_sd^T
  // [Fs][d], W_sgu^T [d][2Fs] (bf16 reads the weights as stored, K-major)
  auto transpose = [&](const void* src, long long ld_src, long long sb, void* dst, long long ld_dst, long long db, int R,
                       int C, int batch, int n_in, const int32_t* map1, const int32_t* map2, int div,
                       const float* scale) {
    TransposeArgs t{};
    t.src = src;
    t.ld_src = ld_src;
    t.src_bstride = sb;
    t.dst = dst;
    t.ld_dst = ld_dst;
    t.dst_bstride = db;
    t.R = R;
    t.C = C;
    t.batch = batch;
    t.n_in = n_in;
    t.map1 = map1;
    t.map2 = map2;
    t.div = div;
    t.scale = scale;
    launch_transpose(act, t, s);
  };
  if (!kmaj) {
    transpose(w->w_down, d.F, (long long)D * F, WdT, d.d, (long long)F * D, d.F, d.d, d.E, d.d, nullptr, nullptr, 1,
              nullptr);
    transpose(w->w_gate_up, d.d, 2LL * F * D, WguT, 2 * d.F, 2LL * F * D, d.d, 2 * d.F, d.E, 2 * d.F, nullptr, nullptr,
              1, nullptr);
    transpose(w->w_sh_down, d.Fs, 0, WsdT, d.d, 0, d.Fs, d.d, 1, d.d, nullptr, nullptr, 1, nullptr);
    transpose(w->w_sh_gate_up, d.d, 0, WsguT, 2 * d.Fs, 0, d.d, 2 * d.Fs, 1, 2 * d.Fs, nullptr, nullptr, 1, nullptr);
  }

  // 3. router and gate gradients
  launch_bwd_gate(act, dy, at<char>(ws, L.Ou), x, w->w_router, routing->idx, routing->gate, routing->pos, d.T, d.d, d.k,
                  dl, krow, s);

  // bf16: the input-gradient launches run on gemm_fwd.hip's 256 x 256 tiles
  // (grouped jobs over the 256-row tile table), fp32 on gemm.hip.
  const bool big = act == MOE_BF16;
  const int tm = big ? kTileMFwd : kTileM;
  const int max_tiles = (int)max_group_tiles(slots, d.E, tm);
  auto gemm_in = big ? launch_gemm_fwd256 : launch_gemm;
  // 4. dH (gate-scaled) -> SwiGLU backward -> dAU (routed) and dAUs (shared)
  GemmJob hr{};
  hr.epi = EPI_SWIGLU_BWD;
  hr.A = dy;
  hr.lda = D;
  hr.a_rows = routing->perm;
  hr.a_div = d.k;
  // B: W_d as stored ([d][F] per expert, K-major over d) for bf16, W_d^T for fp32
  hr.B = kmaj ? w->w_down : WdT;
  hr.ldb = kmaj ? F : D;
  hr.b_estride = (long long)F * D;
  hr.kmaj = kmaj ? 2 : 0;
  hr.K = d.d;
  hr.N = d.F;
  hr.grouped = 1;
  hr.tile_e = at<int32_t>(ws, big ? L.tile2_e : L.tile_e);
  hr.tile_m0 = at<int32_t>(ws, big ? L.tile2_m0 : L.tile_m0);
  hr.tile_count = at<int32_t>(ws, big ? L.tile2_count : L.tile_count);
  hr.offsets = routing->offsets;
  hr.counts = routing->counts;
  hr.max_items = max_tiles;
  hr.C = dAU;
  hr.ldc = 2LL * F;
  hr.aux = at<char>(ws, L.AU);
  hr.ldaux = 2LL * F;
  hr.gate = routing->gate;
  hr.perm = routing->perm;
  hr.hg = Hg;   // K-major dW_d: the gate-scaled activations g * silu(a) * u
  GemmJob hs{};
  hs.epi = EPI_SWIGLU_BWD;
  hs.A = dy;
  hs.lda = D;
  hs.a_div = 1;
  hs.B = kmaj ? w->w_sh_down : WsdT;
  hs.ldb = kmaj ? Fs : D;
  hs.kmaj = kmaj ? 2 : 0;
  hs.K = d.d;
  hs.N = d.Fs;
  hs.M = d.T;
  hs.max_items = (d.T + tm - 1) / tm;
  hs.C = dAUs;
  hs.ldc = 2LL * Fs;
  hs.xcd_cols = dense_order(d.T, Fs);
  hs.aux = at<char>(ws, L.AUs);
  hs.ldaux = 2LL * Fs;
  GemmArgs g1{};
  g1.act = act;
  g1.njobs = 2;
  g1.order = 1;   // routed tiles first (even with the other orders, measured)
  g1.job[0] = hr;
  g1.job[1] = hs;
  gemm_in(g1, s);

  // 5. input gradients: dXp = dAU W_gu (per expert), dXs = dAUs W_sgu
  GemmJob xr = hr;
  xr.epi = EPI_STORE;
  xr.A = dAU;
  xr.lda = 2LL * F;
  xr.a_rows = nullptr;
  xr.a_div = 1;
  xr.B = kmaj ? w->w_gate_up : WguT;   // W_gu as stored: [2F][d] per expert, K-major over 2F
  xr.ldb = kmaj ? D : 2LL * F;
  xr.b_estride = 2LL * F * D;
  xr.K = 2 * d.F;
  xr.N = d.d;
  xr.C = dXp;
  xr.ldc = D;
  xr.aux = nullptr;
  xr.gate = nullptr;
  xr.hg = nullptr;
  GemmJob xs = hs;
  xs.epi = EPI_STORE;
  xs.A = dAUs;
  xs.lda = 2LL * Fs;
  xs.B = kmaj ? w->w_sh_gate_up : WsguT;
  xs.ldb = kmaj ? D : 2LL * Fs;
  xs.K = 2 * d.Fs;
  xs.N = d.d;
  xs.C = dXs;
  xs.ldc = D;
  xs.aux = nullptr;
  xs.xcd_cols = dense_order(d.T, D);
  GemmArgs g2{};
  g2.act = act;
  g2.njobs = 2;
  g2.order = 2;   // shared tiles first: four times the contraction of a routed tile
  g2.job[0] = xr;
  g2.job[1] = xs;
  gemm_in(g2, s);

  // 6-7. weight gradients, contracting over each expert's rows (routed) and
  // the tokens (shared, in S slices into fp32 partials, then added in order).
  // bf16: gemm_fwd.hip's 256 x 256 tiles reading the activations K-major in
  // place (x and dy through the token of each dispatch-order row; dW_d from
  // the gate-scaled activations the dH launch wrote) with an fp32 store.
  // fp32: the activations transposed over padded slot columns (routed) and
  // token columns (shared) for gemm.hip.
  float* dwpart = at<float>(ws, L.dwpart);
  float* dsgu = S > 1 ? dwpart : (float*)dw->dw_sh_gate_up;
  float* dsd = S > 1 ? dwpart : (float*)dw->dw_sh_down;
  GemmArgs g3{}, g4{};
  g3.act = g4.act = act;
  g3.njobs = g4.njobs = 2;
  g3.order = g4.order = 2;   // shared slices first: four times the contraction of a routed tile
  if (kmaj) {
    const void* zr = at<char>(ws, L.zrow);
    // C[e] (M x N) = sum over expert e's rows r of A[r, :]^T B[r, :]
    auto mjob = [&](const void* A, long long lda, const int32_t* amap, const void* B, long long ldb,
                    const int32_t* bmap, int M, int N, int nexp, const int32_t* ko, const int32_t* kl, int K, void* C,
                    long long ldc, long long cstride) {
      GemmJob j{};
      j.epi = EPI_STORE_F32;
      j.kmaj = 1;
      j.A = A;
      j.lda = lda;
      j.a_krow = amap;
      j.B = B;
      j.ldb = ldb;
      j.b_krow = bmap;
      j.zrow = zr;
      j.K = K;
      j.N = N;
      j.M = M;
      j.kgroup = 1;
      j.nexp = nexp;
      j.kofs = ko;
      j.klen = kl;
      j.max_items = nexp * ((M + tm - 1) / tm);
      j.C = C;
      j.ldc = ldc;
      j.c_estride = cstride;
      return j;
    };
    const int sl = (int)slots;
    g3.job[0] = mjob(dAU, 2LL * F, nullptr, x, D, krow, 2 * d.F, d.d, d.E, routing->offsets, routing->counts, sl,
                     dw->dw_gate_up, D, 2LL * F * D);
    g3.job[1] = mjob(dAUs, 2LL * Fs, nullptr, x, D, nullptr, 2 * d.Fs, d.d, S, ksh, ksh + S, d.T, dsgu, D,
                     2LL * Fs * D);
    g4.job[0] = mjob(dy, D, krow, Hg, F, nullptr, d.d, d.F, d.E, routing->offsets, routing->counts, sl, dw->dw_down, F,
                     (long long)D * F);
    g4.job[1] = mjob(dy, D, nullptr, at<char>(ws, L.Hs), Fs, nullptr, d.d, d.Fs, S, ksh, ksh + S, d.T, dsd, Fs,
                     (long long)D * Fs);
  } else {
    transpose(dAU, 2LL * F, 0, dAUT, P, 0, 2 * d.F, P, 1, 0, pcol, nullptr, 1, nullptr);
    transpose(x, D, 0, XpT, P, 0, d.d, P, 1, 0, pcol, routing->perm, d.k, nullptr);
    transpose(dy, D, 0, dOT, P, 0, d.d, P, 1, 0, pcol, routing->perm, d.k, routing->gate);
    transpose(at<char>(ws, L.H), F, 0, HT, P, 0, d.F, P, 1, 0, pcol, nullptr, 1, nullptr);
    transpose(dAUs, 2LL * Fs, 0, dAUsT, Tp, 0, 2 * d.Fs, Tp, 1, d.T, nullptr, nullptr, 1, nullptr);
    transpose(x, D, 0, xT, Tp, 0, d.d, Tp, 1, d.T, nullptr, nullptr, 1, nullptr);
    transpose(dy, D, 0, dyT, Tp, 0, d.d, Tp, 1, d.T, nullptr, nullptr, 1, nullptr);
    transpose(at<char>(ws, L.Hs), Fs, 0, HsT, Tp, 0, d.Fs, Tp, 1, d.T, nullptr, nullptr, 1, nullptr);
    auto kjob = [&](const void* A, long long lda, const void* B, long long ldb, int M, int N, int nexp,
                    const int32_t* ko, const int32_t* kl, void* C, long long ldc, long long cstride) {
      GemmJob j{};
      j.epi = EPI_STORE_F32;
      j.A = A;
      j.lda = lda;
      j.a_div = 1;
      j.B = B;
      j.ldb = ldb;
      j.N = N;
      j.M = M;
      j.kgroup = 1;
      j.nexp = nexp;
      j.kofs = ko;
      j.klen = kl;
      j.max_items = nexp * ((M + tm - 1) / tm);
      j.C = C;
      j.ldc = ldc;
      j.c_estride = cstride;
      return j;
    };
    g3.job[0] = kjob(dAUT, P, XpT, P, 2 * d.F, d.d, d.E, kofs, klen, dw->dw_gate_up, D, 2LL * F * D);
    g3.job[1] = kjob(dAUsT, Tp, xT, Tp, 2 * d.Fs, d.d, S, ksh, ksh + S, dsgu, D, 2LL * Fs * D);
    g4.job[0] = kjob(dOT, P, HT, P, d.d, d.F, d.E, kofs, klen, dw->dw_down, F, (long long)D * F);
    g4.job[1] = kjob(dyT, Tp, HsT, Tp, d.d, d.Fs, S, ksh, ksh + S, dsd, Fs, (long long)D * Fs);
  }
  gemm_in(g3, s);
  if (S > 1) launch_splitk_reduce(dwpart, 2LL * Fs * D, S, (float*)dw->dw_sh_gate_up, s);
  gemm_in(g4, s);
  if (S > 1) launch_splitk_reduce(dwpart, (long long)D * Fs, S, (float*)dw->dw_sh_down, s);

  // 8. router weight gradient and the input gradient
  launch_bwd_dwr(act, x, dl, routing->perm, pcol, P, kofs, klen, d.E, d.d, d.k, at<float>(ws, L.dwr_part),
                 dw->dw_router, s);
  launch_bwd_dx(act, dXs, dXp, w->w_router, dl, routing->idx, routing->pos, d.T, d.d, d.k, dx, s);
  return device_status();
}

}  // extern "C"
