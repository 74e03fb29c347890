// Router, dispatch bookkeeping and the bias step of the MoE layer (gfx950).
//
// Source: seventnews, "A relay race of rented GPUs trained NanoColibri's 2.7B
// MoE for $200", opening section, architecture paragraph: a sigmoid-plus-bias
// router over 64 experts with top-2 routing, and the per-layer expert bias
// nudged by gamma * sign(target - load) (DeepSeek-V3 recipe).
#include "balance.h"
#include "common.h"
#include "kernels.h"

namespace fgmoe {

// ---------------------------------------------------------------------------
// Router logits + sigmoid + bias + top-k + gates + per-block loads and ranks.
//
// A workgroup of 8 waves owns 16 tokens; every byte of x and of the 128 KiB
// router matrix is loaded once per workgroup.  bf16 (route_logits_staged):
// the operands are staged through LDS in 256-element chunks and wave w takes
// expert tile w % 4 over half of each chunk's k steps (two partial tiles per
// logit).  Otherwise the contraction is cut into 128-byte chunks dealt to the
// waves round-robin; for each of its chunks a wave multiplies the 16 token
// rows by all 64 router rows (four 16x16 MFMA tiles), with all of a wave's
// loads requested before its first product (eight partial tiles per logit).
// The partial tiles meet in LDS and are added in a fixed order.
//
// Selection: 8 lanes per token, eight experts per lane.  A lane keeps its k
// best keys (score + bias, then the lower expert on an exact tie, packed as
// one 64-bit key), then three DPP merges combine the 8 lanes (route_select),
// which gives the top-k of s + b in descending order with ties to the lower
// expert.  Gates are the selected scores divided by their sum.
// Per-block expert counts go to block_counts; rank[t*k + j] is the number of
// earlier assignments (t', j') of the same block with the same expert, which
// the dispatch kernel turns into the slot.
// ---------------------------------------------------------------------------
constexpr int kRouteWaves = 8;

__device__ __forceinline__ uint64_t route_key(float v, int e) {
  return ((uint64_t)float_key(v) << 32) | (uint32_t)(63 - e);
}
// Insert key c into the descending list l[0..K-1] (K is a compile-time
// constant, so this is straight-line compare-and-select code).
template <int K>
__device__ __forceinline__ void route_insert(uint64_t (&l)[K], uint64_t c) {
#pragma unroll
  for (int i = 0; i < K; ++i) {
    const bool gt = c > l[i];
    const uint64_t t = l[i];
    l[i] = gt ? c : t;
    c = gt ? t : c;
  }
}

// A lane's 64-bit key from another lane of its group of 8 (DPP, a VALU
// move): CTRL 0xB1 = quad_perm [1,0,3,2] (lane ^ 1), 0x4E = quad_perm
// [2,3,0,1] (lane ^ 2), 0x141 = row_half_mirror (lane 7 - i of the 8).
template <int CTRL>
__device__ __forceinline__ uint64_t route_dpp64(uint64_t v) {
  const uint32_t lo = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)v, CTRL, 0xF, 0xF, false);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)(v >> 32), CTRL, 0xF, 0xF, false);
  return ((uint64_t)hi << 32) | lo;
}
template <int K, int CTRL>
__device__ __forceinline__ void route_merge(uint64_t (&best)[K]) {
  uint64_t other[K];
#pragma unroll
  for (int i = 0; i < K; ++i) other[i] = route_dpp64<CTRL>(best[i]);
#pragma unroll
  for (int i = 0; i < K; ++i) route_insert<K>(best, other[i]);
}

// One token's top K over a group of 8 lanes: lane v scores experts 8v ..
// 8v + 7 (logits lrow), s = sigmoid, key (s + b, 63 - e), and keeps its K
// best; three merges (with lane ^ 1, lane ^ 2, then the mirrored lane of the
// other half, each a disjoint union; the top K of a union is within the
// union of the top Ks) leave the token's top K, descending, in all 8 lanes.
template <int K>
__device__ __forceinline__ void route_select(const float* lrow, const float* bias_s, int E, int v,
                                             uint64_t (&best)[K]) {
#pragma unroll
  for (int i = 0; i < K; ++i) best[i] = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int e = 8 * v + i;
    const float sc = sigmoidf_(lrow[e]);
    if (e < E) route_insert<K>(best, route_key(sc + bias_s[e], e));
  }
  route_merge<K, 0xB1>(best);
  route_merge<K, 0x4E>(best);
  route_merge<K, 0x141>(best);
}

// Workgroup barrier for LDS data only: this wave's LDS accesses are complete
// (lgkmcnt(0)) and every wave has reached the barrier.  Unlike __syncthreads
// it does not wait for the wave's global stores (the selections and gates
// written just before), which would cost a round trip to L2.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Loads and ranks of a block's assignments from emask[e], the block's tokens
// that selected expert e (bit t; a token selects an expert at most once):
// expert e's load in the block is popcount(emask[e]), and assignment a =
// t * K + j of expert e has rank popcount(emask[e] below bit t), the number
// of earlier assignments of the block to e.  Every thread of the block calls
// this after a barrier that follows the last update of emask.
__device__ __forceinline__ void route_loads_ranks(const int* sel, const unsigned long long* emask, int K, int E,
                                                  int na, int32_t* __restrict__ block_counts,
                                                  int32_t* __restrict__ rank) {
  const int tid = threadIdx.x;
  if (tid < E) block_counts[tid] = __popcll(emask[tid]);
  for (int a = tid; a < na; a += blockDim.x) {
    const int t = a / K, e = sel[a];
    rank[a] = __popcll(emask[e] & ((1ull << t) - 1ull));
  }
}

typedef __attribute__((address_space(3))) void* route_lds_ptr_t;

// Partial logits of the bf16 router with coalesced operand loads: the
// contraction runs in chunks of 256 elements (512-byte rows) through a
// two-deep LDS ring, x rows then router rows, copied by direct global->LDS
// loads in which every four lanes fetch 64 contiguous bytes.  (Loads straight
// into the MFMA operand layout put 16 different rows in consecutive lanes;
// measured on gfx950 that made the address unit the bound of the router at
// about 5 us per block.)  The 16-byte pieces of row r are XOR-swizzled by
// 2 (r mod 16), so the 16-row operand reads hit distinct LDS banks.  Wave w
// multiplies the 16 tokens by expert tile w % 4 over k steps 4 (w / 4) ..
// + 3 of every chunk, so each logit has two partial sums (the k halves).
constexpr int kRouteChunk = 256;                        // elements per row chunk
constexpr int kRouteRowB = kRouteChunk * 2;             // 512 bytes
constexpr int kRouteXB = 16 * kRouteRowB;               // 8 KiB of x per chunk
constexpr int kRouteStageB = kRouteXB + 64 * kRouteRowB;   // + 32 KiB of router rows
__device__ __forceinline__ int route_swz(int row, int piece) { return piece ^ ((row & 15) << 1); }

__device__ __forceinline__ void route_logits_staged(const bf16_t* __restrict__ x, const bf16_t* __restrict__ wr,
                                                    int T_, int d, int E, int tok0, char* ring, f32x4_t& acc) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  // wave w copies x rows 2w, 2w+1 and router rows 8w .. 8w+7 of each chunk;
  // one instruction moves two 512-byte rows (lane i: row i / 32, piece i % 32)
  const int half = lane >> 5, ph = lane & 31;
  const char* src[5];
  int dst[5];
  {
    const int r = 2 * wave + half;
    const int t = min(tok0 + r, T_ - 1);              // rows past T re-read the last token; never used
    src[0] = reinterpret_cast<const char*>(x + (long long)t * d) + route_swz(r, ph) * 16;
    dst[0] = 2 * wave * kRouteRowB;
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int r = 8 * wave + 2 * j + half;            // router row (expert)
    src[1 + j] = reinterpret_cast<const char*>(wr + (long long)min(r, E - 1) * d) + route_swz(r, ph) * 16;
    dst[1 + j] = kRouteXB + (8 * wave + 2 * j) * kRouteRowB;
  }
  auto issue = [&](int c) {
    char* st = ring + (c & 1) * kRouteStageB;
#pragma unroll
    for (int j = 0; j < 5; ++j)
      __builtin_amdgcn_global_load_lds(src[j] + c * kRouteRowB, (route_lds_ptr_t)(st + dst[j]), 16, 0, 0);
  };
  const int nch = d / kRouteChunk;
  const int r = lane & 15, g = lane >> 4;
  issue(0);
  if (nch > 1) issue(1);
  for (int c = 0; c < nch; ++c) {
    if (c + 1 < nch) __builtin_amdgcn_s_waitcnt((5 & 0xF) | (0x7 << 4) | (0xF << 8));   // vmcnt(5)
    else __builtin_amdgcn_s_waitcnt((0x7 << 4) | (0xF << 8));                            // vmcnt(0)
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    const char* st = ring + (c & 1) * kRouteStageB;
    const int er = (wave & 3) * 16 + r;                // this wave's expert tile
#pragma unroll
    for (int s4 = 0; s4 < 4; ++s4) {
      const int piece = 4 * (4 * (wave >> 2) + s4) + g;   // k step 4 (w / 4) + s4, lane group g
      const u32x4_t a = ld16(st + r * kRouteRowB + route_swz(r, piece) * 16);
      const u32x4_t b = ld16(st + kRouteXB + er * kRouteRowB + route_swz(er, piece) * 16);
      acc = Mma<bf16_t>::run1(a, b, acc);
    }
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();                      // every wave is done with buffer c % 2
    asm volatile("" ::: "memory");
    if (c + 2 < nch) issue(c + 2);
  }
}

// STAGED: the bf16 path above (d a multiple of 256); otherwise operands are
// loaded straight into registers.
template <typename T, int K, bool STAGED>
__global__ __launch_bounds__(512) void route_topk_kernel(const T* __restrict__ x, const T* __restrict__ wr,
                                                         const float* __restrict__ bias, int T_, int d, int E,
                                                         int32_t* __restrict__ idx,
                                                         float* __restrict__ gate,
                                                         int32_t* __restrict__ block_counts,
                                                         int32_t* __restrict__ rank) {
  // One LDS object: the staging ring, whose start later holds the partial
  // logit tiles, then the reduced logits, per-expert token masks, selections
  // and bias.
  constexpr int kRingB = STAGED ? 2 * kRouteStageB : 0;
  constexpr int kPartB = kRouteWaves * 16 * 65 * 4;
  constexpr int kHeadB = kRingB > kPartB ? kRingB : kPartB;
  __shared__ __attribute__((aligned(16))) char lds[kHeadB + 16 * 65 * 4 + 64 * 8 + 16 * K * 4 + 64 * 4];
  float (*part)[16][65] = reinterpret_cast<float (*)[16][65]>(lds);
  float (*lgs)[65] = reinterpret_cast<float (*)[65]>(lds + kHeadB);
  unsigned long long* emask = reinterpret_cast<unsigned long long*>(lds + kHeadB + 16 * 65 * 4);
  int* sel = reinterpret_cast<int*>(emask + 64);
  float* bias_s = reinterpret_cast<float*>(sel + 16 * K);
  constexpr int k = K;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r = lane & 15, g = lane >> 4;
  if (tid < 64) {
    emask[tid] = 0;
    bias_s[tid] = tid < E ? bias[tid] : 0.f;
  }

  // ---- partial logits of this wave
  const int tok0 = blockIdx.x * 16;
  f32x4_t acc[4];
#pragma unroll
  for (int et = 0; et < 4; ++et) acc[et] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  if constexpr (STAGED) {
    route_logits_staged(x, wr, T_, d, E, tok0, lds, acc[0]);
  } else {
  const int t = min(tok0 + r, T_ - 1);          // rows past T re-read the last token; never used
  const char* xrow = reinterpret_cast<const char*>(x + (long long)t * d) + g * 32;
  const char* wrow[4];
#pragma unroll
  for (int et = 0; et < 4; ++et)                 // rows past E re-read the last expert; never selected
    wrow[et] = reinterpret_cast<const char*>(wr + (long long)min(et * 16 + r, E - 1) * d) + g * 32;
  const int nch = (int)((long long)d * sizeof(T) / 128);
  for (int c0 = wave; c0 < nch; c0 += 2 * kRouteWaves) {
    // up to two chunks (c0 and c0 + 8) in flight; a missing second chunk
    // re-reads the first and is multiplied as zeros
    const int c1 = c0 + kRouteWaves < nch ? c0 + kRouteWaves : c0;
    Frag a[2], b[2][4];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int c = h ? c1 : c0;
      a[h].lo = ld16(xrow + c * 128);
      a[h].hi = ld16(xrow + c * 128 + 16);
#pragma unroll
      for (int et = 0; et < 4; ++et) {
        b[h][et].lo = ld16(wrow[et] + c * 128);
        b[h][et].hi = ld16(wrow[et] + c * 128 + 16);
      }
    }
    __builtin_amdgcn_sched_barrier(0);   // keep every load ahead of the products
    if (c1 == c0) a[1].lo = a[1].hi = u32x4_t{0u, 0u, 0u, 0u};
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int et = 0; et < 4; ++et) acc[et] = Mma<T>::run(a[h], b[h][et], acc[et]);
  }
  }
  // partial tiles: staged, part[k half][token][expert]; otherwise
  // part[wave][token][expert] (wave w: k chunks w, w + 8, ...)
  if constexpr (STAGED) {
#pragma unroll
    for (int i = 0; i < 4; ++i) part[wave >> 2][4 * g + i][(wave & 3) * 16 + r] = acc[0][i];
  } else {
#pragma unroll
    for (int et = 0; et < 4; ++et)
#pragma unroll
      for (int i = 0; i < 4; ++i) part[wave][4 * g + i][et * 16 + r] = acc[et][i];
  }
  __syncthreads();
  constexpr int kParts = STAGED ? 2 : kRouteWaves;
  for (int q = tid; q < 16 * 64; q += 512) {     // fixed-order sum of the partial tiles
    const int tt = q >> 6, e = q & 63;
    float l = 0.f;
#pragma unroll
    for (int w = 0; w < kParts; ++w) l += part[w][tt][e];
    lgs[tt][e] = l;
  }
  __syncthreads();

  // ---- selection: waves 0 and 1 take the 16 tokens, 8 lanes each
  // (route_select); lane 0 of a token's group writes its selections
  if (wave < 2) {
    const int tt = 8 * wave + (lane >> 3), v = lane & 7;
    uint64_t best[K];
    route_select<K>(lgs[tt], bias_s, E, v, best);
    const int tok = tok0 + tt;
    if (v == 0 && tok < T_) {
      float ssel[K];
      float ssum = 0.f;
#pragma unroll
      for (int j = 0; j < K; ++j) {
        const int e = 63 - (int)(uint32_t)best[j];
        ssel[j] = sigmoidf_(lgs[tt][e]);
        ssum += ssel[j];
        sel[tt * K + j] = e;
        idx[(long long)tok * K + j] = e;
        atomicOr(&emask[e], 1ull << tt);
      }
#pragma unroll
      for (int j = 0; j < K; ++j) gate[(long long)tok * K + j] = ssel[j] / ssum;
    }
  }
  lds_barrier();
  route_loads_ranks(sel, emask, K, E, min(16, T_ - tok0) * k, block_counts + (long long)blockIdx.x * E,
                    rank + (long long)tok0 * k);
}

// ---------------------------------------------------------------------------
// The router for large bf16 batches: one workgroup owns 64 tokens, so the
// 128 KiB router matrix is read a quarter as often and a 16384-token batch is
// one round of 256 workgroups instead of four rounds of 1,024.  The staging
// is route_logits_staged's with 64 x rows per chunk (a 128 KiB two-deep
// ring); wave w multiplies token tiles 2 (w & 1) .. + 1 by expert tiles
// 2 ((w >> 1) & 1) .. + 1 over k steps 4 (w >> 2) .. + 3 of every chunk, and
// the two k halves meet in LDS (first half + second half).  Selection,
// gates, per-block loads and ranks are the 16-token kernel's, over 64
// tokens (every wave selects for 8 of them; 64-bit token masks per expert).
// ---------------------------------------------------------------------------
// s_waitcnt vmcnt(N), the other counters left free (gfx9 encoding: vmcnt
// bits [3:0] and [15:14], expcnt [6:4], lgkmcnt [11:8]).
template <int N>
__device__ __forceinline__ void route_wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// RB: bytes of each row per chunk (512: a two-deep ring, the one launched;
// 256: four-deep, which measured the same on the 16384-token batch).
template <int RB>
__device__ __forceinline__ int route64_swz(int row, int piece) {
  return RB == 512 ? piece ^ ((row & 15) << 1) : piece ^ (row & 15);
}

template <int K, int RB>
__global__ __launch_bounds__(512) void route_topk64_kernel(const bf16_t* __restrict__ x,
                                                           const bf16_t* __restrict__ wr,
                                                           const float* __restrict__ bias, int T_, int d, int E,
                                                           int32_t* __restrict__ idx, float* __restrict__ gate,
                                                           int32_t* __restrict__ block_counts,
                                                           int32_t* __restrict__ rank) {
  static_assert(RB == 512 || RB == 256, "row chunks of 256 or 128 elements");
  constexpr int kXB = 64 * RB, kStageB = 2 * kXB;        // x rows, then router rows
  constexpr int kRingB = 128 * 1024, kDepth = kRingB / kStageB;
  constexpr int kPieces = RB / 16;                       // 16-byte pieces per row chunk
  constexpr int kNI = 8 * RB / 1024;                     // wave instructions per matrix and chunk
  constexpr int kKS = RB / 128;                          // k steps of 32 per chunk and k half
  static_assert(2 * 64 * 65 * 4 <= kRingB, "the two partial halves fit in the ring");
  __shared__ __attribute__((aligned(16))) char lds[kRingB + 64 * 65 * 4 + 64 * 8 + 64 * K * 4 + 64 * 4];
  float (*part)[64][65] = reinterpret_cast<float (*)[64][65]>(lds);
  float (*lgs)[65] = reinterpret_cast<float (*)[65]>(lds + kRingB);
  unsigned long long* emask = reinterpret_cast<unsigned long long*>(lds + kRingB + 64 * 65 * 4);
  int* sel = reinterpret_cast<int*>(emask + 64);
  float* bias_s = reinterpret_cast<float*>(sel + 64 * K);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r = lane & 15, g = lane >> 4;
  if (tid < 64) {
    emask[tid] = 0;
    bias_s[tid] = tid < E ? bias[tid] : 0.f;
  }
  const int tok0 = blockIdx.x * 64;

  // ---- partial logits.  Wave w copies x rows 8w .. 8w+7 and router rows
  // 8w .. 8w+7 of each chunk; one instruction moves 1 KiB (lane i: row
  // i / kPieces of the instruction's rows, piece i % kPieces).
  const int rsub = lane / kPieces, ph = lane % kPieces;
  constexpr int kRowsPerI = 1024 / RB;
  const char* src[2 * kNI];
  int dst[2 * kNI];
#pragma unroll
  for (int j = 0; j < kNI; ++j) {
    const int rr = 8 * wave + kRowsPerI * j + rsub;
    const int t = min(tok0 + rr, T_ - 1);             // rows past T re-read the last token; never used
    src[j] = reinterpret_cast<const char*>(x + (long long)t * d) + route64_swz<RB>(rr, ph) * 16;
    dst[j] = (8 * wave + kRowsPerI * j) * RB;
    src[kNI + j] = reinterpret_cast<const char*>(wr + (long long)min(rr, E - 1) * d) + route64_swz<RB>(rr, ph) * 16;
    dst[kNI + j] = kXB + (8 * wave + kRowsPerI * j) * RB;
  }
  auto issue = [&](int c) {
    char* st = lds + (c % kDepth) * kStageB;
#pragma unroll
    for (int j = 0; j < 2 * kNI; ++j) {
      // (operands computed outside the builtin: a template-dependent builtin
      // argument makes the host pass drop the kernel's launch stub)
      const char* gsrc = src[j] + c * RB;
      char* ldst = st + dst[j];
      __builtin_amdgcn_global_load_lds(gsrc, (route_lds_ptr_t)ldst, 16, 0, 0);
    }
  };
  const int tp = wave & 1, ep = (wave >> 1) & 1, kh = wave >> 2;
  f32x4_t acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  const int nch = d / (RB / 2);
#pragma unroll
  for (int c = 0; c < kDepth; ++c)
    if (c < nch) issue(c);
  for (int c = 0; c < nch; ++c) {
    // chunks issued after c: min(nch, c + kDepth) - c - 1, kNI * 2 loads each
    const int after = min(nch, c + kDepth) - c - 1;
    if (after >= 3) route_wait_vm<6 * kNI>();
    else if (after == 2) route_wait_vm<4 * kNI>();
    else if (after == 1) route_wait_vm<2 * kNI>();
    else route_wait_vm<0>();
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    const char* st = lds + (c % kDepth) * kStageB;
#pragma unroll
    for (int s = 0; s < kKS; ++s) {
      const int piece = 4 * (kKS * kh + s) + g;        // k step kKS kh + s, lane group g
      u32x4_t a[2], b[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int xr = (2 * tp + i) * 16 + r, er = (2 * ep + i) * 16 + r;
        a[i] = ld16(st + xr * RB + route64_swz<RB>(xr, piece) * 16);
        b[i] = ld16(st + kXB + er * RB + route64_swz<RB>(er, piece) * 16);
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = Mma<bf16_t>::run1(a[i], b[j], acc[i][j]);
    }
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();                      // every wave is done with buffer c % kDepth
    asm volatile("" ::: "memory");
    if (c + kDepth < nch) issue(c + kDepth);
  }
  // acc[i][j][q]: token (2 tp + i) * 16 + 4 g + q, expert (2 ep + j) * 16 + r
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q) part[kh][(2 * tp + i) * 16 + 4 * g + q][(2 * ep + j) * 16 + r] = acc[i][j][q];
  __syncthreads();
  for (int q = tid; q < 64 * 64; q += 512) {
    const int tt = q >> 6, e = q & 63;
    lgs[tt][e] = part[0][tt][e] + part[1][tt][e];
  }
  __syncthreads();

  // ---- selection: wave w takes tokens 8w .. 8w + 7, 8 lanes each
  // (route_select); lane 0 of a token's group writes its selections
  {
    const int tt = 8 * wave + (lane >> 3), v = lane & 7;
    uint64_t best[K];
    route_select<K>(lgs[tt], bias_s, E, v, best);
    const int tok = tok0 + tt;
    if (v == 0 && tok < T_) {
      float ssel[K];
      float ssum = 0.f;
#pragma unroll
      for (int j = 0; j < K; ++j) {
        const int e = 63 - (int)(uint32_t)best[j];
        ssel[j] = sigmoidf_(lgs[tt][e]);
        ssum += ssel[j];
        sel[tt * K + j] = e;
        idx[(long long)tok * K + j] = e;
        atomicOr(&emask[e], 1ull << tt);
      }
#pragma unroll
      for (int j = 0; j < K; ++j) gate[(long long)tok * K + j] = ssel[j] / ssum;
    }
  }
  lds_barrier();
  route_loads_ranks(sel, emask, K, E, min(64, T_ - tok0) * K, block_counts + (long long)blockIdx.x * E,
                    rank + (long long)tok0 * K);
}

// ---------------------------------------------------------------------------
// Loads, offsets, the grouped-GEMM tile table and the dispatch order, in one
// launch without a grid-wide barrier.  A dispatch block of 1024 threads owns
// 256 tokens, i.e. sub = 256 / tpb router blocks of tpb tokens; it sums the
// per-router-block expert counts itself (all of them for the loads, those
// before its first router block for its prefix), so every block knows
//   slot(t, j) = offsets[e] + sum over earlier router blocks of their loads of e
//                + rank(t, j) (earlier assignments to e in t's router block),
// i.e. slots of an expert ascend in t*k + j, independent of scheduling.
// Block 0 also writes counts, offsets and the tile tables, which list
// (expert, first row) for every kTileM (kTileMFwd) rows of each expert, in
// expert order.
// ---------------------------------------------------------------------------
constexpr int kDispatchTokens = 256;

// Lane e (one wave, 64 lanes) lists the tm-row tiles of expert e, which has
// cnt rows, after those of experts 0..e-1.
__device__ __forceinline__ void write_tiles(TileTable t, int tm, int cnt, int e) {
  const int nt = (cnt + tm - 1) / tm;
  int tincl = nt;
  for (int off = 1; off < 64; off <<= 1) {
    const int o = __shfl_up(tincl, off);
    if (e >= off) tincl += o;
  }
  const int texcl = tincl - nt;
  for (int m = 0; m < nt; ++m) {
    t.e[texcl + m] = e;
    t.m0[texcl + m] = m * tm;
  }
  if (e == 63) *t.count = tincl;
}
constexpr int kDispatchBatch = 16;   // count loads a thread keeps in flight
__global__ __launch_bounds__(1024) void route_dispatch_kernel(const int32_t* __restrict__ block_counts,
                                                              const int32_t* __restrict__ idx,
                                                              const int32_t* __restrict__ rank, int nblk, int T_,
                                                              int E, int k, int32_t* __restrict__ counts,
                                                              int32_t* __restrict__ offsets,
                                                              TileTable tiles, TileTable tiles_fwd,
                                                              int32_t* __restrict__ perm, int32_t* __restrict__ pos,
                                                              float gamma, float* __restrict__ bias,
                                                              float* __restrict__ stats, int tpb) {
  __shared__ int part_tot[16][64];
  __shared__ int part_pre[16][64];
  __shared__ int sub_cnt[16][64];
  __shared__ int base[16][64];
  const int tid = threadIdx.x, e = tid & 63, part = tid >> 6;
  const int sub = kDispatchTokens / tpb;         // router blocks per dispatch block: 16 or 4
  const int first = blockIdx.x * sub;            // first router block of this dispatch block
  // This block's assignments (at most 256 tokens x 8 = 2048, two per
  // thread): their experts and ranks are requested first, beside the loads
  // below, so the scatter at the end waits for no further round trip.
  const long long a0 = (long long)first * tpb * k;
  const int ntok = max(0, min(kDispatchTokens, T_ - first * tpb));
  const int na = ntok * k, per = tpb * k;
  static_assert(kDispatchTokens * 8 <= 2 * 1024, "two assignments per thread");
  int my_e[2], my_r[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int a = min(tid + 1024 * i, max(na - 1, 0));   // rows past na re-read the last one; not used
    my_e[i] = na > 0 ? idx[a0 + a] : 0;
    my_r[i] = na > 0 ? rank[a0 + a] : 0;
  }

  // loads of every router block: thread (part, e) takes blocks part, part + 16, ...;
  // the prefix counts only blocks before `first`
  int tot = 0, pre = 0;
  const int ec = min(e, E - 1);
  for (int b0 = part; b0 < nblk; b0 += 16 * kDispatchBatch) {
    int v[kDispatchBatch];
#pragma unroll
    for (int j = 0; j < kDispatchBatch; ++j)
      v[j] = block_counts[(long long)min(b0 + 16 * j, nblk - 1) * E + ec];
#pragma unroll
    for (int j = 0; j < kDispatchBatch; ++j) {
      const int b = b0 + 16 * j;
      const int vv = (b < nblk && e < E) ? v[j] : 0;
      tot += vv;
      pre += b < first ? vv : 0;
    }
  }
  part_tot[part][e] = tot;
  part_pre[part][e] = pre;
  sub_cnt[part][e] = (e < E && part < sub && first + part < nblk) ? block_counts[(long long)(first + part) * E + e] : 0;
  __syncthreads();

  if (part == 0) {
    int cnt = 0, pr = 0;
    for (int q = 0; q < 16; ++q) {
      cnt += part_tot[q][e];
      pr += part_pre[q][e];
    }
    if (e >= E) cnt = 0;
    int incl = cnt;
    for (int off = 1; off < 64; off <<= 1) {
      const int o = __shfl_up(incl, off);
      if (e >= off) incl += o;
    }
    const int excl = incl - cnt;
    int run = excl + pr;
    for (int sb = 0; sb < sub; ++sb) {
      base[sb][e] = run;
      run += sub_cnt[sb][e];
    }
    if (blockIdx.x == 0) {
      if (e < E) {
        counts[e] = cnt;
        offsets[e] = excl;
      }
      if (e == E - 1) offsets[E] = incl;
      write_tiles(tiles, kTileM, cnt, e);
      if (tiles_fwd.e) write_tiles(tiles_fwd, kTileMFwd, cnt, e);
      // the fused bias step: the router has read the bias (it ran before this launch)
      if (bias) bias_step_wave(e, E, (long long)T_ * k, cnt, gamma, bias, stats);
    }
  }
  __syncthreads();

#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int a = tid + 1024 * i;
    if (a < na) {
      const int slot = base[a / per][my_e[i]] + my_r[i];
      perm[slot] = (int32_t)(a0 + a);
      pos[a0 + a] = slot;
    }
  }
}

// ---------------------------------------------------------------------------
// bias[e] <- fl32(bias[e] + gamma * sign(total - E * counts[e])).
// ---------------------------------------------------------------------------
__global__ void bias_update_kernel(int E, long long total, const int32_t* __restrict__ counts, float gamma,
                                   float* __restrict__ bias) {
  const int e = blockIdx.x * blockDim.x + threadIdx.x;
  if (e < E) {
    const long long diff = total - (long long)E * (long long)counts[e];
    const float sg = (float)((diff > 0) - (diff < 0));
    bias[e] = __fadd_rn(bias[e], gamma * sg);
  }
}

// ---------------------------------------------------------------------------
// The bias step plus the batch's expert-balance telemetry (bias_step_wave).
// One wave, lane e for expert e.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(64) void bias_update_stats_kernel(int E, long long total,
                                                               const int32_t* __restrict__ counts, float gamma,
                                                               float* __restrict__ bias, float* __restrict__ stats) {
  const int e = threadIdx.x;
  bias_step_wave(e, E, total, e < E ? counts[e] : 0, gamma, bias, stats);
}

template <typename A, int K>
void launch_topk_k(const void* x, const void* w_router, const float* bias, int T, int d, int E, int32_t* idx,
                   float* gate, int32_t* block_counts, int32_t* rank, hipStream_t s) {
  constexpr int act = sizeof(A) == 2 ? 1 : 0;
  const int tpb = route_tpb(T, act, d), nblk = route_blocks(T, tpb);
  if constexpr (sizeof(A) == 2) {
    if (tpb == 64) {
      hipLaunchKernelGGL((route_topk64_kernel<K, 512>), dim3(nblk), dim3(512), 0, s, (const A*)x, (const A*)w_router, bias,
                         T, d, E, idx, gate, block_counts, rank);
      return;
    }
    if (d % kRouteChunk == 0) {
      hipLaunchKernelGGL((route_topk_kernel<A, K, true>), dim3(nblk), dim3(512), 0, s, (const A*)x,
                         (const A*)w_router, bias, T, d, E, idx, gate, block_counts, rank);
      return;
    }
  }
  hipLaunchKernelGGL((route_topk_kernel<A, K, false>), dim3(nblk), dim3(512), 0, s, (const A*)x,
                       (const A*)w_router, bias, T, d, E, idx, gate, block_counts, rank);
}
template <typename A>
void launch_topk_t(const void* x, const void* w_router, const float* bias, int T, int d, int E, int k, int32_t* idx,
                   float* gate, int32_t* block_counts, int32_t* rank, hipStream_t s) {
  switch (k) {
    case 1: launch_topk_k<A, 1>(x, w_router, bias, T, d, E, idx, gate, block_counts, rank, s); break;
    case 2: launch_topk_k<A, 2>(x, w_router, bias, T, d, E, idx, gate, block_counts, rank, s); break;
    case 3: launch_topk_k<A, 3>(x, w_router, bias, T, d, E, idx, gate, block_counts, rank, s); break;
    case 4: launch_topk_k<A, 4>(x, w_router, bias, T, d, E, idx, gate, block_counts, rank, s); break;
    case 5: launch_topk_k<A, 5>(x, w_router, bias, T, d, E, idx, gate, block_counts, rank, s); break;
    case 6: launch_topk_k<A, 6>(x, w_router, bias, T, d, E, idx, gate, block_counts, rank, s); break;
    case 7: launch_topk_k<A, 7>(x, w_router, bias, T, d, E, idx, gate, block_counts, rank, s); break;
    default: launch_topk_k<A, 8>(x, w_router, bias, T, d, E, idx, gate, block_counts, rank, s); break;
  }
}

// k is 1..8 (checked on the host).
void launch_route_topk(int act, const void* x, const void* w_router, const float* bias, int T, int d, int E,
                       int k, int32_t* idx, float* gate, int32_t* block_counts, int32_t* rank, hipStream_t s) {
  if (T == 0) return;
  if (act == 1) launch_topk_t<bf16_t>(x, w_router, bias, T, d, E, k, idx, gate, block_counts, rank, s);
  else launch_topk_t<float>(x, w_router, bias, T, d, E, k, idx, gate, block_counts, rank, s);
}

void launch_route_dispatch(const int32_t* block_counts, const int32_t* idx, const int32_t* rank, int tpb, int T,
                           int E, int k, int32_t* counts, int32_t* offsets, TileTable tiles, TileTable tiles_fwd,
                           int32_t* perm, int32_t* pos, float gamma, float* bias, float* stats, hipStream_t s) {
  const int nblk = route_blocks(T, tpb), sub = kDispatchTokens / tpb;
  const int grid = nblk > 0 ? (nblk + sub - 1) / sub : 1;   // block 0 runs even for T = 0
  hipLaunchKernelGGL(route_dispatch_kernel, dim3(grid), dim3(1024), 0, s, block_counts, idx, rank, nblk, T, E, k,
                     counts, offsets, tiles, tiles_fwd, perm, pos, gamma, bias, stats, tpb);
}

void launch_bias_update(int E, long long total, const int32_t* counts, float gamma, float* bias, float* stats,
                        hipStream_t s) {
  if (stats)
    hipLaunchKernelGGL(bias_update_stats_kernel, dim3(1), dim3(64), 0, s, E, total, counts, gamma, bias, stats);
  else
    hipLaunchKernelGGL(bias_update_kernel, dim3(1), dim3(64), 0, s, E, total, counts, gamma, bias);
}

}  // namespace fgmoe
