// Top-1 serving path of the MoE layer with int4 routed experts (gfx950).
//
// Source: seventnews, "A relay race of rented GPUs trained NanoColibri's 2.7B
// MoE for $200".  "Relay training" section, top-2 paragraph: at serving time
// the engine runs one expert per token (top-1, so the routing weight is 1).
// Opening section, proof-of-loop paragraph: experts ship in int4 containers;
// the shared expert never leaves memory.  The int4 format (symmetric, one
// bf16 scale per 128 consecutive elements of a row, two's-complement nibbles,
// element 2i in the low nibble) is this library's reading; the article names
// only "int4".
//
// Three launches for a batch of at most 64 tokens (a launch costs about
// 1.3 us on the device even when empty, so the work is packed into as few
// dependent steps as the data flow allows):
//   stage 1  router (logits on MFMA, top-1, gate) beside the shared
//            expert's gate/up, which does not depend on the routing; a
//            workgroup per 16 weight rows, over every 16-token tile (in the
//            MoE block, at most 16 tokens, every workgroup first normalises
//            the rows of h, and the router's first expert tile writes them
//            for stage 2);
//   stage 2  one workgroup writes the routing outputs (loads, offsets,
//            dispatch order, active experts) and takes the bias step of
//            moe_forward_bias_step; the shared down in four
//            contraction quarters (fp32 partials); the routed gate/up of each
//            active expert over its own tokens (int4 dequantised in
//            registers);
//   stage 3  the routed down of each active expert, fused with the combine:
//            y = (the four shared partials added in order) + the token's
//            routed row, rounded once (top-1: the gate is 1).
// Every workgroup streams 8 to 32 KiB of weights, all of it requested before
// the first product, so that every CU has its loads in flight at once.
// Operands reach the MFMAs through LDS: an MFMA operand held in registers
// puts 16 different rows in consecutive lanes, and a CU's address unit then
// spends 64 cycles instead of 16 on each 1 KiB wave load (measured with the
// TA busy counter), which made the address units, not HBM, the limit.
// Weight rows are copied with direct global->LDS loads in which four
// consecutive lanes fetch 64 contiguous bytes of one row; activation rows
// are copied row-contiguously (only the rows that exist) into XOR-swizzled
// LDS rows; each wave then reads its fragments from LDS.
// Serving callers should capture the forward in a HIP graph (the host's
// launch cost exceeds the GPU time at this size); nothing here allocates,
// synchronises or clears memory with hipMemsetAsync, so the calls are
// capturable.
// int4 products: nibbles are exact small integers in bf16, so each
// 128-element group is multiplied on MFMA into a fresh accumulator and then
// scaled once in fp32 (w = q * scale is never rounded to bf16).
// The path is HBM-bound: every weight byte is read once per call.
#include "balance.h"
#include "common.h"
#include "kernels.h"

namespace fgmoe {

namespace {


constexpr int kGroup = 128;   // int4 scale group along the contraction dimension

// 8 nibbles (one 32-bit word, element 2i in the low nibble of byte i) -> the
// 8 bf16 values of the signed integers they hold, in element order (one
// 16-byte MFMA operand).  Exact: every integer in [-8, 7] is a bf16.
__device__ __forceinline__ u32x4_t int4x8_to_bf16(uint32_t w) {
  u32x4_t r;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const float lo = (float)(((int)(w << (28 - 8 * j))) >> 28);
    const float hi = (float)(((int)(w << (24 - 8 * j))) >> 28);
    r[j] = __builtin_amdgcn_perm(__float_as_uint(hi), __float_as_uint(lo), 0x07060302u);
  }
  return r;
}

__device__ __forceinline__ float sum4(const float* p, int stride) {
  return ((p[0] + p[stride]) + p[2 * stride]) + p[3 * stride];
}

// Pack 8 floats as 8 bf16 (round to nearest even).
__device__ __forceinline__ u32x4_t pack8(const float* v) {
  u32x4_t r;
#pragma unroll
  for (int j = 0; j < 4; ++j) r[j] = (uint32_t)f32_to_bf16(v[2 * j]) | ((uint32_t)f32_to_bf16(v[2 * j + 1]) << 16);
  return r;
}



typedef __attribute__((address_space(3))) void* lds_ptr_t;

// Weight blocks in LDS: 16 rows x 64 bytes (1 KiB), the 16-byte piece p of
// row r at physical piece p ^ wswz(r), so that the 32 pieces of a half-wave
// MFMA operand read (16 rows x 2 pieces) fall in distinct bank groups.
__device__ __forceinline__ int wswz(int row) { return ((row >> 3) & 1) << 1; }

// Copy NB consecutive 64-byte blocks of 16 weight rows into LDS (block b at
// dst + 1024 b).  Lane l fetches piece (l % 4) ^ wswz(l / 4) of row l / 4;
// row_k is this lane's row address at the first block.
template <int NB>
__device__ __forceinline__ void dma_w(const char* row_k, char* dst, int lane) {
  const char* src = row_k + (((lane & 3) ^ wswz(lane >> 2)) << 4);
#pragma unroll
  for (int b = 0; b < NB; ++b) __builtin_amdgcn_global_load_lds(src + b * 64, (lds_ptr_t)(dst + b * 1024), 16, 0, 0);
}

// Lane (fr, g)'s MFMA operand from a weight block: piece g of row fr.
__device__ __forceinline__ u32x4_t wfrag(const char* blk, int fr, int g) {
  return *reinterpret_cast<const u32x4_t*>(blk + fr * 64 + ((g ^ wswz(fr)) << 4));
}

// Activation rows in LDS: 16 rows of Q bytes, piece c of row r at c ^ xsw(r).
// The XOR makes the bf16 MFMA reads (pieces 4b + g of rows 0..15) hit 32
// distinct bank groups per half-wave.
template <int Q> __device__ __forceinline__ int xsw(int r) { return Q == 512 ? (2 * r) & 31 : r & 14; }

// Copy rows 0 .. n-1 (1 <= n <= 16) of this wave's Q-byte slice of an
// activation operand into LDS.  Row r is read at base + idx(r) * stride with
// idx(r) = list[r] (or r).  Lane l of step i copies piece 64 i + l of the 16
// rows, so the reads are row-contiguous; all loads are issued before the
// stores, unconditionally (lanes past row n - 1 re-read it): a load under a
// lane condition would be waited for at the end of its branch.
template <int Q>
__device__ __forceinline__ void stage_rows(char* dst, const char* base, long long stride, const int* list, int n,
                                           int lane) {
  constexpr int PR = Q / 16, NS = 16 * PR / 64;
  u32x4_t v[NS];
#pragma unroll
  for (int i = 0; i < NS; ++i) {
    const int pc = i * 64 + lane, r = min(pc / PR, n - 1), c = pc % PR;
    v[i] = ld16(base + (long long)(list ? list[r] : r) * stride + c * 16);
  }
#pragma unroll
  for (int i = 0; i < NS; ++i) {
    const int pc = i * 64 + lane, r = pc / PR, c = pc % PR;
    if (r < n) st16(dst + r * Q + ((c ^ xsw<Q>(r)) << 4), v[i]);
  }
}

// stage_rows<512> for the MoE block: the staged quarter (wave w holds
// columns 256 w .. 256 w + 255 of the 16 rows) is normalised on the way to
// LDS, x = bf16(h / sqrt(mean(h^2) + eps) * gamma).  Each wave sums the
// squares of its quarter per row (lane order, then a butterfly over the 32
// lanes of a row), the 4 quarters meet in red[4][16] and are added in wave
// order; every wave of the workgroup calls this (it holds a barrier).  With
// xn, the normalised rows 0 .. n-1 are also written there.
__device__ __forceinline__ void stage_rows_norm(char* dst, const char* base, long long stride, int n, int lane,
                                                int wave, int d, const float* gamma, float eps, float* red,
                                                uint16_t* xn) {
  constexpr int PR = 32, NS = 8;                     // 512-byte quarters: 32 pieces per row
  u32x4_t v[NS];
#pragma unroll
  for (int i = 0; i < NS; ++i) {
    const int pc = i * 64 + lane, r = min(pc / PR, n - 1), c = pc % PR;
    v[i] = ld16(base + (long long)r * stride + c * 16);
  }
  float ps[NS];
#pragma unroll
  for (int i = 0; i < NS; ++i) {
    ps[i] = 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float lo = bf16_to_f32((bf16_t)(v[i][j] & 0xFFFF)), hi = bf16_to_f32((bf16_t)(v[i][j] >> 16));
      ps[i] += lo * lo;
      ps[i] += hi * hi;
    }
#pragma unroll
    for (int off = 1; off < 32; off <<= 1) ps[i] += __shfl_xor(ps[i], off);
  }
  // lane 0 holds rows 0, 2, .., 14 of this quarter, lane 32 rows 1, 3, .., 15
  if ((lane & 31) == 0) {
#pragma unroll
    for (int i = 0; i < NS; ++i) red[wave * 16 + 2 * i + (lane >> 5)] = ps[i];
  }
  __syncthreads();
  const int c = lane % PR;
  const float4 g0 = *reinterpret_cast<const float4*>(gamma + wave * 256 + c * 8);
  const float4 g1 = *reinterpret_cast<const float4*>(gamma + wave * 256 + c * 8 + 4);
  const float gm[8] = {g0.x, g0.y, g0.z, g0.w, g1.x, g1.y, g1.z, g1.w};
#pragma unroll
  for (int i = 0; i < NS; ++i) {
    const int r = 2 * i + (lane >> 5);
    const float ss = ((red[r] + red[16 + r]) + red[32 + r]) + red[48 + r];
    const float rstd = 1.f / sqrtf(ss / (float)d + eps);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float lo = bf16_to_f32((bf16_t)(v[i][j] & 0xFFFF)), hi = bf16_to_f32((bf16_t)(v[i][j] >> 16));
      v[i][j] = pack_bf16x2(lo * rstd * gm[2 * j], hi * rstd * gm[2 * j + 1]);
    }
    if (r < n) {
      st16(dst + r * 512 + ((c ^ xsw<512>(r)) << 4), v[i]);
      if (xn) st16(xn + (long long)r * d + wave * 256 + c * 8, v[i]);
    }
  }
}

// Lane fr's operand piece `piece` of activation row fr.  Rows >= n hold stale
// data; they only feed MFMA output rows that are never stored.
template <int Q>
__device__ __forceinline__ u32x4_t xfrag(const char* src, int fr, int piece) {
  return *reinterpret_cast<const u32x4_t*>(src + fr * Q + ((piece ^ xsw<Q>(fr)) << 4));
}

// This wave's direct LDS loads and LDS stores have completed
// (s_waitcnt vmcnt(0) expcnt(0) lgkmcnt(0)).
__device__ __forceinline__ void wait_all() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0);
  asm volatile("" ::: "memory");
}

// Token-tiled items: item i of a launch goes to weight block `blk` and token
// tile `tile` such that the tiles of one weight block share i % 8, hence the
// XCD (consecutive workgroups are dealt to the 8 XCDs in turn), and read the
// block's weights through one L2.  nblk must be a multiple of 8.
__device__ __forceinline__ void xcd_item(int i, int ntile, int& blk, int& tile) {
  const int x = i & 7, j = i >> 3;
  const int jb = j / ntile;
  blk = jb * 8 + x;
  tile = j - jb * ntile;
}

// ---------------------------------------------------------------------------
// Stage 1.  A workgroup multiplies 16 bf16 weight rows by 16 tokens of x over
// the whole contraction d; wave w takes contraction quarter w (8 MFMA steps
// of 32); the 4 partial 16x16 tiles are added in LDS in a fixed order.
//   shared gate/up item (hb, tt): rows = 8 gate rows 8 hb .. + 7 (MFMA
//     columns 0-7) and the matching up rows (8-15); h = silu(gate) * up.
//   router item (tt, et): rows = experts 16 et .. + 15 (rows past E re-read
//     expert E - 1 and are not used).  s = sigmoid(logit); key = (order key
//     of s + b, 63 - e), so the largest key is the largest s + b and an exact
//     tie goes to the lower expert.  Each token's largest key in the tile
//     and its s go to rkey/rscore [et][t]; the top-1 is the largest of the 4
//     tile keys (stage 2).
// LDS per wave: 8 weight blocks (8 KiB), then 16 x rows (8 KiB), whose space
// takes the wave's partial tile [16][17] after the products.  Launched for
// one token tile (at most 16 tokens, with the MoE block's norm); above that
// decode_stage1_wide_kernel below takes the tiles of a weight block together.
// ---------------------------------------------------------------------------
constexpr int kS1Wave = 16384;

// write_xn: the MoE block's normalised rows of this token tile go to p.xn.
template <int D>
__device__ f32x4_t stage1_tile(const char* wrow, int tt, int T, const DecodeArgs& p, char* wreg, float* red,
                               bool write_xn) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int fr = lane & 15, g = lane >> 4;
  static_assert(D == 1024, "one contraction quarter is 512 bytes");
  dma_w<8>(wrow + wave * (D / 2), wreg, lane);
  const char* xq = reinterpret_cast<const char*>(p.x) + (long long)tt * 16 * D * 2 + wave * (D / 2);
  if (p.gamma)
    stage_rows_norm(wreg + 8192, xq, (long long)D * 2, min(16, T - tt * 16), lane, wave, D, p.gamma, p.eps, red,
                    write_xn ? p.xn + (long long)tt * 16 * D : nullptr);
  else
    stage_rows<512>(wreg + 8192, xq, (long long)D * 2, nullptr, min(16, T - tt * 16), lane);
  wait_all();
  f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int b = 0; b < 8; ++b) acc = Mma<bf16_t>::run1(xfrag<512>(wreg + 8192, fr, 4 * b + g), wfrag(wreg + b * 1024, fr, g), acc);
  // acc[i]: token row 4g + i, weight row fr
  float* part = reinterpret_cast<float*>(wreg + 8192);
#pragma unroll
  for (int i = 0; i < 4; ++i) part[(4 * g + i) * 17 + fr] = acc[i];
  return acc;
}

// the sum over the 4 waves of partial element (r, c), in wave order
__device__ __forceinline__ float part_sum(const char* lds, int wave_bytes, int off_bytes, int idx) {
  const float* q = reinterpret_cast<const float*>(lds + off_bytes) + idx;
  const int st = wave_bytes / 4;
  return ((q[0] + q[st]) + q[2 * st]) + q[3 * st];
}

template <int D, int FS>
__global__ __launch_bounds__(256) void decode_stage1_kernel(DecodeArgs p, int ntile) {
  __shared__ __align__(16) char lds[4 * kS1Wave];
  __shared__ float red[64];                           // the MoE block's per-quarter sums of squares
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  char* wreg = lds + wave * kS1Wave;
  const int n_sh = (FS / 8) * ntile;
  const int blk = blockIdx.x, T = p.T;
  const int r = lane >> 2;                            // the weight row this lane's direct loads fetch
  if (blk < n_sh) {
    int hb, tt;
    xcd_item(blk, ntile, hb, tt);
    const int f = hb * 8 + (r & 7);
    const int wr = r < 8 ? f : FS + f;
    stage1_tile<D>(reinterpret_cast<const char*>(p.w_sh_gate_up) + (long long)wr * D * 2, tt, T, p, wreg, red,
                   false);
    __syncthreads();
    const int t = tt * 16 + tid;
    if (tid < 16 && t < T) {
      float h[8];
#pragma unroll
      for (int c = 0; c < 8; ++c)
        h[c] = siluf_(part_sum(lds, kS1Wave, 8192, tid * 17 + c)) * part_sum(lds, kS1Wave, 8192, tid * 17 + 8 + c);
      st16(p.Hs + (long long)t * FS + hb * 8, pack8(h));
    }
  } else {
    const int rr = blk - n_sh, tt = rr >> 2, et = rr & 3;
    const int t = tid >> 4, c = tid & 15, e = et * 16 + c;
    const float b = e < p.E ? p.bias[e] : 0.f;
    stage1_tile<D>(reinterpret_cast<const char*>(p.w_router) + (long long)min(et * 16 + r, p.E - 1) * D * 2, tt, T, p,
                   wreg, red, et == 0);
    __syncthreads();
    const float sc = 1.0f / (1.0f + expf(-part_sum(lds, kS1Wave, 8192, t * 17 + c)));
    uint64_t key = e < p.E ? (((uint64_t)float_key(sc + b) << 32) | (uint32_t)(63 - e)) : 0ull;
    float ks = sc;
#pragma unroll
    for (int off = 1; off < 16; off <<= 1) {
      const uint32_t lo = __shfl_xor((uint32_t)key, off), hi = __shfl_xor((uint32_t)(key >> 32), off);
      const float os = __shfl_xor(ks, off);
      const uint64_t o = ((uint64_t)hi << 32) | lo;
      if (o > key) {
        key = o;
        ks = os;
      }
    }
    if (c == 0 && tt * 16 + t < T) {
      p.rkey[et * 64 + tt * 16 + t] = key;
      p.rscore[et * 64 + tt * 16 + t] = ks;
    }
  }
}

// ---------------------------------------------------------------------------
// Stage 1 above 16 tokens (NT = 2 .. 4 token tiles; the MoE block's norm is
// then a launch of its own, so gamma is not used here).  A workgroup owns one
// weight block (the same 16 rows as above) and every token tile, so the
// block is read once per launch instead of once per tile, and the grid is
// one round of FS / 8 + 4 workgroups instead of NT rounds' worth: a CU takes
// in 160 KiB at 64 tokens instead of 256 KiB (the bound here is what a CU's
// vector memory path delivers, about 60 GB/s on this access pattern).  Wave
// w copies its contraction quarter of the block into LDS and reads it into
// registers (8 MFMA operands); its LDS space then holds two token tiles at a
// time.  Every load is issued at the start (the weights, then each tile's
// rows, row-contiguously into registers), so each wave has up to 40 KiB in
// flight, and a tile is multiplied, reduced and finished while the later
// tiles' rows are still arriving.  The four partial tiles meet in LDS in two
// alternating buffers (one barrier per tile) and are added in wave order, as
// above.
// ---------------------------------------------------------------------------
template <int D, int FS, int NT>
__global__ __launch_bounds__(256) void decode_stage1_wide_kernel(DecodeArgs p) {
  static_assert(D == 1024, "one contraction quarter is 512 bytes");
  static_assert(NT >= 2 && NT <= 4, "17 to 64 tokens");
  __shared__ __align__(16) char lds[4 * kS1Wave];
  __shared__ float part[2][4][16 * 17];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int fr = lane & 15, g = lane >> 4;
  char* wreg = lds + wave * kS1Wave;
  const int blk = blockIdx.x, T = p.T;
  const int n_sh = FS / 8;
  const int r = lane >> 2;                            // the weight row this lane's direct loads fetch
  const bool is_sh = blk < n_sh;
  const char* wrow;
  if (is_sh) {
    const int f = blk * 8 + (r & 7);
    wrow = reinterpret_cast<const char*>(p.w_sh_gate_up) + (long long)(r < 8 ? f : FS + f) * D * 2;
  } else {
    wrow = reinterpret_cast<const char*>(p.w_router) + (long long)min((blk - n_sh) * 16 + r, p.E - 1) * D * 2;
  }
  dma_w<8>(wrow + wave * (D / 2), wreg, lane);
  __builtin_amdgcn_sched_barrier(0);                  // the weight loads are the oldest in flight
  // a router item's bias of expert 16 et + (tid % 16), loaded unconditionally
  // (a load under a branch is waited for where the branch ends)
  const float bias_c = p.bias[is_sh ? 0 : min((blk - n_sh) * 16 + (tid & 15), p.E - 1)];
  // this wave's quarter of every tile's rows: lane l of step i holds piece
  // 64 i + l of the 16 rows (rows past T re-read the last token)
  constexpr int PR = 32, NS = 8;
  const char* xq = reinterpret_cast<const char*>(p.x) + wave * (D / 2);
  u32x4_t v[NT][NS];
#pragma unroll
  for (int tt = 0; tt < NT; ++tt) {
#pragma unroll
    for (int i = 0; i < NS; ++i) {
      const int pc = i * 64 + lane, t = min(tt * 16 + pc / PR, T - 1), c = pc % PR;
      v[tt][i] = ld16(xq + (long long)t * D * 2 + c * 16);
    }
    __builtin_amdgcn_sched_barrier(0);                // tile by tile, in order
  }
  // s_waitcnt vmcnt(8 NT + 1): the weight copies, issued first, have landed
  constexpr int kAfterW = 8 * NT + 1;
  __builtin_amdgcn_s_waitcnt((kAfterW & 0xF) | ((kAfterW >> 4) << 14) | (0x7 << 4) | (0xF << 8));
  asm volatile("" ::: "memory");
  u32x4_t wf[8];
#pragma unroll
  for (int b = 0; b < 8; ++b) wf[b] = wfrag(wreg + b * 1024, fr, g);

#pragma unroll
  for (int tt = 0; tt < NT; ++tt) {
    // even tiles past the weights, odd tiles over them (their products read
    // into wf before the first tile's barrier)
    char* xb = wreg + ((tt & 1) ? 0 : 8192);
    // every row is stored (rows past T hold the last token again and feed
    // only outputs that are never written): no branch, so each store waits
    // for its own load only
#pragma unroll
    for (int i = 0; i < NS; ++i) {
      const int pc = i * 64 + lane, rr = pc / PR, c = pc % PR;
      st16(xb + rr * 512 + ((c ^ xsw<512>(rr)) << 4), v[tt][i]);
    }
    __builtin_amdgcn_s_waitcnt(0xC07F);               // lgkmcnt(0): this wave's rows are in LDS
    asm volatile("" ::: "memory");
    f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int b = 0; b < 8; ++b) acc = Mma<bf16_t>::run1(xfrag<512>(xb, fr, 4 * b + g), wf[b], acc);
    // acc[i]: token row 4g + i of the tile, weight row fr
    float* pw = part[tt & 1][wave];
#pragma unroll
    for (int i = 0; i < 4; ++i) pw[(4 * g + i) * 17 + fr] = acc[i];
    __syncthreads();
    const float* pt = part[tt & 1][0];
    if (is_sh) {
      const int t = tt * 16 + tid;
      if (tid < 16 && t < T) {
        float h[8];
#pragma unroll
        for (int c = 0; c < 8; ++c)
          h[c] = siluf_(sum4(pt + tid * 17 + c, 16 * 17)) * sum4(pt + tid * 17 + 8 + c, 16 * 17);
        st16(p.Hs + (long long)t * FS + blk * 8, pack8(h));
      }
    } else {
      const int et = blk - n_sh;
      const int t = tid >> 4, c = tid & 15, e = et * 16 + c;
      const float b = e < p.E ? bias_c : 0.f;
      const float sc = 1.0f / (1.0f + expf(-sum4(pt + t * 17 + c, 16 * 17)));
      uint64_t key = e < p.E ? (((uint64_t)float_key(sc + b) << 32) | (uint32_t)(63 - e)) : 0ull;
      float ks = sc;
#pragma unroll
      for (int off = 1; off < 16; off <<= 1) {
        const uint32_t lo = __shfl_xor((uint32_t)key, off), hi = __shfl_xor((uint32_t)(key >> 32), off);
        const float os = __shfl_xor(ks, off);
        const uint64_t o = ((uint64_t)hi << 32) | lo;
        if (o > key) {
          key = o;
          ks = os;
        }
      }
      if (c == 0 && tt * 16 + t < T) {
        p.rkey[et * 64 + tt * 16 + t] = key;
        p.rscore[et * 64 + tt * 16 + t] = ks;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Top-1 dispatch bookkeeping for T <= 64 tokens from the router's tile keys:
// each token's expert (largest of its 4 tile keys) and s, loads, offsets,
// the stable dispatch order (slots of an expert ascend in t) and the
// ascending list of experts with a load.  Computed by every stage-2
// workgroup that needs it (a few hundred cycles), so no launch is spent on
// it.
// ---------------------------------------------------------------------------
struct Book {
  unsigned long long mask[64];   // tokens of each expert, one bit per token
  int idx[64], off[64], perm[64], pos[64];
  int act_e[64], act_s0[64], act_n[64];
  float sc[64];
  int n_active;
};

__device__ void decode_book(const DecodeArgs& p, Book& B) {
  const int tid = threadIdx.x, T = p.T;
  int e = -1;
  if (tid < 64) {
    // the first wave alone loads the keys (entries past T are stale and not
    // used); they are consumed inside this branch, so only this wave waits
    uint64_t k[4];
    float s[4];
#pragma unroll
    for (int et = 0; et < 4; ++et) {
      k[et] = p.rkey[et * 64 + tid];
      s[et] = p.rscore[et * 64 + tid];
    }
    uint64_t kb = k[0];
    float sc = s[0];
#pragma unroll
    for (int et = 1; et < 4; ++et)
      if (k[et] > kb) {
        kb = k[et];
        sc = s[et];
      }
    if (tid < T) e = min(63 - (int)(uint32_t)kb, p.E - 1);   // a NaN score can leave every key 0; keep idx in range
    B.mask[tid] = 0ull;
    B.idx[tid] = e;
    B.sc[tid] = sc;
  }
  __syncthreads();
  if (tid < T) atomicOr(&B.mask[e], 1ull << tid);
  __syncthreads();
  if (tid < 64) {
    const int c = __popcll(B.mask[tid]);
    int incl = c;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int v = __shfl_up(incl, o);
      if (tid >= o) incl += v;
    }
    B.off[tid] = incl - c;
    const unsigned long long m = __ballot(c > 0);
    const int r = __popcll(m & ((1ull << tid) - 1ull));
    if (c > 0) {
      B.act_e[r] = tid;
      B.act_s0[r] = incl - c;
      B.act_n[r] = c;
    }
    if (tid == 0) B.n_active = __popcll(m);
  }
  __syncthreads();
  if (tid < T) {
    const int slot = B.off[e] + __popcll(B.mask[e] & ((1ull << tid) - 1ull));
    B.perm[slot] = tid;
    B.pos[tid] = slot;
  }
  __syncthreads();
}

// The routing outputs of the call (stage 3 reads perm and the active list).
__device__ void decode_write_routing(const DecodeArgs& p, const Book& B) {
  const int tid = threadIdx.x;
  if (tid < p.T) {
    p.idx[tid] = B.idx[tid];
    p.gate[tid] = B.sc[tid] / B.sc[tid];
    p.perm[tid] = B.perm[tid];
    p.pos[tid] = B.pos[tid];
  }
  if (tid < p.E) {
    p.counts[tid] = __popcll(B.mask[tid]);
    p.offsets[tid] = B.off[tid];
  }
  if (tid == p.E - 1) p.offsets[p.E] = B.off[tid] + __popcll(B.mask[tid]);
  if (tid < B.n_active) {
    p.active[3 * tid] = B.act_e[tid];
    p.active[3 * tid + 1] = B.act_s0[tid];
    p.active[3 * tid + 2] = B.act_n[tid];
  }
  if (tid == 0) *p.n_active = B.n_active;
}

// Prefetch of the next layer's router and shared gate/up (DecodeArgs::pf_*),
// by workgroups past stage 3's items.  Mirror m reads the 16 weight rows that
// the next layer's stage-1 workgroup m reads (shared gate/up rows 8m .. + 7
// and Fs + 8m .. + 7, or router rows 16 (m - Fs / 8) .. + 15).  Workgroup b
// of a launch runs on XCD b mod 8 and the mirror's index is m past a
// multiple of 8, so its rows land in the L2 of the XCD that reads them next
// (measured: a mirror one XCD off makes the next layer slower than none).
// The loads go to LDS and are never read.
template <int D, int FS>
__device__ void decode_prefetch(const DecodeArgs& p, int m, char* lds) {
  if (m >= FS / 8 + 4) return;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  char* dst = lds + wave * 1024;
  static_assert(D * 2 % 1024 == 0, "whole 1 KiB pieces of a row");
#pragma unroll
  for (int i = 0; i < 4; ++i) {                      // wave w: rows 4w .. 4w + 3
    const int r = 4 * wave + i;
    const char* row;
    if (m < FS / 8) {
      const int f = m * 8 + (r & 7);
      row = reinterpret_cast<const char*>(p.pf_sh_gate_up + (long long)(r < 8 ? f : FS + f) * D);
    } else {
      row = reinterpret_cast<const char*>(p.pf_router + (long long)min((m - FS / 8) * 16 + r, p.E - 1) * D);
    }
#pragma unroll
    for (int q = 0; q < D * 2 / 1024; ++q)
      __builtin_amdgcn_global_load_lds(row + q * 1024 + lane * 16, (lds_ptr_t)dst, 16, 0, 0);
  }
  __builtin_amdgcn_s_waitcnt(0);                     // every load has landed before the wave ends
}

// ---------------------------------------------------------------------------
// Stage 2.  Operands go to the MFMAs straight from global memory: these
// workgroups are bound by the latency of their two dependent round trips
// (bookkeeping, then operands), not by the address units, and the LDS
// staging of stage 1 cost them occupancy (measured).
//   shared down item (j, tt): output columns 16 (j / 4) .. + 15, contraction
//     quarter j % 4 of Fs, tokens 16 tt .. + 15; wave w takes a quarter of
//     that quarter (128 elements, 4 MFMA steps).  The partial tiles are added
//     in a fixed order and written as fp32 part_sh[quarter][slot][n], in
//     dispatch (slot) order so that stage 3 reads one expert's rows
//     contiguously.
//   routed gate/up item i: active expert a = i / (F/16), h columns 16 fb ..
//     + 15 (fb = i % (F/16)) over that expert's tokens: a gate tile (rows
//     16 fb + r) and an up tile (rows F + 16 fb + r).  Wave w takes
//     contraction quarter w (two scale groups).  A lane's 16-byte weight
//     load holds 32 consecutive nibbles of one group; its 4 words feed 4
//     MFMAs with the matching 8-element pieces of x.  h = silu(gate) * up.
// Rows past a tile's tokens re-read its last token (loads under a lane
// condition would be waited for at the end of their branch) and are not
// stored.
// ---------------------------------------------------------------------------
template <int D, int FS, int NT>
__device__ void decode_shared_down(const DecodeArgs& p, int j, int tt0, float* lds, Book& B) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int fr = lane & 15, g = lane >> 4;
  constexpr int J = FS / 16 / 32;                    // MFMA K-steps per wave (4)
  const int cb = j >> 2, quarter = j & 3, T = p.T;
  const int kofs = quarter * (FS / 2) + wave * (FS / 8) + g * 16;   // bytes into a row
  const char* wr = reinterpret_cast<const char*>(p.w_sh_down + (long long)(cb * 16 + fr) * FS) + kofs;
  u32x4_t wv[J], ha[NT][J];
#pragma unroll
  for (int i = 0; i < J; ++i) wv[i] = ld16(wr + i * 64);
#pragma unroll
  for (int tt = 0; tt < NT; ++tt) {
    const char* hr = reinterpret_cast<const char*>(p.Hs + (long long)min((tt0 + tt) * 16 + fr, T - 1) * FS) + kofs;
#pragma unroll
    for (int i = 0; i < J; ++i) ha[tt][i] = ld16(hr + i * 64);
  }
  // partial tiles: lds[token tile][wave][16][17]
#pragma unroll
  for (int tt = 0; tt < NT; ++tt) {
    f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < J; ++i) acc = Mma<bf16_t>::run1(ha[tt][i], wv[i], acc);
#pragma unroll
    for (int i = 0; i < 4; ++i) lds[((tt * 4 + wave) * 16 + 4 * g + i) * 17 + fr] = acc[i];
  }
  decode_book(p, B);                                 // its loads follow the operand loads; it ends with a barrier
  const int tt = tid >> 6, m = (tid >> 2) & 15, c4 = (tid & 3) * 4, t = (tt0 + tt) * 16 + m;
  if (tt < NT && t < T) {
    const float* q = lds + (tt * 4 * 16 + m) * 17 + c4;
    f32x4_t v;
#pragma unroll
    for (int c = 0; c < 4; ++c) v[c] = sum4(q + c, 16 * 17);
    *reinterpret_cast<f32x4_t*>(p.part_sh + ((long long)quarter * T + B.pos[t]) * D + cb * 16 + c4) = v;
  }
}

// Where expert e's int4 weights sit: its own index, or with expert
// streaming the slot the cache gave it (clamped, so a stale table cannot
// address outside the slots).
__device__ __forceinline__ int weight_slot(const DecodeArgs& p, int e) {
  if (!p.slot) return e;
  const int s = p.slot[e];
  return s < 0 ? 0 : (s >= p.n_slots ? p.n_slots - 1 : s);
}

template <int D, int FR, int FBN>
__device__ void decode_routed_gate_up(const DecodeArgs& p, int item, float* lds, Book& B) {
  decode_book(p, B);
  constexpr int nfb = FR / 16 / FBN;                 // items per active expert
  const int a = item / nfb, fb0 = (item - a * nfb) * FBN;
  if (a >= B.n_active) return;                       // uniform over the workgroup
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int fr = lane & 15, g = lane >> 4;
  const int e = B.act_e[a], s0 = B.act_s0[a], n = B.act_n[a];
  const int qofs = wave * (D / 8) + g * 16;          // bytes into a packed row
  u32x4_t wg[FBN][2], wu[FBN][2];
  uint32_t sg[FBN], su[FBN];
#pragma unroll
  for (int f = 0; f < FBN; ++f) {
    const long long rg = (long long)weight_slot(p, e) * 2 * FR + (fb0 + f) * 16 + fr, ru = rg + FR;
#pragma unroll
    for (int grp = 0; grp < 2; ++grp) {
      wg[f][grp] = ld16(p.q_gate_up + rg * (D / 2) + qofs + grp * 64);
      wu[f][grp] = ld16(p.q_gate_up + ru * (D / 2) + qofs + grp * 64);
    }
    sg[f] = *reinterpret_cast<const uint32_t*>(p.s_gate_up + rg * (D / kGroup) + wave * 2);
    su[f] = *reinterpret_cast<const uint32_t*>(p.s_gate_up + ru * (D / kGroup) + wave * 2);
  }
  for (int m0 = 0; m0 < n; m0 += 16) {
    const int nt = min(16, n - m0);
    const int tok = B.perm[s0 + m0 + min(fr, nt - 1)];
    const uint16_t* xsrc = p.gamma ? p.xn : p.x;     // the MoE block: the rows stage 1 normalised
    const char* xr = reinterpret_cast<const char*>(xsrc + (long long)tok * D) + wave * (D / 2) + g * 64;
    u32x4_t xa[2][4];
#pragma unroll
    for (int grp = 0; grp < 2; ++grp)
#pragma unroll
      for (int j = 0; j < 4; ++j) xa[grp][j] = ld16(xr + grp * 256 + j * 16);
#pragma unroll
    for (int f = 0; f < FBN; ++f) {
      f32x4_t ag = {0.f, 0.f, 0.f, 0.f}, au = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int grp = 0; grp < 2; ++grp) {
        f32x4_t tg = {0.f, 0.f, 0.f, 0.f}, tu = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          tg = Mma<bf16_t>::run1(xa[grp][j], int4x8_to_bf16(wg[f][grp][j]), tg);
          tu = Mma<bf16_t>::run1(xa[grp][j], int4x8_to_bf16(wu[f][grp][j]), tu);
        }
        const float scg = bf16_to_f32((bf16_t)(grp ? sg[f] >> 16 : sg[f] & 0xFFFFu));
        const float scu = bf16_to_f32((bf16_t)(grp ? su[f] >> 16 : su[f] & 0xFFFFu));
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          ag[i] += tg[i] * scg;
          au[i] += tu[i] * scu;
        }
      }
      // lds: [column block][wave][token][column], row stride 33 (gate columns 0-15, up 16-31)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        lds[((f * 4 + wave) * 16 + 4 * g + i) * 33 + fr] = ag[i];
        lds[((f * 4 + wave) * 16 + 4 * g + i) * 33 + 16 + fr] = au[i];
      }
    }
    __syncthreads();
    if (tid < 2 * nt * FBN) {
      const int f = tid / (2 * nt), r = tid - f * 2 * nt, m = r >> 1, c8 = (r & 1) * 8;
      const float* q = lds + (f * 4 * 16 + m) * 33 + c8;
      float h[8];
#pragma unroll
      for (int c = 0; c < 8; ++c) h[c] = siluf_(sum4(q + c, 16 * 33)) * sum4(q + 16 + c, 16 * 33);
      st16(p.H + (long long)(s0 + m0 + m) * FR + (fb0 + f) * 16 + c8, pack8(h));
    }
    __syncthreads();                                 // before the next tile reuses the partials
  }
}

// Block 0 writes the routing (and takes the bias step of
// moe_forward_bias_step); then the shared down; then the routed gate/up
// (items of experts past the active count exit after the bookkeeping).
// NT = 1: one shared-down item per weight block and token tile (256 x the
// token tiles).  Above 16 tokens (NT = 2 or 4) a shared-down item takes
// every token tile of its weight block (the weights are read once), so that
// fewer rounds of the workgroups a CU holds at once (four, by registers)
// cover the grid: at 64 tokens 2305 workgroups became 1537.  FBN = 2 (32 h
// columns per routed item) would halve the routed items but needs more than
// the 128 registers of four waves per SIMD (it spilled).
template <int D, int FR, int FS, int NT, int FBN>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(4))) void decode_stage2_kernel(DecodeArgs p, int ntile) {
  constexpr int kSd = NT * 4 * 16 * 17, kGu = FBN * 4 * 16 * 33;
  __shared__ float lds[kSd > kGu ? kSd : kGu];
  __shared__ Book B;
  const int n_sd = NT == 1 ? 4 * (D / 16) * ntile : 4 * (D / 16);
  const int blk = blockIdx.x;
  if (blk == 0) {
    decode_book(p, B);
    decode_write_routing(p, B);
    // the bias step (stage 1's router was the bias's only reader)
    if (p.step_bias && threadIdx.x < 64) {
      const int e = threadIdx.x;
      bias_step_wave(e, p.E, (long long)p.T * p.k, e < p.E ? (int)__popcll(B.mask[e]) : 0, p.step_gamma,
                     p.step_bias, p.step_stats);
    }
  } else if (blk <= n_sd) {
    if constexpr (NT == 1) {
      int j, tt;
      xcd_item(blk - 1, ntile, j, tt);
      decode_shared_down<D, FS, 1>(p, j, tt, lds, B);
    } else {
      decode_shared_down<D, FS, NT>(p, blk - 1, 0, lds, B);
    }
  } else {
    decode_routed_gate_up<D, FR, FBN>(p, blk - 1 - n_sd, lds, B);
  }
}

// ---------------------------------------------------------------------------
// Stage 3, routed down + combine: item i takes active expert a = i / (D/32)
// and output columns 32 cb .. 32 cb + 31 (cb = i % (D/32)), two 16-row
// tiles; wave w takes scale group w of the contraction F.  For each of the
// expert's tokens t (slot s): y[t] = (((sh0 + sh1) + sh2) + sh3)[s] + o
// (+ resid[t] in the MoE block), rounded once, where sh_q are the shared-down
// partials and o the routed row (top-1: gate 1).  Every token belongs to exactly one active expert, so
// every y row is written once.  Operands come straight from global memory
// (as in stage 2).
// ---------------------------------------------------------------------------
template <int D, int FR, int CBN>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(CBN == 1 ? 4 : 3))) void decode_stage3_kernel(DecodeArgs p, int n_items) {
  constexpr int W = 32 * CBN, LS = W + 1;            // output columns per item, LDS row stride
  __shared__ __align__(16) float lds[4 * 16 * LS];
  static_assert(4 * 16 * LS * 4 >= 4 * 1024, "a 1 KiB prefetch target per wave");
  if ((int)blockIdx.x >= n_items) {
    decode_prefetch<D, kDecodeFs>(p, blockIdx.x - n_items, reinterpret_cast<char*>(lds));
    return;
  }
  static_assert(FR / kGroup == 4, "one scale group per wave");
  constexpr int ncb = D / W, NTL = W / 16, TPT = W / 8;   // 16-column tiles, threads per token
  const int a = blockIdx.x / ncb, cb = blockIdx.x - a * ncb;
  // the active entry is read together with the count; a < E keeps it in bounds
  const int na = *p.n_active;
  const int e = min(max(p.active[3 * a], 0), p.E - 1), s0 = p.active[3 * a + 1], n = p.active[3 * a + 2];
  if (a >= na) return;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int fr = lane & 15, g = lane >> 4;
  u32x4_t wq[NTL];
  float sc[NTL];
#pragma unroll
  for (int tile = 0; tile < NTL; ++tile) {
    const long long r = (long long)weight_slot(p, e) * D + cb * W + tile * 16 + fr;
    wq[tile] = ld16(p.q_down + r * (FR / 2) + wave * 64 + g * 16);
    sc[tile] = bf16_to_f32(p.s_down[r * (FR / kGroup) + wave]);
  }
  const long long q1 = (long long)p.T * D;
  for (int m0 = 0; m0 < n; m0 += 16) {
    const int nt = min(16, n - m0);
    const char* hr = reinterpret_cast<const char*>(p.H + (long long)(s0 + m0 + min(fr, nt - 1)) * FR) + wave * 256 + g * 64;
    u32x4_t ha[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) ha[j] = ld16(hr + j * 16);
    // combine operands of this thread's output piece (TPT nt <= 16 TPT
    // threads, the first CBN waves), requested after the operands, before
    // the products
    const bool out = tid < TPT * nt;
    const int m = tid / TPT, c8 = (tid - m * TPT) * 8;
    int tok = 0;
    f32x4_t sh[4][2];
    u32x4_t rs = {0u, 0u, 0u, 0u};                   // the block's residual input (bf16), if any
    if (tid < 16 * TPT) {
      const int mc = min(m, nt - 1);
      tok = p.perm[s0 + m0 + mc];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float* src = p.part_sh + q * q1 + (long long)(s0 + m0 + mc) * D + cb * W + c8;
        sh[q][0] = *reinterpret_cast<const f32x4_t*>(src);
        sh[q][1] = *reinterpret_cast<const f32x4_t*>(src + 4);
      }
      if (p.resid) rs = ld16(p.resid + (long long)tok * D + cb * W + c8);
    }
#pragma unroll
    for (int tile = 0; tile < NTL; ++tile) {
      f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int j = 0; j < 4; ++j) acc = Mma<bf16_t>::run1(ha[j], int4x8_to_bf16(wq[tile][j]), acc);
#pragma unroll
      for (int i = 0; i < 4; ++i) lds[(wave * 16 + 4 * g + i) * LS + tile * 16 + fr] = acc[i] * sc[tile];
    }
    __syncthreads();
    if (out) {
      float v[8];
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        const float o = sum4(lds + m * LS + c8 + c, 16 * LS);
        const float s = ((sh[0][c >> 2][c & 3] + sh[1][c >> 2][c & 3]) + sh[2][c >> 2][c & 3]) + sh[3][c >> 2][c & 3];
        v[c] = s + o;
        if (p.resid) v[c] += bf16_to_f32((bf16_t)((rs[c >> 1] >> (16 * (c & 1))) & 0xFFFF));
      }
      st16(p.y + (long long)tok * D + cb * W + c8, pack8(v));
    }
    __syncthreads();                                 // before the next tile reuses the partials
  }
}

}  // namespace

bool decode_shape_supported(int d, int F, int Fs) { return d == kDecodeD && F == kDecodeF && Fs == kDecodeFs; }

void launch_decode(const DecodeArgs& a, hipStream_t s) {
  constexpr int D = kDecodeD, FR = kDecodeF, FS = kDecodeFs;
  static_assert((FS / 8) % 8 == 0 && (4 * (D / 16)) % 8 == 0, "token-tiled items need weight blocks in eights");
  const int ntile = (a.T + 15) / 16;
  if (a.T == 0) {   // only the (empty) routing outputs
    hipLaunchKernelGGL((decode_stage2_kernel<D, FR, FS, 1, 1>), dim3(1), dim3(256), 0, s, a, 0);
    return;
  }
  const int max_active = a.T * a.k < a.E ? a.T * a.k : a.E;
  if (ntile == 1)
    hipLaunchKernelGGL((decode_stage1_kernel<D, FS>), dim3(FS / 8 + 4), dim3(256), 0, s, a, 1);
  else if (ntile == 2)
    hipLaunchKernelGGL((decode_stage1_wide_kernel<D, FS, 2>), dim3(FS / 8 + 4), dim3(256), 0, s, a);
  else if (ntile == 3)
    hipLaunchKernelGGL((decode_stage1_wide_kernel<D, FS, 3>), dim3(FS / 8 + 4), dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL((decode_stage1_wide_kernel<D, FS, 4>), dim3(FS / 8 + 4), dim3(256), 0, s, a);
  // stage 2 and 3 grids sized to one round of resident workgroups (see the kernels)
  if (ntile == 1) {
    hipLaunchKernelGGL((decode_stage2_kernel<D, FR, FS, 1, 1>), dim3(1 + 4 * (D / 16) + max_active * (FR / 16)),
                       dim3(256), 0, s, a, ntile);
  } else if (ntile == 2) {
    hipLaunchKernelGGL((decode_stage2_kernel<D, FR, FS, 2, 1>), dim3(1 + 4 * (D / 16) + max_active * (FR / 16)),
                       dim3(256), 0, s, a, ntile);
  } else {
    hipLaunchKernelGGL((decode_stage2_kernel<D, FR, FS, 4, 1>), dim3(1 + 4 * (D / 16) + max_active * (FR / 16)),
                       dim3(256), 0, s, a, ntile);
  }
  // stage 3's items, then (with a next layer) the prefetch mirrors of its
  // stage-1 workgroups; the item count is a multiple of 8, so each mirror
  // keeps its workgroup's XCD.  (Mirrors of the next stage 2's shared-down
  // reads, in this stage or in stage 2, measured no gain: those workgroups
  // are not on the critical path.)
  const int n_pf = a.pf_router && a.pf_sh_gate_up ? FS / 8 + 4 : 0;
  if (a.T <= 32) {
    const int n3 = max_active * (D / 32);
    hipLaunchKernelGGL((decode_stage3_kernel<D, FR, 1>), dim3(n3 + n_pf), dim3(256), 0, s, a, n3);
  } else {
    const int n3 = max_active * (D / 64);
    hipLaunchKernelGGL((decode_stage3_kernel<D, FR, 2>), dim3(n3 + n_pf), dim3(256), 0, s, a, n3);
  }
}

}  // namespace fgmoe
