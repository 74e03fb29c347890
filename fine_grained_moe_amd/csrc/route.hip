// Router, dispatch bookkeeping and the bias step of the MoE layer (gfx950).
//
// Source: seventnews, "A relay race of rented GPUs trained NanoColibri's 2.7B
// MoE for $200", opening section, architecture paragraph: a sigmoid-plus-bias
// router over 64 experts with top-2 routing, and the per-layer expert bias
// nudged by gamma * sign(target - load) (DeepSeek-V3 recipe).
#include "common.h"
#include "kernels.h"

namespace fgmoe {

// ---------------------------------------------------------------------------
// Router logits + sigmoid + bias + wave-level top-k + gates + block histogram.
//
// A workgroup owns 16 tokens; wave w computes their logits for experts
// 16w..16w+15 as one 16x16 MFMA tile, accumulated over d in 128-byte chunks
// read straight from HBM (x) and L2 (the 128 KiB router matrix).  The tile
// goes through LDS so that each token's E logits sit one per lane; each wave
// then selects for 4 tokens: k rounds of a 64-lane max-reduction over
// (score + bias, 63 - expert) keys, which gives the larger key and, on an
// exact tie, the lower expert.  Gates are the selected scores divided by
// their sum.  Per-block expert counts go to block_counts (LDS integer
// atomics, so the counts are exact).
// ---------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(256) void route_topk_kernel(const T* __restrict__ x, const T* __restrict__ wr,
                                                         const float* __restrict__ bias, int T_, int d, int E,
                                                         int k, int32_t* __restrict__ idx,
                                                         float* __restrict__ gate,
                                                         int32_t* __restrict__ block_counts) {
  __shared__ float lg[16][65];
  __shared__ int hist[64];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r = lane & 15, g = lane >> 4;
  if (tid < 64) hist[tid] = 0;

  const int tok0 = blockIdx.x * kRouteTokensPerBlock;
  if (wave * 16 < E) {
    const int t = min(tok0 + r, T_ - 1);          // rows past T re-read the last token; never used
    const int e = min(wave * 16 + r, E - 1);      // columns past E likewise
    const char* xrow = reinterpret_cast<const char*>(x + (long long)t * d) + g * 32;
    const char* wrow = reinterpret_cast<const char*>(wr + (long long)e * d) + g * 32;
    f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
    const int nch = (int)((long long)d * sizeof(T) / 128);
    // four chunks in flight: chunk c + 4 is requested as chunk c is multiplied
    Frag a[4], b[4];
    auto load = [&](int c, Frag& fa, Frag& fb) {
      fa.lo = ld16(xrow + c * 128);
      fa.hi = ld16(xrow + c * 128 + 16);
      fb.lo = ld16(wrow + c * 128);
      fb.hi = ld16(wrow + c * 128 + 16);
    };
#pragma unroll
    for (int j = 0; j < 4; ++j)
      if (j < nch) load(j, a[j], b[j]);
    for (int c = 0; c < nch; c += 4) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if (c + j < nch) {
          acc = Mma<T>::run(a[j], b[j], acc);
          if (c + j + 4 < nch) load(c + j + 4, a[j], b[j]);
        }
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) lg[4 * g + i][wave * 16 + r] = acc[i];
  }
  __syncthreads();

  const float b_e = lane < E ? bias[lane] : 0.f;
  for (int tt = wave * 4; tt < wave * 4 + 4; ++tt) {
    const int tok = tok0 + tt;
    if (tok >= T_) break;
    const float l = lane < E ? lg[tt][lane] : 0.f;
    const float s = 1.0f / (1.0f + expf(-l));
    const float v = s + b_e;
    bool taken = lane >= E;
    int esel[8];
    float ssel[8];
    float ssum = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if (j >= k) break;
      uint32_t hi = taken ? 0u : float_key(v);
      uint32_t lo = taken ? 0u : (uint32_t)(63 - lane);
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) {
        const uint32_t ohi = __shfl_xor(hi, off);
        const uint32_t olo = __shfl_xor(lo, off);
        const bool take = (ohi > hi) || (ohi == hi && olo > lo);
        hi = take ? ohi : hi;
        lo = take ? olo : lo;
      }
      const int w = 63 - (int)lo;
      const float sw = __shfl(s, w);
      if (lane == w) taken = true;
      esel[j] = w;
      ssel[j] = sw;
      ssum += sw;
    }
    if (lane == 0) {
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        if (j >= k) break;
        idx[(long long)tok * k + j] = esel[j];
        gate[(long long)tok * k + j] = ssel[j] / ssum;
        atomicAdd(&hist[esel[j]], 1);
      }
    }
  }
  __syncthreads();
  if (tid < E) block_counts[(long long)blockIdx.x * E + tid] = hist[tid];
}

// ---------------------------------------------------------------------------
// Loads, offsets and the grouped-GEMM tile table (one workgroup of 1024).
// counts[e] = sum over routing blocks; offsets = exclusive scan over experts;
// block_base[b][e] = offsets[e] + loads of expert e in blocks before b; the
// tile table lists (expert, first row) for every kTileM rows of each expert,
// in expert order.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(1024) void route_scan_kernel(const int32_t* __restrict__ block_counts, int nblk,
                                                          int E, int32_t* __restrict__ counts,
                                                          int32_t* __restrict__ offsets,
                                                          int32_t* __restrict__ block_base,
                                                          int32_t* __restrict__ tile_e,
                                                          int32_t* __restrict__ tile_m0,
                                                          int32_t* __restrict__ tile_count) {
  __shared__ int part_sum[16][64];
  __shared__ int part_pre[16][64];
  __shared__ int off_s[64];
  const int tid = threadIdx.x, e = tid & 63, part = tid >> 6;
  const int chunk = (nblk + 15) / 16;
  const int b0 = min(nblk, part * chunk), b1 = min(nblk, b0 + chunk);
  int s = 0;
  if (e < E) {
#pragma unroll 8
    for (int b = b0; b < b1; ++b) s += block_counts[(long long)b * E + e];
  }
  part_sum[part][e] = s;
  __syncthreads();
  if (part == 0) {
    int run = 0;
    for (int p = 0; p < 16; ++p) {
      part_pre[p][e] = run;
      run += part_sum[p][e];
    }
    const int cnt = e < E ? run : 0;
    int incl = cnt;
    for (int off = 1; off < 64; off <<= 1) {
      const int o = __shfl_up(incl, off);
      if (e >= off) incl += o;
    }
    const int excl = incl - cnt;
    off_s[e] = excl;
    if (e < E) {
      counts[e] = cnt;
      offsets[e] = excl;
    }
    if (e == E - 1) offsets[E] = incl;
    const int nt = (cnt + kTileM - 1) / kTileM;
    int tincl = nt;
    for (int off = 1; off < 64; off <<= 1) {
      const int o = __shfl_up(tincl, off);
      if (e >= off) tincl += o;
    }
    const int texcl = tincl - nt;
    for (int m = 0; m < nt; ++m) {
      tile_e[texcl + m] = e;
      tile_m0[texcl + m] = m * kTileM;
    }
    if (e == 63) *tile_count = tincl;
  }
  __syncthreads();
  if (e < E) {
    int run = off_s[e] + part_pre[part][e];
#pragma unroll 8
    for (int b = b0; b < b1; ++b) {
      block_base[(long long)b * E + e] = run;
      run += block_counts[(long long)b * E + e];
    }
  }
}

// ---------------------------------------------------------------------------
// Dispatch order: slot of (t, j) = block_base[block][e] + number of earlier
// assignments of the same block to e.  Slots of an expert therefore ascend in
// t*k + j, independent of scheduling.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void route_scatter_kernel(const int32_t* __restrict__ idx,
                                                            const int32_t* __restrict__ block_base, int T_,
                                                            int E, int k, int32_t* __restrict__ perm,
                                                            int32_t* __restrict__ pos) {
  __shared__ int ids[kRouteTokensPerBlock * 8];
  const int blk = blockIdx.x;
  const long long a0 = (long long)blk * kRouteTokensPerBlock * k;
  const int nt = min(kRouteTokensPerBlock, T_ - blk * kRouteTokensPerBlock);
  const int na = nt * k;
  for (int a = threadIdx.x; a < na; a += blockDim.x) ids[a] = idx[a0 + a];
  __syncthreads();
  for (int a = threadIdx.x; a < na; a += blockDim.x) {
    const int e = ids[a];
    int rank = 0;
    for (int b = 0; b < a; ++b) rank += (ids[b] == e) ? 1 : 0;
    const int slot = block_base[(long long)blk * E + e] + rank;
    perm[slot] = (int32_t)(a0 + a);
    pos[a0 + a] = slot;
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

void launch_route_topk(int act, const void* x, const void* w_router, const float* bias, int T, int d, int E,
                       int k, int32_t* idx, float* gate, int32_t* block_counts, hipStream_t s) {
  const int nblk = route_blocks(T);
  if (nblk == 0) return;
  if (act == 1)
    hipLaunchKernelGGL(route_topk_kernel<bf16_t>, dim3(nblk), dim3(256), 0, s, (const bf16_t*)x,
                       (const bf16_t*)w_router, bias, T, d, E, k, idx, gate, block_counts);
  else
    hipLaunchKernelGGL(route_topk_kernel<float>, dim3(nblk), dim3(256), 0, s, (const float*)x,
                       (const float*)w_router, bias, T, d, E, k, idx, gate, block_counts);
}

void launch_route_scan(const int32_t* block_counts, int nblk, int E, int32_t* counts, int32_t* offsets,
                       int32_t* block_base, int32_t* tile_e, int32_t* tile_m0, int32_t* tile_count,
                       hipStream_t s) {
  hipLaunchKernelGGL(route_scan_kernel, dim3(1), dim3(1024), 0, s, block_counts, nblk, E, counts, offsets,
                     block_base, tile_e, tile_m0, tile_count);
}

void launch_route_scatter(const int32_t* idx, const int32_t* block_base, int T, int E, int k, int32_t* perm,
                          int32_t* pos, hipStream_t s) {
  const int nblk = route_blocks(T);
  if (nblk == 0) return;
  hipLaunchKernelGGL(route_scatter_kernel, dim3(nblk), dim3(128), 0, s, idx, block_base, T, E, k, perm, pos);
}

void launch_bias_update(int E, long long total, const int32_t* counts, float gamma, float* bias, hipStream_t s) {
  hipLaunchKernelGGL(bias_update_kernel, dim3(1), dim3(64), 0, s, E, total, counts, gamma, bias);
}

}  // namespace fgmoe
