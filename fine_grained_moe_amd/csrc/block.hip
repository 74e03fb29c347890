// Pre-norm of the MoE block (gfx950): x = bf16(h / sqrt(mean(h^2) + eps) *
// gamma) per token row.  The seventnews article "A relay race of rented GPUs
// trained NanoColibri's 2.7B MoE for $200" (opening section, architecture
// paragraph) places the MoE FFN in 23 of the model's 24 transformer layers;
// the norm in front of it and the residual add after it (done in the combine,
// combine.hip, and in the decode's last stage) are this library's reading of
// that block.
//
// One wave per row: each lane keeps its 16-byte vectors of the row in
// registers, the sum of squares runs in fp32 (lane order, then a butterfly in
// a fixed order), and the same registers are scaled and stored.  HBM-bound:
// the row is read once and x written once.
#include "common.h"
#include "kernels.h"

namespace fgmoe {

namespace {

constexpr int kNormWaves = 4;

__global__ __launch_bounds__(64 * kNormWaves) void rmsnorm_kernel(const bf16_t* __restrict__ h,
                                                                  const float* __restrict__ gamma, float eps,
                                                                  int T, int d, bf16_t* __restrict__ x) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int t = blockIdx.x * kNormWaves + wave;
  if (t >= T) return;
  const int nv = d / 8;                              // 16-byte vectors per row
  const bf16_t* row = h + (long long)t * d;
  u32x4_t v[kNormMaxVec];
  float ss = 0.f;
#pragma unroll
  for (int i = 0; i < kNormMaxVec; ++i) {
    const int c = lane + 64 * i;
    if (c < nv) {
      v[i] = ld16(row + c * 8);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float lo = bf16_to_f32((bf16_t)(v[i][j] & 0xFFFF)), hi = bf16_to_f32((bf16_t)(v[i][j] >> 16));
        ss += lo * lo;
        ss += hi * hi;
      }
    }
  }
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) ss += __shfl_xor(ss, off);
  const float rstd = 1.f / sqrtf(ss / (float)d + eps);
#pragma unroll
  for (int i = 0; i < kNormMaxVec; ++i) {
    const int c = lane + 64 * i;
    if (c < nv) {
      const float4 g0 = *reinterpret_cast<const float4*>(gamma + c * 8);
      const float4 g1 = *reinterpret_cast<const float4*>(gamma + c * 8 + 4);
      const float g[8] = {g0.x, g0.y, g0.z, g0.w, g1.x, g1.y, g1.z, g1.w};
      u32x4_t out;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float lo = bf16_to_f32((bf16_t)(v[i][j] & 0xFFFF)), hi = bf16_to_f32((bf16_t)(v[i][j] >> 16));
        out[j] = pack_bf16x2(lo * rstd * g[2 * j], hi * rstd * g[2 * j + 1]);
      }
      st16(x + (long long)t * d + c * 8, out);
    }
  }
}

}  // namespace

void launch_rmsnorm(const void* h, const float* gamma, float eps, int T, int d, void* x, hipStream_t s) {
  if (T == 0) return;
  hipLaunchKernelGGL(rmsnorm_kernel, dim3((T + kNormWaves - 1) / kNormWaves), dim3(64 * kNormWaves), 0, s,
                     (const bf16_t*)h, gamma, eps, T, d, (bf16_t*)x);
}

}  // namespace fgmoe
