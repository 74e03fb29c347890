// Weighted combine of the MoE layer (gfx950): y_t = S_t + sum_j O[pos(t, j)].
// With a contraction-split shared down, S_t arrives as nS slices added in order;
// in the MoE block the residual input h_t is added last.
//
// O rows already carry their routing weight (the routed down GEMM scaled
// them), S is the shared expert's output; the article's proof-of-loop
// paragraph (seventnews, "A relay race of rented GPUs trained NanoColibri's
// 2.7B MoE for $200", opening section) has every token use the shared expert
// plus its routed experts.  The sum runs in fp32 in a fixed order (S, then
// slice by slice, j = 0..k-1) and is rounded once, so the result does not depend on
// scheduling.  HBM-bound: each thread moves 16 bytes of every operand.
#include "common.h"
#include "kernels.h"

namespace fgmoe {

namespace {

template <typename T>
__device__ __forceinline__ void add_vec(float (&acc)[16 / sizeof(T)], const u32x4_t w) {
  if constexpr (sizeof(T) == 2) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      acc[2 * i] += bf16_to_f32((bf16_t)(w[i] & 0xFFFF));
      acc[2 * i + 1] += bf16_to_f32((bf16_t)(w[i] >> 16));
    }
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[i] += __uint_as_float(w[i]);
  }
}

template <typename T>
__global__ __launch_bounds__(256) void combine_kernel(const T* __restrict__ S, int nS, long long s_stride,
                                                      const T* __restrict__ O,
                                                      const int32_t* __restrict__ pos, int T_, int d, int k,
                                                      const T* __restrict__ resid, T* __restrict__ y) {
  constexpr int V = 16 / sizeof(T);            // elements per 16-byte vector
  const int vec_per_row = d / V;
  const long long gid = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (gid >= (long long)T_ * vec_per_row) return;
  const int t = (int)(gid / vec_per_row);
  const int c = (int)(gid - (long long)t * vec_per_row) * V;
  float acc[V];
#pragma unroll
  for (int i = 0; i < V; ++i) acc[i] = 0.f;
  for (int z = 0; z < nS; ++z) add_vec<T>(acc, ld16(S + z * s_stride + (long long)t * d + c));
  for (int j = 0; j < k; ++j) {
    const long long slot = pos[(long long)t * k + j];
    add_vec<T>(acc, ld16(O + slot * d + c));
  }
  if (resid) add_vec<T>(acc, ld16(resid + (long long)t * d + c));
  u32x4_t out;
  if constexpr (sizeof(T) == 2) {
#pragma unroll
    for (int i = 0; i < 4; ++i) out[i] = pack_bf16x2(acc[2 * i], acc[2 * i + 1]);
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) out[i] = __float_as_uint(acc[i]);
  }
  st16(y + (long long)t * d + c, out);
}

}  // namespace

void launch_combine(int act, const void* S, int nS, const void* O, const int32_t* pos, int T, int d, int k,
                    const void* resid, void* y, hipStream_t s) {
  const long long s_stride = (long long)T * d;
  const int es = act == 1 ? 2 : 4;
  const long long n = (long long)T * (d * es / 16);
  if (n == 0) return;
  const unsigned blocks = (unsigned)((n + 255) / 256);
  if (act == 1)
    hipLaunchKernelGGL(combine_kernel<bf16_t>, dim3(blocks), dim3(256), 0, s, (const bf16_t*)S, nS, s_stride, (const bf16_t*)O,
                       pos, T, d, k, (const bf16_t*)resid, (bf16_t*)y);
  else
    hipLaunchKernelGGL(combine_kernel<float>, dim3(blocks), dim3(256), 0, s, (const float*)S, nS, s_stride, (const float*)O, pos,
                       T, d, k, (const float*)resid, (float*)y);
}

}  // namespace fgmoe
