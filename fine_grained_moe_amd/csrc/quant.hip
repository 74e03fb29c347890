// int4 export: bf16 or fp32 expert weights -> the int4 container of the
// serving path.  The article (opening section, proof-of-loop paragraph) says
// only that the containers are int4; the format is this library's reading:
// symmetric groups of 128 consecutive elements of a row, scale = absmax / 7
// rounded once to bf16, q = clamp(rne(w / scale), -8, 7) as a two's-complement
// nibble, element 2i of a row in the low nibble of byte i.
//
// The decisions that turn floating point into integers (the scale's rounding
// and each q) are taken in float64 from the exact input values, so the codes
// do not depend on how the quotient would round in a narrower type.
// HBM-bound: rows * K * (input bytes + 1/2) + rows * K / 64 bytes.
#include "common.h"
#include "kernels.h"

namespace fgmoe {

namespace {

constexpr int kGroup = 128;

// A positive float64 rounded to 8 significant bits (bfloat16's precision),
// ties to even, from its own bits: one rounding.  Normal range.
__device__ __forceinline__ double round_to_8_bits(double v) {
  unsigned long long b = (unsigned long long)__double_as_longlong(v);
  constexpr unsigned long long low = (1ull << 45) - 1;   // the 45 of 52 fraction bits dropped
  b += (low >> 1) + ((b >> 45) & 1ull);
  b &= ~low;
  return __longlong_as_double((long long)b);
}

__device__ __forceinline__ int quant_one(float w, double scale) {
  if (scale == 0.0) return 0;                              // all-zero group
  const double q = rint((double)w / scale);
  return q < -8.0 ? -8 : (q > 7.0 ? 7 : (int)q);
}

// One wave per group: lane l holds elements 2l and 2l + 1 and writes their
// byte; lane 0 writes the group's scale.
template <typename T>
__global__ __launch_bounds__(256) void quant_int4_kernel(const T* __restrict__ w, long long groups,
                                                         uint8_t* __restrict__ packed,
                                                         uint16_t* __restrict__ scales) {
  const long long grp = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (grp >= groups) return;
  const int lane = threadIdx.x & 63;
  float w0, w1;
  if constexpr (sizeof(T) == 2) {
    const uint32_t two = *reinterpret_cast<const uint32_t*>(w + grp * kGroup + 2 * lane);
    w0 = bf16_to_f32((bf16_t)(two & 0xFFFFu));
    w1 = bf16_to_f32((bf16_t)(two >> 16));
  } else {
    const float2 two = *reinterpret_cast<const float2*>(w + grp * kGroup + 2 * lane);
    w0 = two.x;
    w1 = two.y;
  }
  float a = fmaxf(fabsf(w0), fabsf(w1));
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) a = fmaxf(a, __shfl_xor(a, off));
  const double scale = a > 0.f ? round_to_8_bits((double)a / 7.0) : 0.0;
  const int q0 = quant_one(w0, scale), q1 = quant_one(w1, scale);
  packed[grp * (kGroup / 2) + lane] = (uint8_t)((q0 & 0xF) | ((q1 & 0xF) << 4));
  // scale has at most 8 significant bits: exact as a float, whose upper half
  // is the bf16
  if (lane == 0) scales[grp] = (uint16_t)(__float_as_uint((float)scale) >> 16);
}

// The int4 prefill's weights: out[e] = bf16(q * scale) (q * scale is exact
// in fp32; one rounding to bf16, ties to even) for every expert with a
// nonzero load; the others are left as they are (no GEMM tile reads them).
// Thread i of expert e's grid row converts 8 consecutive elements: one
// 4-byte read of nibbles, one scale, one 16-byte write.
__global__ __launch_bounds__(256) void dequant_int4_kernel(const uint8_t* __restrict__ packed,
                                                           const uint16_t* __restrict__ scales, int rows_e, int K,
                                                           const int32_t* __restrict__ counts,
                                                           uint16_t* __restrict__ out) {
  const int e = blockIdx.y;
  if (counts[e] == 0) return;
  const long long n8 = (long long)rows_e * K / 8;
  const long long i8 = (long long)blockIdx.x * 256 + threadIdx.x;
  if (i8 >= n8) return;
  const long long base = (long long)e * rows_e * K + i8 * 8;   // element index
  const long long row = base / K;                               // row of the expert stack
  const int group = (int)((base - row * K) / kGroup);
  const float sc = bf16_to_f32(scales[row * (K / kGroup) + group]);
  const uint32_t nib = *reinterpret_cast<const uint32_t*>(packed + base / 2);
  uint32_t w[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    // byte i: element 2i in the low nibble; sign-extend each nibble
    const int lo = (int)((nib >> (8 * i)) << 28) >> 28;
    const int hi = (int)((nib >> (8 * i + 4)) << 28) >> 28;
    w[i] = pack_bf16x2((float)lo * sc, (float)hi * sc);
  }
  *reinterpret_cast<uint4*>(out + base) = make_uint4(w[0], w[1], w[2], w[3]);
}

}  // namespace

void launch_dequant_int4(const void* packed, const void* scales, int E, int rows_e, int K, const int32_t* counts,
                         void* out, hipStream_t s) {
  const long long n8 = (long long)rows_e * K / 8;
  if (E <= 0 || n8 <= 0) return;
  const dim3 grid((unsigned)((n8 + 255) / 256), (unsigned)E);
  hipLaunchKernelGGL(dequant_int4_kernel, grid, dim3(256), 0, s, (const uint8_t*)packed, (const uint16_t*)scales,
                     rows_e, K, counts, (uint16_t*)out);
}

void launch_quant_int4(int act, const void* w, long long rows, int K, uint8_t* packed, void* scales,
                       hipStream_t s) {
  const long long groups = rows * (K / kGroup);
  if (groups <= 0) return;
  const dim3 grid((unsigned)((groups + 3) / 4));
  if (act == 1)
    hipLaunchKernelGGL(quant_int4_kernel<bf16_t>, grid, dim3(256), 0, s, (const bf16_t*)w, groups, packed,
                       (uint16_t*)scales);
  else
    hipLaunchKernelGGL(quant_int4_kernel<float>, grid, dim3(256), 0, s, (const float*)w, groups, packed,
                       (uint16_t*)scales);
}

}  // namespace fgmoe
