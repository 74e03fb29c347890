// int4 export: bf16 or fp32 expert weights -> the int4 container of the
// serving path.  The article (opening section, proof-of-loop paragraph) says
// only that the containers are int4; the format is this library's reading:
// symmetric groups of 128 consecutive elements of a row, scale = absmax / 7
// rounded once to bf16, q = clamp(rne(w / scale), -8, 7) as a two's-complement
// nibble, element 2i of a row in the low nibble of byte i.
//
// The decisions that turn floating point into integers (the scale's rounding
// and each q) are exact: the scale rounds the float64 quotient absmax / 7
// once, and each q is the round-half-even of w / scale, found from an fp32
// guess and an exact residual (quant_one).
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

// q = clamp(rne(w / scale), -8, 7) without a division per element: the
// guess t = rne(w * fl32(1 / scale)) in fp32 errs by at most one step (its
// quotient errs by ~2^-20 absolute), and the exact residual w - t * scale
// (t * scale has 12 significant bits, exact in fp32; the difference is exact
// in fp64) decides: more than half a scale away moves t one step, exactly
// half is a tie and goes to the even neighbour.
__device__ __forceinline__ int quant_one(float w, float scale, float inv) {
  if (scale == 0.f) return 0;                              // all-zero group
  int q = (int)rintf(w * inv);
  const double d = (double)w - (double)((float)q * scale);
  const double ad = fabs(d), half = 0.5 * (double)scale;
  if (ad > half || (ad == half && (q & 1))) q += d > 0.0 ? 1 : -1;
  return q < -8 ? -8 : (q > 7 ? 7 : q);
}

// Sixteen lanes per group: lane l of a wave holds elements 8 (l % 16) ..
// 8 (l % 16) + 7 of group l / 16 of the wave's four (one 16-byte load of bf16,
// two of fp32), reduces the absmax over its sixteen lanes, and writes the
// group's 64 packed bytes as one 4-byte store per lane; lane 0 of each group
// writes its scale.  Waves stride over the groups.  (Measured on gfx950 at
// about 2.9 TB/s over a layer's routed weights; four sets loaded ahead per
// wave measured no faster.  The export runs once per model.)
template <typename T>
__global__ __launch_bounds__(256) void quant_int4_kernel(const T* __restrict__ w, long long groups,
                                                         uint8_t* __restrict__ packed,
                                                         uint16_t* __restrict__ scales) {
  const int lane = threadIdx.x & 63, sub = lane & 15;
  const long long nwaves = (long long)gridDim.x * 4;
  for (long long wv = (long long)blockIdx.x * 4 + (threadIdx.x >> 6); wv * 4 < groups; wv += nwaves) {
    const long long grp = wv * 4 + (lane >> 4);
    const bool live = grp < groups;                      // lanes past the last group keep the shuffles whole
    const long long e0 = (live ? grp : 0) * kGroup + 8 * sub;
    float v[8];
    if constexpr (sizeof(T) == 2) {
      const uint4 r = *reinterpret_cast<const uint4*>(w + e0);
      const uint32_t h[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        v[2 * i] = bf16_to_f32((bf16_t)(h[i] & 0xFFFFu));
        v[2 * i + 1] = bf16_to_f32((bf16_t)(h[i] >> 16));
      }
    } else {
      const float4 r0 = *reinterpret_cast<const float4*>(w + e0);
      const float4 r1 = *reinterpret_cast<const float4*>(w + e0 + 4);
      v[0] = r0.x; v[1] = r0.y; v[2] = r0.z; v[3] = r0.w;
      v[4] = r1.x; v[5] = r1.y; v[6] = r1.z; v[7] = r1.w;
    }
    float a = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) a = fmaxf(a, fabsf(v[i]));
#pragma unroll
    for (int off = 8; off >= 1; off >>= 1) a = fmaxf(a, __shfl_xor(a, off));
    // at most 8 significant bits: exact as a float, whose upper half is the bf16
    const float scale = a > 0.f ? (float)round_to_8_bits((double)a / 7.0) : 0.f;
    const float inv = scale > 0.f ? 1.f / scale : 0.f;
    uint32_t word = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) word |= (uint32_t)(quant_one(v[i], scale, inv) & 0xF) << (4 * i);
    if (live) {
      *reinterpret_cast<uint32_t*>(packed + grp * (kGroup / 2) + 4 * sub) = word;
      if (sub == 0) scales[grp] = (uint16_t)(__float_as_uint(scale) >> 16);
    }
  }
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
  // four groups per wave, four waves per block
  const long long blocks = (groups + 15) / 16;
  const dim3 grid((unsigned)(blocks < 4096 ? blocks : 4096));
  if (act == 1)
    hipLaunchKernelGGL(quant_int4_kernel<bf16_t>, grid, dim3(256), 0, s, (const bf16_t*)w, groups, packed,
                       (uint16_t*)scales);
  else
    hipLaunchKernelGGL(quant_int4_kernel<float>, grid, dim3(256), 0, s, (const float*)w, groups, packed,
                       (uint16_t*)scales);
}

}  // namespace fgmoe
