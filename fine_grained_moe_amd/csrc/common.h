// Device helpers shared by the gfx950 kernels of the MoE layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fgmoe {

typedef uint16_t bf16_t;  // bfloat16 bit pattern
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

__device__ __forceinline__ float bf16_to_f32(bf16_t b) { return __uint_as_float((uint32_t)b << 16); }

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

// Two floats -> two bfloat16 (a in the low half), round to nearest, ties to
// even: one v_cvt_pk_bf16_f32 on gfx950.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t{a, b}), bf16x2_t));
}

// float -> bfloat16, round to nearest, ties to even.
__device__ __forceinline__ bf16_t f32_to_bf16(float f) { return (bf16_t)(pack_bf16x2(f, 0.f) & 0xFFFFu); }

template <typename T> __device__ __forceinline__ float to_f32(T v);
template <> __device__ __forceinline__ float to_f32<float>(float v) { return v; }
template <> __device__ __forceinline__ float to_f32<bf16_t>(bf16_t v) { return bf16_to_f32(v); }

template <typename T> __device__ __forceinline__ T from_f32(float v);
template <> __device__ __forceinline__ float from_f32<float>(float v) { return v; }
template <> __device__ __forceinline__ bf16_t from_f32<bf16_t>(float v) { return f32_to_bf16(v); }

// Activations of the expert FFNs and the router's scores: exp2 and the
// hardware reciprocal (about 1 ulp each) instead of an IEEE divide, whose
// sequence is several times longer; the FFN results are rounded to bf16, and
// a score error of a few ulp moves no selection that is not a tie to within
// that much.
// exp(-z) overflows to +inf for very negative z, and rcp(inf) = 0.
__device__ __forceinline__ float sigmoidf_(float z) { return __builtin_amdgcn_rcpf(1.0f + __expf(-z)); }
__device__ __forceinline__ float siluf_(float z) { return z * __builtin_amdgcn_rcpf(1.0f + __expf(-z)); }

// A 32-byte slice of one operand row held by one lane: 16 bf16 or 8 float.
struct Frag {
  u32x4_t lo, hi;
};

// One lane-group slice of a 128-byte row chunk feeds the 16x16 MFMA tile.
// Each lane holds 32 contiguous bytes of its row (lane group g = lane/16 owns
// bytes [32g, 32g+32) of the chunk).  Both operands use the same mapping, so
// the products are paired correctly whatever the order of K inside a chunk.
template <typename T> struct Mma;

template <> struct Mma<bf16_t> {
  // one 16-byte piece per lane: 8 consecutive K of the lane group's slice
  static __device__ __forceinline__ f32x4_t run1(u32x4_t a, u32x4_t b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b), c,
                                                   0, 0, 0);
  }
  static __device__ __forceinline__ f32x4_t run(const Frag& a, const Frag& b, f32x4_t c) {
    c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a.lo),
                                               __builtin_bit_cast(bf16x8_t, b.lo), c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a.hi),
                                               __builtin_bit_cast(bf16x8_t, b.hi), c, 0, 0, 0);
    return c;
  }
};

template <> struct Mma<float> {
  static __device__ __forceinline__ f32x4_t run1(u32x4_t a, u32x4_t b, f32x4_t c) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a[i]), __uint_as_float(b[i]), c, 0, 0, 0);
    return c;
  }
  static __device__ __forceinline__ f32x4_t run(const Frag& a, const Frag& b, f32x4_t c) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.lo[i]), __uint_as_float(b.lo[i]), c, 0, 0, 0);
#pragma unroll
    for (int i = 0; i < 4; ++i)
      c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.hi[i]), __uint_as_float(b.hi[i]), c, 0, 0, 0);
    return c;
  }
};

__device__ __forceinline__ u32x4_t ld16(const void* p) { return *reinterpret_cast<const u32x4_t*>(p); }
__device__ __forceinline__ void st16(void* p, u32x4_t v) { *reinterpret_cast<u32x4_t*>(p) = v; }

// Order-preserving map of a float to an unsigned key (larger float -> larger key).
__device__ __forceinline__ uint32_t float_key(float v) {
  uint32_t u = __float_as_uint(v);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

}  // namespace fgmoe
