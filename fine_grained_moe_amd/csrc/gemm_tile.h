// Pieces shared by the two MFMA GEMM kernels (gemm.hip: 128 x 256 tiles, two
// workgroups per CU; gemm_fwd.hip: 256 x 256 tiles, one workgroup per CU).
#pragma once

#include "common.h"
#include "kernels.h"

namespace fgmoe {

typedef __attribute__((address_space(3))) void* lds_ptr_t;

// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding:
// vmcnt bits [3:0] and [15:14], expcnt [6:4] and lgkmcnt [11:8] left at max).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// Workgroup barrier without the memory fences of __syncthreads: the direct
// LDS loads are waited for explicitly with wait_vmcnt.  The empty asm keeps
// the compiler from moving memory accesses across it.
__device__ __forceinline__ void block_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// LDS swizzle of the 16-byte pieces of 64-byte operand rows.  gfx950 serves a
// 16-byte-per-lane LDS read 32 lanes at a time over 128 four-byte banks
// (fitted to measured SQ_LDS_BANK_CONFLICT counts of probe access patterns).
// An MFMA operand read has 16 consecutive rows x 2 piece indices per
// half-wave; this XOR makes those 32 pieces hit 32 distinct bank groups.
constexpr int kRowB = 64;
__device__ __forceinline__ int swz_piece(int row, int piece) { return piece ^ (((row >> 3) & 1) << 1); }
__device__ __forceinline__ int swz(int row, int piece) { return row * kRowB + (swz_piece(row, piece) << 4); }

// N consecutive outputs (N = 1, 2, 4 or 8), rounded to T.
template <typename T, int N>
__device__ __forceinline__ void store_vec(T* p, const float (&v)[N]) {
  if constexpr (N == 1) {
    if constexpr (sizeof(T) == 2) *reinterpret_cast<uint16_t*>(p) = f32_to_bf16(v[0]);
    else *reinterpret_cast<float*>(p) = v[0];
  } else if constexpr (sizeof(T) == 2) {
    uint32_t w[N / 2];
#pragma unroll
    for (int i = 0; i < N; i += 2)
      w[i / 2] = pack_bf16x2(v[i], v[i + 1]);
    if constexpr (N == 2) *reinterpret_cast<uint32_t*>(p) = w[0];
    else if constexpr (N == 4) *reinterpret_cast<uint2*>(p) = make_uint2(w[0], w[1]);
    else *reinterpret_cast<uint4*>(p) = make_uint4(w[0], w[1], w[2], w[3]);
  } else if constexpr (N == 2) {
    *reinterpret_cast<float2*>(p) = make_float2(v[0], v[1]);
  } else {
#pragma unroll
    for (int i = 0; i < N; i += 4)
      *reinterpret_cast<float4*>(p + i) = make_float4(v[i], v[i + 1], v[i + 2], v[i + 3]);
  }
}

// N consecutive values (N = 4 or 8) of T, widened to float.
template <typename T, int N>
__device__ __forceinline__ void load_vec(const T* p, float (&v)[N]) {
  if constexpr (sizeof(T) == 2) {
#pragma unroll
    for (int i = 0; i < N; i += 4) {
      const uint2 w = *reinterpret_cast<const uint2*>(p + i);
      v[i] = bf16_to_f32((bf16_t)(w.x & 0xFFFF));
      v[i + 1] = bf16_to_f32((bf16_t)(w.x >> 16));
      v[i + 2] = bf16_to_f32((bf16_t)(w.y & 0xFFFF));
      v[i + 3] = bf16_to_f32((bf16_t)(w.y >> 16));
    }
  } else {
#pragma unroll
    for (int i = 0; i < N; i += 4) {
      const float4 w = *reinterpret_cast<const float4*>(p + i);
      v[i] = w.x;
      v[i + 1] = w.y;
      v[i + 2] = w.z;
      v[i + 3] = w.w;
    }
  }
}

// Which job of a two-job launch block `blk` serves, and its block index
// inside that job.  Chunks of 8 blocks (one per XCD) either alternate between
// the jobs while both have chunks left, or come job by job (the hardware
// starts blocks in index order, so the job whose tiles take longest goes
// first).
__device__ __forceinline__ void select_job(const GemmArgs& args, int blk, int& jid, int& bid) {
  const int chunk = blk >> 3;
  const int c0 = args.chunks[0], c1 = args.njobs > 1 ? args.chunks[1] : 0;
  int jc;
  if (args.njobs > 1 && args.order != 0) {
    const int f = args.order - 1, cf = f ? c1 : c0;
    jid = chunk < cf ? f : 1 - f;
    jc = chunk < cf ? chunk : chunk - cf;
  } else {
    const int both = c0 < c1 ? c0 : c1;
    if (chunk < 2 * both) {
      jid = chunk & 1;
      jc = chunk >> 1;
    } else {
      jid = c0 > c1 ? 0 : 1;
      jc = both + (chunk - 2 * both);
    }
  }
  bid = jc * 8 + (blk & 7);
}

}  // namespace fgmoe
