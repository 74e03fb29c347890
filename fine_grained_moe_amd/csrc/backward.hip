// Backward of the MoE layer (gfx950): helper kernels around the MFMA GEMMs.
//
// Source: seventnews, "A relay race of rented GPUs trained NanoColibri's 2.7B
// MoE for $200", "Relay training" section, top-2 paragraph: with two winners
// the router receives gradient through the competition between them (with
// top-1 the routing weight is a constant and that gradient vanishes).  With
// g_j = s_j / S (S = sum of the selected sigmoid scores) the chain rule gives
//   dL/dg_j = <dy, o_j>            (o_j the expert's ungated output row)
//   dL/ds_i = (dL/dg_i - sum_j g_j dL/dg_j) / S
//   dL/dl_i = dL/ds_i * s_i (1 - s_i)       (l_i the router logit)
// and nothing flows into the bias or the unselected experts.
//
// The weight gradients contract over tokens, i.e. over the rows of the
// stored activations; they run on the same NT GEMM as the forward after the
// operands are transposed here.  (d, F and Fs are multiples of 128, so every
// row here is a whole number of 8-element vectors.)  Each expert's rows are laid out in its own
// column range padded to a multiple of 64 with zeros, so that a grouped GEMM
// with a per-expert contraction range can run over it.
#include "common.h"
#include "kernels.h"

namespace fgmoe {

namespace {

// ---------------------------------------------------------------------------
// Per-expert padded column ranges: klen[e] = roundup(count[e], 64),
// kofs = exclusive scan; pcol[c] = slot held by padded column c, or -1.
// Also the tables of the shared expert's weight gradients, whose contraction
// over Tp tokens is split into S slices of `step` columns (a multiple of 64):
// ksh[i] = i * step, ksh[S + i] = its length.  Workgroup e (of E, 256
// threads) writes expert e's padded range of pcol; workgroup 0 also the
// tables and the tail of pcol past the last range.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void bwd_prep_kernel(const int32_t* __restrict__ counts,
                                                       const int32_t* __restrict__ offsets, int E, int Pmax, int Tp,
                                                       int S, int step, int32_t* __restrict__ kofs,
                                                       int32_t* __restrict__ klen, int32_t* __restrict__ ksh,
                                                       int32_t* __restrict__ pcol, int32_t* __restrict__ krow_pad,
                                                       int32_t* __restrict__ zrow) {
  __shared__ int s_kofs[64], s_klen[64];
  const int tid = threadIdx.x, e = blockIdx.x;
  if (tid < 64) {
    const int c = tid < E ? counts[tid] : 0;
    const int kl = (c + kPadK - 1) / kPadK * kPadK;
    int incl = kl;
    for (int o = 1; o < 64; o <<= 1) {
      const int v = __shfl_up(incl, o);
      if (tid >= o) incl += v;
    }
    s_kofs[tid] = incl - kl;
    s_klen[tid] = kl;
    if (e == 0 && tid < E) {
      kofs[tid] = incl - kl;
      klen[tid] = kl;
    }
  }
  if (e == 0) {
    // K-major weight gradients: the token map's readable tail and the zero row
    if (krow_pad && tid < 32) krow_pad[tid] = 0;
    if (zrow && tid < 128) zrow[tid] = 0;
    if (tid < S) {
      ksh[tid] = tid * step;
      ksh[S + tid] = max(0, min(step, Tp - tid * step));
    }
  }
  __syncthreads();
  if (e < E) {
    const int c0 = s_kofs[e], n = counts[e], o = offsets[e], kl = s_klen[e];
    for (int i = tid; i < kl; i += blockDim.x) pcol[c0 + i] = i < n ? o + i : -1;
  }
  if (e == 0) {
    const int end = E > 0 ? s_kofs[E - 1] + s_klen[E - 1] : 0;
    for (int c = end + tid; c < Pmax; c += blockDim.x) pcol[c] = -1;
  }
}

// 8 consecutive values of T as float, and back (16 bytes for bf16, 32 for float).
template <typename T>
__device__ __forceinline__ void load8(const T* p, float (&v)[8]) {
  if constexpr (sizeof(T) == 2) {
    const u32x4_t w = ld16(p);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = bf16_to_f32((bf16_t)(w[i] & 0xFFFFu));
      v[2 * i + 1] = bf16_to_f32((bf16_t)(w[i] >> 16));
    }
  } else {
    const u32x4_t a = ld16(p), b = ld16(p + 4);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[i] = __uint_as_float(a[i]);
      v[4 + i] = __uint_as_float(b[i]);
    }
  }
}
template <typename T>
__device__ __forceinline__ void store8(T* p, const float (&v)[8]) {
  if constexpr (sizeof(T) == 2) {
    u32x4_t w;
#pragma unroll
    for (int i = 0; i < 4; ++i) w[i] = (uint32_t)f32_to_bf16(v[2 * i]) | ((uint32_t)f32_to_bf16(v[2 * i + 1]) << 16);
    st16(p, w);
  } else {
    st16(p, u32x4_t{__float_as_uint(v[0]), __float_as_uint(v[1]), __float_as_uint(v[2]), __float_as_uint(v[3])});
    st16(p + 4, u32x4_t{__float_as_uint(v[4]), __float_as_uint(v[5]), __float_as_uint(v[6]), __float_as_uint(v[7])});
  }
}

// ---------------------------------------------------------------------------
// Gather-transpose: dst[b][r][c] = scale * src[b][row(c)][r], for r < R and
// c < C, where row(c) is c (c < n_in), map1[c] (>= 0), or, with map2,
// map2[map1[c]] / div; a column without a row is zero.  The scale is
// scale[map2 ? map2[map1[c]] : map1[c]] when given.  64 x 64 tiles through
// LDS; every global access moves 8 consecutive elements (R and C are
// multiples of 8, as are the leading dimensions).
// ---------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(256) void transpose_kernel(TransposeArgs a) {
  __shared__ float tile[64][65];                     // [c][r]
  const int tid = threadIdx.x;
  const int c0 = blockIdx.x * 64, r0 = blockIdx.y * 64;
  const T* src = reinterpret_cast<const T*>(a.src) + (long long)blockIdx.z * a.src_bstride;
  T* dst = reinterpret_cast<T*>(a.dst) + (long long)blockIdx.z * a.dst_bstride;
  // load: thread (cl = tid / 8 + 32h, rq = tid % 8) reads r0 + 8rq .. +7 of column c0 + cl's source row
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int cl = (tid >> 3) + 32 * h, rq = tid & 7, c = c0 + cl, r = r0 + 8 * rq;
    float v[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    if (c < a.C && r < a.R) {
      int m = a.map1 ? a.map1[c] : (c < a.n_in ? c : -1);
      if (m >= 0) {
        int sidx = m;
        if (a.map2) {
          sidx = a.map2[m];
          m = sidx / a.div;
        }
        load8<T>(src + (long long)m * a.ld_src + r, v);
        if (a.scale) {
          const float sc = a.scale[sidx];
#pragma unroll
          for (int i = 0; i < 8; ++i) v[i] *= sc;
        }
      }
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) tile[cl][8 * rq + i] = v[i];
  }
  __syncthreads();
  // store: thread (rl = tid / 8 + 32h, cq = tid % 8) writes c0 + 8cq .. +7 of row r0 + rl
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int rl = (tid >> 3) + 32 * h, cq = tid & 7, rr = r0 + rl, c = c0 + 8 * cq;
    if (rr < a.R && c < a.C) {
      float v[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] = tile[8 * cq + i][rl];
      store8<T>(dst + (long long)rr * a.ld_dst + c, v);
    }
  }
}

// Sum of v over the wave, the same in every lane: DPP rotations by 1, 2, 4
// and 8 lanes within each 16-lane row (after them every lane holds its row's
// sum: each step adds a disjoint neighbouring range), then the four row sums
// (lanes 0, 16, 32, 48) added in row order.
__device__ __forceinline__ float wave_sum(float v) {
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x121, 0xF, 0xF, false));
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x122, 0xF, 0xF, false));
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x124, 0xF, 0xF, false));
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x128, 0xF, 0xF, false));
  const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
  const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
  const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
  const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
  return ((r0 + r1) + r2) + r3;
}

// ---------------------------------------------------------------------------
// Router and gate gradients, one wave per token: dg_j = <dy_t, o_j>; the
// selected scores are recomputed from the logits x_t . W_r[e_j]; then the
// formulas at the top of this file.  dl: [T, k] fp32.  Each lane takes two
// 8-element pieces of every row (all of its loads in flight at once).
// ---------------------------------------------------------------------------
template <typename T, int KM>
__global__ __launch_bounds__(256) void bwd_gate_kernel(const T* __restrict__ dy, const T* __restrict__ ou,
                                                       const T* __restrict__ x, const T* __restrict__ wr,
                                                       const int32_t* __restrict__ idx, const float* __restrict__ gate,
                                                       const int32_t* __restrict__ pos, int T_, int d, int k,
                                                       float* __restrict__ dl, int32_t* __restrict__ krow) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T_) return;
  // A lane's pieces of each row: elements c .. c + 7 and c + 512 .. c + 519,
  // so that every wave load reads one contiguous KiB (bf16).  A piece past d
  // re-reads the first one and counts zero.  Every load is unconditional
  // (entry j past k re-reads entry k - 1), so none sits under a branch and
  // waits at its end; the dispatch-order token map is written at the end.
  // experts and slots are non-negative: zero-extended into the 64-bit row
  // offsets, which (unlike a sign extension) takes no instruction on the
  // loaded value, so nothing waits for the loads before the rows are requested
  uint32_t e[KM], slot[KM];
  float gt[KM];
  float dga[KM], sb[KM];
#pragma unroll
  for (int j = 0; j < KM; ++j) dga[j] = sb[j] = 0.f;
  auto load_meta = [&]() {
#pragma unroll
    for (int j = 0; j < KM; ++j) {
      const long long q = (long long)t * k + min(j, k - 1);
      e[j] = (uint32_t)idx[q];
      slot[j] = (uint32_t)pos[q];
      gt[j] = gate[q];
    }
  };
  if constexpr (sizeof(T) == 2) {
    // bf16: the products are taken on the packed pairs (v_dot2c_f32_bf16: two
    // exact bf16 products added into the fp32 sum), no unpacking.  The
    // token's experts and slots are requested first, its own rows behind them
    // (the vector memory counter completes in order, so waiting for the slots
    // leaves the rows in flight), then the expert rows.
    typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;
    auto dot = [](uint32_t a, uint32_t b, float c) {
      return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a), __builtin_bit_cast(bf16x2_t, b), c,
                                             false);
    };
    const u32x4_t zero = {0u, 0u, 0u, 0u};
    auto chunk = [&](int c0, bool meta_first) {
      const int ca = c0 + lane * 8, cb = ca + 512;
      const bool va = ca < d, vb = cb < d;
      const int pa = va ? ca : 0, pb = vb ? cb : pa;
      if (meta_first) load_meta();
      __builtin_amdgcn_sched_barrier(0);
      const u32x4_t ydy0 = ld16(dy + (long long)t * d + pa), ydy1 = ld16(dy + (long long)t * d + pb);
      const u32x4_t yx0 = ld16(x + (long long)t * d + pa), yx1 = ld16(x + (long long)t * d + pb);
      __builtin_amdgcn_sched_barrier(0);
      u32x4_t yo[KM][2], yw[KM][2];
#pragma unroll
      for (int j = 0; j < KM; ++j) {
        yo[j][0] = ld16(ou + (unsigned long long)slot[j] * d + pa);
        yo[j][1] = ld16(ou + (unsigned long long)slot[j] * d + pb);
        yw[j][0] = ld16(wr + (unsigned long long)e[j] * d + pa);
        yw[j][1] = ld16(wr + (unsigned long long)e[j] * d + pb);
      }
      __builtin_amdgcn_sched_barrier(0);
      const u32x4_t ydy[2] = {va ? ydy0 : zero, vb ? ydy1 : zero}, yx[2] = {va ? yx0 : zero, vb ? yx1 : zero};
#pragma unroll
      for (int j = 0; j < KM; ++j)
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            dga[j] = dot(ydy[h][q], yo[j][h][q], dga[j]);
            sb[j] = dot(yx[h][q], yw[j][h][q], sb[j]);
          }
    };
    chunk(0, true);
    for (int c0 = 1024; c0 < d; c0 += 1024) chunk(c0, false);
  } else {
    load_meta();
    for (int c0 = 0; c0 < d; c0 += 1024) {
      const int ca = c0 + lane * 8, cb = ca + 512;
      const float ma = ca < d ? 1.f : 0.f, mb = cb < d ? 1.f : 0.f;
      const int pa = ca < d ? ca : 0, pb = cb < d ? cb : pa;
      float vdy[16], vx[16];
      load8<T>(dy + (long long)t * d + pa, *reinterpret_cast<float(*)[8]>(vdy));
      load8<T>(dy + (long long)t * d + pb, *reinterpret_cast<float(*)[8]>(vdy + 8));
      load8<T>(x + (long long)t * d + pa, *reinterpret_cast<float(*)[8]>(vx));
      load8<T>(x + (long long)t * d + pb, *reinterpret_cast<float(*)[8]>(vx + 8));
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        vdy[i] *= ma;
        vdy[8 + i] *= mb;
        vx[i] *= ma;
        vx[8 + i] *= mb;
      }
#pragma unroll
      for (int j = 0; j < KM; ++j) {
        if (j >= k) break;
        float vo[16], vw[16];
        load8<T>(ou + (unsigned long long)slot[j] * d + pa, *reinterpret_cast<float(*)[8]>(vo));
        load8<T>(ou + (unsigned long long)slot[j] * d + pb, *reinterpret_cast<float(*)[8]>(vo + 8));
        load8<T>(wr + (unsigned long long)e[j] * d + pa, *reinterpret_cast<float(*)[8]>(vw));
        load8<T>(wr + (unsigned long long)e[j] * d + pb, *reinterpret_cast<float(*)[8]>(vw + 8));
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          dga[j] += vdy[i] * vo[i];
          sb[j] += vx[i] * vw[i];
        }
      }
    }
  }
  float dg[KM], s[KM];
#pragma unroll
  for (int j = 0; j < KM; ++j) {
    if (j >= k) break;
    dg[j] = wave_sum(dga[j]);
    s[j] = 1.0f / (1.0f + expf(-wave_sum(sb[j])));
  }
  // the token of each dispatch-order row (K-major weight gradients)
#pragma unroll
  for (int j = 0; j < KM; ++j)
    if (j < k && krow && lane == j) krow[slot[j]] = t;
  if (lane == 0) {
    float S = 0.f, G = 0.f;
#pragma unroll
    for (int j = 0; j < KM; ++j) {
      if (j >= k) break;
      S += s[j];
      G += gt[j] * dg[j];
    }
#pragma unroll
    for (int j = 0; j < KM; ++j) {
      if (j >= k) break;
      dl[(long long)t * k + j] = (dg[j] - G) / S * s[j] * (1.f - s[j]);
    }
  }
}

// ---------------------------------------------------------------------------
// Router weight gradient dW_r[e][c] = sum over the slots of e of
// dl[perm[s]] * x[token][c], in two passes.  Pass 1: one workgroup per
// 64-column chunk of the padded slot layout (every chunk lies inside one
// expert's range); its two halves each sum 32 slots in slot order for every
// column, and chunk partial = half 0 + half 1.  Pass 2: dW_r[e] = the
// partials of e's chunks added in chunk order.
// ---------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(256) void bwd_dwr_chunk_kernel(const T* __restrict__ x, const float* __restrict__ dl,
                                                            const int32_t* __restrict__ perm,
                                                            const int32_t* __restrict__ pcol, int P, int d, int k,
                                                            float* __restrict__ part) {
  __shared__ int s_tok[64];
  __shared__ float s_dl[64];
  __shared__ float half1[1024];                     // half 1's sums for one block of 1024 columns
  const int tid = threadIdx.x, h = tid >> 7, co = tid & 127;
  const int ch = blockIdx.x;
  if (tid < 64) {
    const int col = ch * 64 + tid;
    const int sl = col < P ? pcol[col] : -1;
    const int a = sl >= 0 ? perm[sl] : -1;
    s_tok[tid] = a >= 0 ? a / k : -1;
    s_dl[tid] = a >= 0 ? dl[a] : 0.f;
  }
  __syncthreads();
  for (int cb = 0; cb < d; cb += 1024) {
    const int c = cb + co * 8;
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    if (c < d) {
#pragma unroll 8
      for (int i = 0; i < 32; ++i) {
        const int sl = h * 32 + i, tk = s_tok[sl];
        if (tk >= 0) {
          float v[8];
          load8<T>(x + (long long)tk * d + c, v);
          const float w = s_dl[sl];
#pragma unroll
          for (int q = 0; q < 8; ++q) acc[q] += w * v[q];
        }
      }
    }
    if (h == 1 && c < d)
#pragma unroll
      for (int q = 0; q < 8; ++q) half1[co * 8 + q] = acc[q];
    __syncthreads();
    if (h == 0 && c < d) {
      float out[8];
#pragma unroll
      for (int q = 0; q < 8; ++q) out[q] = acc[q] + half1[co * 8 + q];
      float* dst = part + (long long)ch * d + c;
      st16(dst, u32x4_t{__float_as_uint(out[0]), __float_as_uint(out[1]), __float_as_uint(out[2]), __float_as_uint(out[3])});
      st16(dst + 4, u32x4_t{__float_as_uint(out[4]), __float_as_uint(out[5]), __float_as_uint(out[6]), __float_as_uint(out[7])});
    }
    __syncthreads();
  }
}

__global__ __launch_bounds__(256) void bwd_dwr_reduce_kernel(const float* __restrict__ part,
                                                             const int32_t* __restrict__ kofs,
                                                             const int32_t* __restrict__ klen, int d,
                                                             float* __restrict__ dwr) {
  const int e = blockIdx.x;
  const int c = blockIdx.y * 256 + threadIdx.x;
  if (c >= d) return;
  const int c0 = kofs[e] / kPadK, c1 = (kofs[e] + klen[e]) / kPadK;
  float acc = 0.f;
  for (int ch = c0; ch < c1; ++ch) acc += part[(long long)ch * d + c];
  dwr[(long long)e * d + c] = acc;
}

// ---------------------------------------------------------------------------
// dx[t] = dXs[t] + sum_j dXp[pos[t, j]] + sum_j dl[t, j] W_r[idx[t, j]], in that
// order in fp32, rounded once.  Each thread takes 8 consecutive columns.
// ---------------------------------------------------------------------------
template <typename T, int KM>
__global__ __launch_bounds__(256) void bwd_dx_kernel(const T* __restrict__ dxs, const T* __restrict__ dxp,
                                                     const T* __restrict__ wr, const float* __restrict__ dl,
                                                     const int32_t* __restrict__ idx, const int32_t* __restrict__ pos,
                                                     int T_, int d, int k, T* __restrict__ dx) {
  const long long i8 = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  const int per = d / 8;
  if (i8 >= (long long)T_ * per) return;
  const int t = (int)(i8 / per), c = (int)(i8 - (long long)t * per) * 8;
  // the token's slots, experts and router-logit gradients first (k <= KM, all
  // requested at once), then every row they select
  int sl[KM], ex[KM];
  float w[KM];
#pragma unroll
  for (int j = 0; j < KM; ++j)
    if (j < k) {
      sl[j] = pos[(long long)t * k + j];
      ex[j] = idx[(long long)t * k + j];
      w[j] = dl[(long long)t * k + j];
    }
  float v[8], u[KM][8], r[KM][8];
  load8<T>(dxs + (long long)t * d + c, v);
#pragma unroll
  for (int j = 0; j < KM; ++j)
    if (j < k) {
      load8<T>(dxp + (long long)sl[j] * d + c, u[j]);
      load8<T>(wr + (long long)ex[j] * d + c, r[j]);
    }
#pragma unroll
  for (int j = 0; j < KM; ++j)
    if (j < k)
#pragma unroll
      for (int q = 0; q < 8; ++q) v[q] += u[j][q];
#pragma unroll
  for (int j = 0; j < KM; ++j)
    if (j < k)
#pragma unroll
      for (int q = 0; q < 8; ++q) v[q] += w[j] * r[j][q];
  store8<T>(dx + (long long)t * d + c, v);
}

// ---------------------------------------------------------------------------
// out[i] = part[0][i] + part[1][i] + ... + part[S-1][i], in that order (the
// contraction slices of a split weight gradient).  4 floats per thread.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void splitk_reduce_kernel(const float* __restrict__ part, long long n, int S,
                                                            float* __restrict__ out) {
  const long long i4 = ((long long)blockIdx.x * blockDim.x + threadIdx.x) * 4;
  if (i4 >= n) return;
  u32x4_t a = ld16(part + i4);
  float v[4] = {__uint_as_float(a[0]), __uint_as_float(a[1]), __uint_as_float(a[2]), __uint_as_float(a[3])};
  for (int sl = 1; sl < S; ++sl) {
    a = ld16(part + (long long)sl * n + i4);
#pragma unroll
    for (int q = 0; q < 4; ++q) v[q] += __uint_as_float(a[q]);
  }
  st16(out + i4, u32x4_t{__float_as_uint(v[0]), __float_as_uint(v[1]), __float_as_uint(v[2]), __float_as_uint(v[3])});
}

__global__ void fill_zero_kernel(uint32_t* __restrict__ p, long long n) {
  const long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0u;
}

template <typename T>
void launch_transpose_t(const TransposeArgs& a, hipStream_t s) {
  if (a.R <= 0 || a.C <= 0 || a.batch <= 0) return;
  const dim3 grid((a.C + 63) / 64, (a.R + 63) / 64, a.batch);
  hipLaunchKernelGGL(transpose_kernel<T>, grid, dim3(256), 0, s, a);
}

}  // namespace

void launch_fill_zero(void* p, size_t bytes, hipStream_t s) {
  const long long n = (long long)(bytes / 4);
  if (n == 0) return;
  hipLaunchKernelGGL(fill_zero_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, (uint32_t*)p, n);
}

void launch_bwd_prep(const int32_t* counts, const int32_t* offsets, int E, int Pmax, int Tp, int S, int step,
                     int32_t* kofs, int32_t* klen, int32_t* ksh, int32_t* pcol, int32_t* krow_pad, int32_t* zrow,
                     hipStream_t s) {
  hipLaunchKernelGGL(bwd_prep_kernel, dim3(E > 0 ? E : 1), dim3(256), 0, s, counts, offsets, E, Pmax, Tp, S, step, kofs,
                     klen, ksh, pcol, krow_pad, zrow);
}

void launch_splitk_reduce(const float* part, long long n, int S, float* out, hipStream_t s) {
  if (n <= 0) return;
  hipLaunchKernelGGL(splitk_reduce_kernel, dim3((unsigned)((n / 4 + 255) / 256)), dim3(256), 0, s, part, n, S, out);
}

void launch_transpose(int act, const TransposeArgs& a, hipStream_t s) {
  if (act == 1) launch_transpose_t<bf16_t>(a, s);
  else launch_transpose_t<float>(a, s);
}

void launch_bwd_gate(int act, const void* dy, const void* ou, const void* x, const void* wr, const int32_t* idx,
                     const float* gate, const int32_t* pos, int T, int d, int k, float* dl, int32_t* krow,
                     hipStream_t s) {
  if (T == 0) return;
  const dim3 grid((T + 3) / 4);
  // register arrays sized for k <= 2 (the common case) or k <= 8
  if (act == 1 && k <= 2)
    hipLaunchKernelGGL((bwd_gate_kernel<bf16_t, 2>), grid, dim3(256), 0, s, (const bf16_t*)dy, (const bf16_t*)ou,
                       (const bf16_t*)x, (const bf16_t*)wr, idx, gate, pos, T, d, k, dl, krow);
  else if (act == 1)
    hipLaunchKernelGGL((bwd_gate_kernel<bf16_t, 8>), grid, dim3(256), 0, s, (const bf16_t*)dy, (const bf16_t*)ou,
                       (const bf16_t*)x, (const bf16_t*)wr, idx, gate, pos, T, d, k, dl, krow);
  else
    hipLaunchKernelGGL((bwd_gate_kernel<float, 8>), grid, dim3(256), 0, s, (const float*)dy, (const float*)ou,
                       (const float*)x, (const float*)wr, idx, gate, pos, T, d, k, dl, krow);
}

void launch_bwd_dwr(int act, const void* x, const float* dl, const int32_t* perm, const int32_t* pcol, int P,
                    const int32_t* kofs, const int32_t* klen, int E, int d, int k, float* part, float* dwr,
                    hipStream_t s) {
  const int nch = (P + kPadK - 1) / kPadK;
  if (nch > 0) {
    if (act == 1)
      hipLaunchKernelGGL(bwd_dwr_chunk_kernel<bf16_t>, dim3(nch), dim3(256), 0, s, (const bf16_t*)x, dl, perm, pcol, P,
                         d, k, part);
    else
      hipLaunchKernelGGL(bwd_dwr_chunk_kernel<float>, dim3(nch), dim3(256), 0, s, (const float*)x, dl, perm, pcol, P, d,
                         k, part);
  }
  hipLaunchKernelGGL(bwd_dwr_reduce_kernel, dim3(E, (d + 255) / 256), dim3(256), 0, s, part, kofs, klen, d, dwr);
}

void launch_bwd_dx(int act, const void* dxs, const void* dxp, const void* wr, const float* dl, const int32_t* idx,
                   const int32_t* pos, int T, int d, int k, void* dx, hipStream_t s) {
  const long long n = (long long)T * (d / 8);
  if (n == 0) return;
  const dim3 grid((unsigned)((n + 255) / 256));
  if (act == 1 && k <= 2)
    hipLaunchKernelGGL((bwd_dx_kernel<bf16_t, 2>), grid, dim3(256), 0, s, (const bf16_t*)dxs, (const bf16_t*)dxp,
                       (const bf16_t*)wr, dl, idx, pos, T, d, k, (bf16_t*)dx);
  else if (act == 1)
    hipLaunchKernelGGL((bwd_dx_kernel<bf16_t, 8>), grid, dim3(256), 0, s, (const bf16_t*)dxs, (const bf16_t*)dxp,
                       (const bf16_t*)wr, dl, idx, pos, T, d, k, (bf16_t*)dx);
  else
    hipLaunchKernelGGL((bwd_dx_kernel<float, 8>), grid, dim3(256), 0, s, (const float*)dxs, (const float*)dxp,
                       (const float*)wr, dl, idx, pos, T, d, k, (float*)dx);
}

}  // namespace fgmoe
