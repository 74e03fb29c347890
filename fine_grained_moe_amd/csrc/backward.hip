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
// operands are transposed here.  Each expert's rows are laid out in its own
// column range padded to a multiple of 64 with zeros, so that a grouped GEMM
// with a per-expert contraction range can run over it.
#include "common.h"
#include "kernels.h"

namespace fgmoe {

namespace {

// ---------------------------------------------------------------------------
// Per-expert padded column ranges: klen[e] = roundup(count[e], 64),
// kofs = exclusive scan; pcol[c] = slot held by padded column c, or -1.
// Also the single-range tables of the shared expert: kofs_sh = 0, klen_sh = Tp.
// One workgroup of 1024 threads.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(1024) void bwd_prep_kernel(const int32_t* __restrict__ counts,
                                                        const int32_t* __restrict__ offsets, int E, int Pmax, int Tp,
                                                        int32_t* __restrict__ kofs, int32_t* __restrict__ klen,
                                                        int32_t* __restrict__ ksh, int32_t* __restrict__ pcol) {
  __shared__ int s_kofs[64], s_klen[64];
  const int tid = threadIdx.x;
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
    if (tid < E) {
      kofs[tid] = incl - kl;
      klen[tid] = kl;
    }
  }
  if (tid == 0) {
    ksh[0] = 0;
    ksh[1] = Tp;
  }
  __syncthreads();
  for (int c = tid; c < Pmax; c += blockDim.x) pcol[c] = -1;
  __syncthreads();
  for (int e = 0; e < E; ++e) {
    const int c0 = s_kofs[e], n = counts[e], o = offsets[e];
    for (int i = tid; i < n; i += blockDim.x) pcol[c0 + i] = o + i;
  }
}

// ---------------------------------------------------------------------------
// Gather-transpose: dst[b][r][c] = scale * src[b][row(c)][r], for r < R and
// c < C, where row(c) is c (c < n_in), map1[c] (>= 0), or, with map2,
// map2[map1[c]] / div; a column without a row is zero.  The scale is
// scale[map2 ? map2[map1[c]] : map1[c]] when given.  64 x 64 tiles via LDS.
// ---------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(256) void transpose_kernel(TransposeArgs a) {
  __shared__ float tile[64][65];
  const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
  const int c0 = blockIdx.x * 64, r0 = blockIdx.y * 64;
  const T* src = reinterpret_cast<const T*>(a.src) + (long long)blockIdx.z * a.src_bstride;
  T* dst = reinterpret_cast<T*>(a.dst) + (long long)blockIdx.z * a.dst_bstride;
  const int r = r0 + tx;
#pragma unroll 4
  for (int i = 0; i < 16; ++i) {
    const int cl = ty * 16 + i, c = c0 + cl;
    float v = 0.f;
    if (c < a.C && r < a.R) {
      int m = a.map1 ? a.map1[c] : (c < a.n_in ? c : -1);
      if (m >= 0) {
        int sidx = m;
        if (a.map2) {
          sidx = a.map2[m];
          m = sidx / a.div;
        }
        v = to_f32<T>(src[(long long)m * a.ld_src + r]);
        if (a.scale) v *= a.scale[sidx];
      }
    }
    tile[cl][tx] = v;
  }
  __syncthreads();
#pragma unroll 4
  for (int i = 0; i < 16; ++i) {
    const int rl = ty * 16 + i, rr = r0 + rl, c = c0 + tx;
    if (rr < a.R && c < a.C) dst[(long long)rr * a.ld_dst + c] = from_f32<T>(tile[tx][rl]);
  }
}

// ---------------------------------------------------------------------------
// Router and gate gradients, one wave per token: dg_j = <dy_t, o_j>; the
// selected scores are recomputed from the logits x_t . W_r[e_j]; then the
// formulas at the top of this file.  dl: [T, k] fp32.
// ---------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(256) void bwd_gate_kernel(const T* __restrict__ dy, const T* __restrict__ ou,
                                                       const T* __restrict__ x, const T* __restrict__ wr,
                                                       const int32_t* __restrict__ idx, const float* __restrict__ gate,
                                                       const int32_t* __restrict__ pos, int T_, int d, int k,
                                                       float* __restrict__ dl) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T_) return;
  float dg[8], s[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    if (j >= k) break;
    const int e = idx[(long long)t * k + j];
    const long long slot = pos[(long long)t * k + j];
    float a = 0.f, b = 0.f;
    for (int c = lane; c < d; c += 64) {
      a += to_f32<T>(dy[(long long)t * d + c]) * to_f32<T>(ou[slot * d + c]);
      b += to_f32<T>(x[(long long)t * d + c]) * to_f32<T>(wr[(long long)e * d + c]);
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
      a += __shfl_xor(a, o);
      b += __shfl_xor(b, o);
    }
    dg[j] = a;
    s[j] = 1.0f / (1.0f + expf(-b));
  }
  if (lane == 0) {
    float S = 0.f, G = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if (j >= k) break;
      S += s[j];
      G += gate[(long long)t * k + j] * dg[j];
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if (j >= k) break;
      dl[(long long)t * k + j] = (dg[j] - G) / S * s[j] * (1.f - s[j]);
    }
  }
}

// ---------------------------------------------------------------------------
// dW_r[e][c] = sum over the slots of e, in slot order, of dl[perm[s]] * x[token][c].
// ---------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(256) void bwd_dwr_kernel(const T* __restrict__ x, const float* __restrict__ dl,
                                                      const int32_t* __restrict__ perm,
                                                      const int32_t* __restrict__ counts,
                                                      const int32_t* __restrict__ offsets, int d, int k,
                                                      float* __restrict__ dwr) {
  const int e = blockIdx.x;
  const int c = blockIdx.y * 256 + threadIdx.x;
  if (c >= d) return;
  const int o = offsets[e], n = counts[e];
  float acc = 0.f;
  for (int i = 0; i < n; ++i) {
    const int a = perm[o + i];
    acc += dl[a] * to_f32<T>(x[(long long)(a / k) * d + c]);
  }
  dwr[(long long)e * d + c] = acc;
}

// ---------------------------------------------------------------------------
// dx[t] = dXs[t] + sum_j dXp[pos[t, j]] + sum_j dl[t, j] W_r[idx[t, j]], in that
// order in fp32, rounded once.
// ---------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(256) void bwd_dx_kernel(const T* __restrict__ dxs, const T* __restrict__ dxp,
                                                     const T* __restrict__ wr, const float* __restrict__ dl,
                                                     const int32_t* __restrict__ idx, const int32_t* __restrict__ pos,
                                                     int T_, int d, int k, T* __restrict__ dx) {
  const long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= (long long)T_ * d) return;
  const int t = (int)(i / d), c = (int)(i - (long long)t * d);
  float v = to_f32<T>(dxs[i]);
  for (int j = 0; j < k; ++j) v += to_f32<T>(dxp[(long long)pos[(long long)t * k + j] * d + c]);
  for (int j = 0; j < k; ++j)
    v += dl[(long long)t * k + j] * to_f32<T>(wr[(long long)idx[(long long)t * k + j] * d + c]);
  dx[i] = from_f32<T>(v);
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

void launch_bwd_prep(const int32_t* counts, const int32_t* offsets, int E, int Pmax, int Tp, int32_t* kofs,
                     int32_t* klen, int32_t* ksh, int32_t* pcol, hipStream_t s) {
  hipLaunchKernelGGL(bwd_prep_kernel, dim3(1), dim3(1024), 0, s, counts, offsets, E, Pmax, Tp, kofs, klen, ksh, pcol);
}

void launch_transpose(int act, const TransposeArgs& a, hipStream_t s) {
  if (act == 1) launch_transpose_t<bf16_t>(a, s);
  else launch_transpose_t<float>(a, s);
}

void launch_bwd_gate(int act, const void* dy, const void* ou, const void* x, const void* wr, const int32_t* idx,
                     const float* gate, const int32_t* pos, int T, int d, int k, float* dl, hipStream_t s) {
  if (T == 0) return;
  const dim3 grid((T + 3) / 4);
  if (act == 1)
    hipLaunchKernelGGL(bwd_gate_kernel<bf16_t>, grid, dim3(256), 0, s, (const bf16_t*)dy, (const bf16_t*)ou,
                       (const bf16_t*)x, (const bf16_t*)wr, idx, gate, pos, T, d, k, dl);
  else
    hipLaunchKernelGGL(bwd_gate_kernel<float>, grid, dim3(256), 0, s, (const float*)dy, (const float*)ou,
                       (const float*)x, (const float*)wr, idx, gate, pos, T, d, k, dl);
}

void launch_bwd_dwr(int act, const void* x, const float* dl, const int32_t* perm, const int32_t* counts,
                    const int32_t* offsets, int E, int d, int k, float* dwr, hipStream_t s) {
  const dim3 grid(E, (d + 255) / 256);
  if (act == 1)
    hipLaunchKernelGGL(bwd_dwr_kernel<bf16_t>, grid, dim3(256), 0, s, (const bf16_t*)x, dl, perm, counts, offsets, d,
                       k, dwr);
  else
    hipLaunchKernelGGL(bwd_dwr_kernel<float>, grid, dim3(256), 0, s, (const float*)x, dl, perm, counts, offsets, d, k,
                       dwr);
}

void launch_bwd_dx(int act, const void* dxs, const void* dxp, const void* wr, const float* dl, const int32_t* idx,
                   const int32_t* pos, int T, int d, int k, void* dx, hipStream_t s) {
  const long long n = (long long)T * d;
  if (n == 0) return;
  const dim3 grid((unsigned)((n + 255) / 256));
  if (act == 1)
    hipLaunchKernelGGL(bwd_dx_kernel<bf16_t>, grid, dim3(256), 0, s, (const bf16_t*)dxs, (const bf16_t*)dxp,
                       (const bf16_t*)wr, dl, idx, pos, T, d, k, (bf16_t*)dx);
  else
    hipLaunchKernelGGL(bwd_dx_kernel<float>, grid, dim3(256), 0, s, (const float*)dxs, (const float*)dxp,
                       (const float*)wr, dl, idx, pos, T, d, k, (float*)dx);
}

}  // namespace fgmoe
