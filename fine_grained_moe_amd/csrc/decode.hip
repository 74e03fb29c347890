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
// Five launches for a batch of at most 64 tokens:
//   decode_logits     router logits, 16 workgroups, fp32 partial sums;
//   decode_select     one workgroup: top-1 selection, gates, loads, offsets,
//                     dispatch order and the list of active experts;
//   decode_gate_up    H = silu(x Wg^T) * (x Wu^T) for the shared expert
//                     (bf16) and for each active routed expert over its own
//                     tokens (int4, dequantised in registers);
//   decode_down       fp32 partial sums of Hs Wsd^T (four contraction
//                     quarters) and of H Wd^T (per active expert);
//   decode_combine    y = the four shared partials + the token's routed row,
//                     added in a fixed order and rounded once.
// The weights are read by many small workgroups (one 16-row MFMA tile of a
// weight matrix each, its contraction split over the 4 waves) so that every
// CU streams: with one workgroup per 32 columns the shared expert alone
// occupied only 64 CUs.  At this size the host's launch cost (about 3 us per
// kernel) exceeds the GPU time, so serving callers should capture the
// forward in a HIP graph; nothing here allocates, synchronises or clears
// memory with hipMemsetAsync, so the calls are capturable.
// int4 products: the nibbles are exact small integers in bf16, so each
// 128-element group is multiplied on MFMA into a fresh accumulator and then
// scaled once in fp32 (w = q * scale is never rounded to bf16).
// The path is HBM-bound: every weight byte is read once per launch.
#include "common.h"
#include "kernels.h"

namespace fgmoe {

namespace {

constexpr int kGroup = 128;   // int4 scale group along the contraction dimension

// 16 nibbles (8 bytes) -> 16 bf16 values of the integers they hold, as the two
// 16-byte MFMA operand halves.
__device__ __forceinline__ Frag int4x16_to_bf16(uint2 p) {
  uint32_t out[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const uint32_t byte = ((i < 4 ? p.x : p.y) >> (8 * (i & 3))) & 0xFFu;
    const int lo = (int)(byte & 0xF) - (int)((byte & 0x8) << 1);
    const int hi = (int)(byte >> 4) - (int)((byte & 0x80) >> 3);
    out[i] = (__float_as_uint((float)lo) >> 16) | (__float_as_uint((float)hi) & 0xFFFF0000u);
  }
  Frag f;
  f.lo = u32x4_t{out[0], out[1], out[2], out[3]};
  f.hi = u32x4_t{out[4], out[5], out[6], out[7]};
  return f;
}

// ---------------------------------------------------------------------------
// Router logits for a small batch (T <= 64), split over 16 workgroups so that
// the 128 KiB router matrix is read by 16 CUs at once: workgroup b takes
// experts 16 (b / 4) .. +15 and contraction quarter b % 4; its wave w takes
// 128-byte chunk 4 (b % 4) + w of every row.  The 4 wave tiles are added in
// LDS in a fixed order and written as lpart[b % 4][t][e] (fp32); the
// consumer adds the 4 quarters in a fixed order.
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void decode_logits_kernel(DecodeArgs p) {
  __shared__ float part[4][64][17];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int fr = lane & 15, g = lane >> 4;
  const int kq = blockIdx.x & 3, et = blockIdx.x >> 2;
  if (et * 16 >= p.E) return;
  const int c = kq * 4 + wave;                       // this wave's 128-byte chunk of a row
  const int e = min(et * 16 + fr, p.E - 1);          // rows past E re-read the last expert; never used
  const char* wrow = reinterpret_cast<const char*>(p.w_router + (long long)e * D) + g * 32 + c * 128;
  Frag wf;
  wf.lo = ld16(wrow);
  wf.hi = ld16(wrow + 16);
  for (int m0 = 0; m0 < p.T; m0 += 16) {
    const int t = min(m0 + fr, p.T - 1);
    const char* xrow = reinterpret_cast<const char*>(p.x + (long long)t * D) + g * 32 + c * 128;
    Frag xa;
    xa.lo = ld16(xrow);
    xa.hi = ld16(xrow + 16);
    f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
    acc = Mma<bf16_t>::run(xa, wf, acc);
#pragma unroll
    for (int i = 0; i < 4; ++i) part[wave][(m0 + 4 * g + i) & 63][fr] = acc[i];
  }
  __syncthreads();
  for (int i = tid; i < p.T * 16; i += 256) {
    const int t = i >> 4, cc = i & 15;
    const float v = ((part[0][t][cc] + part[1][t][cc]) + part[2][t][cc]) + part[3][t][cc];
    p.lpart[((long long)kq * p.T + t) * 64 + et * 16 + cc] = v;
  }
}

// ---------------------------------------------------------------------------
// Top-1 selection and dispatch bookkeeping for T <= 64 tokens, run by a whole
// workgroup from the partial logits: logits = the 4 quarters in order;
// s = sigmoid; each token's expert is the largest s + b (an exact tie goes
// to the lower expert); gate = s / s = 1; loads, offsets, the stable
// dispatch order (slots of an expert ascend in t) and the ascending list of
// experts with a load.  Thread (t = tid / 4, q = tid % 4) scans experts
// 16q..16q+15 of token t; two quad merges combine the quarters.
// ---------------------------------------------------------------------------
struct DecodeSel {
  float lg[64][65];
  int ids[64], cnt[64], off[65], perm[64], pos[64];
  int act_e[64], act_s0[64], act_n[64];
  int n_active;
  float bias[64];
};

__device__ void decode_select(const DecodeArgs& p, DecodeSel& S) {
  const int tid = threadIdx.x;
  const int T_ = p.T, E = p.E;
  if (tid < 64) {
    S.bias[tid] = tid < E ? p.bias[tid] : 0.f;
    S.cnt[tid] = 0;
  }
  const long long q1 = (long long)T_ * 64;
  for (int i = tid; i < T_ * 64; i += 256)
    S.lg[i >> 6][i & 63] = ((p.lpart[i] + p.lpart[q1 + i]) + p.lpart[2 * q1 + i]) + p.lpart[3 * q1 + i];
  __syncthreads();
  {
    const int t = tid >> 2, q = tid & 3;
    uint64_t best = 0;
    if (t < T_) {
      float l[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) l[i] = S.lg[t][q * 16 + i];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int e = q * 16 + i;
        const float sc = 1.0f / (1.0f + expf(-l[i]));
        const uint64_t key = ((uint64_t)float_key(sc + S.bias[e]) << 32) | (uint32_t)(63 - e);
        best = (e < E && key > best) ? key : best;
      }
    }
#pragma unroll
    for (int off = 1; off <= 2; off <<= 1) {
      const uint32_t lo = __shfl_xor((uint32_t)best, off), hi = __shfl_xor((uint32_t)(best >> 32), off);
      const uint64_t o = ((uint64_t)hi << 32) | lo;
      best = o > best ? o : best;
    }
    if (q == 0 && t < T_) {
      const int e = 63 - (int)(uint32_t)best;
      S.ids[t] = e;
      atomicAdd(&S.cnt[e], 1);
    }
  }
  __syncthreads();
  if (tid < 64) {
    const int c = S.cnt[tid];
    int incl = c;
    for (int o = 1; o < 64; o <<= 1) {
      const int v = __shfl_up(incl, o);
      if (tid >= o) incl += v;
    }
    S.off[tid] = incl - c;
    if (tid == 63) S.off[64] = incl;
    const bool act = c > 0;
    const unsigned long long m = __ballot(act);
    const int before = __popcll(m & ((1ull << tid) - 1ull));
    if (act) {
      S.act_e[before] = tid;
      S.act_s0[before] = incl - c;
      S.act_n[before] = c;
    }
    if (tid == 0) S.n_active = __popcll(m);
  }
  __syncthreads();
  if (tid < T_) {
    const int e = S.ids[tid];
    int rank = 0;
    for (int b = 0; b < tid; ++b) rank += S.ids[b] == e ? 1 : 0;
    const int slot = S.off[e] + rank;
    S.perm[slot] = tid;
    S.pos[tid] = slot;
  }
  __syncthreads();
}

// The routing outputs of the call.
__device__ void decode_write_routing(const DecodeArgs& p, const DecodeSel& S) {
  const int tid = threadIdx.x;
  if (tid < p.T) {
    const int e = S.ids[tid];
    const float sc = 1.0f / (1.0f + expf(-S.lg[tid][e]));
    p.idx[tid] = e;
    p.gate[tid] = sc / sc;
    p.perm[tid] = S.perm[tid];
    p.pos[tid] = S.pos[tid];
  }
  if (tid < p.E) {
    p.counts[tid] = S.cnt[tid];
    p.offsets[tid] = S.off[tid];
  }
  if (tid == p.E - 1) p.offsets[p.E] = S.off[tid] + S.cnt[tid];
  if (tid < S.n_active) {
    p.active[3 * tid] = S.act_e[tid];
    p.active[3 * tid + 1] = S.act_s0[tid];
    p.active[3 * tid + 2] = S.act_n[tid];
  }
  if (tid == 0) *p.n_active = S.n_active;
}

// One workgroup: selection, bookkeeping and the routing outputs (the
// large-batch router's rules; top-1).
__global__ __launch_bounds__(256) void decode_select_kernel(DecodeArgs p) {
  __shared__ DecodeSel S;
  decode_select(p, S);
  decode_write_routing(p, S);
}

// ---------------------------------------------------------------------------
// Gate/up.  Item i < FS/8: shared expert, h columns 8i .. 8i+7; item >= FS/8:
// routed expert active[(i - FS/8) / (FR/8)], h columns 8 * ((i - FS/8) % (FR/8)).
// The item's 16 weight rows (8 gate rows in MFMA columns 0-7, the matching 8
// up rows in columns 8-15) form one 16x16 MFMA tile; wave w multiplies the
// w-th quarter of the contraction for every 16-token tile and the 4 partial
// tiles are added in LDS in a fixed order, then silu(gate) * up.
// int4 products: each 128-element group goes through MFMA into a fresh
// accumulator and is scaled once in fp32.
// ---------------------------------------------------------------------------
template <int D, int FR, int FS>
__global__ __launch_bounds__(256) void decode_gate_up_kernel(DecodeArgs p) {
  __shared__ float part[4][64][17];                  // [wave][token][MFMA column]
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int fr = lane & 15, g = lane >> 4;
  constexpr int n_sh = FS / 8, nfb = FR / 8;
  const int item = blockIdx.x;
  const bool shared = item < n_sh;
  int e = 0, fblk, ntok, slot0 = 0;
  if (shared) {
    fblk = item;
    ntok = p.T;
  } else {
    const int a = (item - n_sh) / nfb;
    if (a >= *p.n_active) return;
    e = p.active[3 * a];
    slot0 = p.active[3 * a + 1];
    ntok = p.active[3 * a + 2];
    fblk = (item - n_sh) - a * nfb;
  }
  const int N = shared ? FS : FR;                    // rows per half (gate | up)
  const int f = fblk * 8 + (fr & 7);                 // h column of MFMA column fr
  const int wrow = (fr < 8) ? f : N + f;             // its weight row (gate, then up)
  constexpr int nq = D * 2 / 128 / 4;                // 128-byte chunks of a bf16 row per quarter (4)
  const int c0 = wave * nq;

  // this lane's quarter of its weight row, requested before any product
  Frag wbf[nq];
  uint2 wq4[nq];
  uint16_t wsc[nq / 2];
  if (shared) {
    const char* wb = reinterpret_cast<const char*>(p.w_sh_gate_up) + (long long)wrow * D * 2 + g * 32;
#pragma unroll
    for (int c = 0; c < nq; ++c) {
      wbf[c].lo = ld16(wb + (c0 + c) * 128);
      wbf[c].hi = ld16(wb + (c0 + c) * 128 + 16);
    }
  } else {
    const long long r = (long long)e * 2 * FR + wrow;
    const uint8_t* wq = p.q_gate_up + r * (D / 2) + g * 8;
    const bf16_t* ws = p.s_gate_up + r * (D / kGroup);
#pragma unroll
    for (int c = 0; c < nq; ++c) wq4[c] = *reinterpret_cast<const uint2*>(wq + (c0 + c) * 32);
#pragma unroll
    for (int c = 0; c < nq / 2; ++c) wsc[c] = ws[c0 / 2 + c];
  }

  for (int m0 = 0; m0 < ntok; m0 += 16) {
    const int mm = min(m0 + fr, ntok - 1);
    const int tok = shared ? mm : p.perm[slot0 + mm];
    const char* xrow = reinterpret_cast<const char*>(p.x + (long long)tok * D) + g * 32;
    Frag xa[nq];
#pragma unroll
    for (int c = 0; c < nq; ++c) {
      xa[c].lo = ld16(xrow + (c0 + c) * 128);
      xa[c].hi = ld16(xrow + (c0 + c) * 128 + 16);
    }
    f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
    if (shared) {
#pragma unroll
      for (int c = 0; c < nq; ++c) acc = Mma<bf16_t>::run(xa[c], wbf[c], acc);
    } else {
#pragma unroll
      for (int c = 0; c < nq; c += 2) {              // one scale group = 2 chunks of 64 elements
        f32x4_t tmp = {0.f, 0.f, 0.f, 0.f};
        tmp = Mma<bf16_t>::run(xa[c], int4x16_to_bf16(wq4[c]), tmp);
        tmp = Mma<bf16_t>::run(xa[c + 1], int4x16_to_bf16(wq4[c + 1]), tmp);
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[i] += tmp[i] * bf16_to_f32(wsc[c / 2]);
      }
    }
    // acc[i]: token row m0 + 4g + i, MFMA column fr
#pragma unroll
    for (int i = 0; i < 4; ++i) part[wave][(m0 + 4 * g + i) & 63][fr] = acc[i];
  }
  __syncthreads();
  // h = silu(gate) * up from the 4 quarters, added in order
  for (int i = tid; i < ntok * 8; i += 256) {
    const int m = i >> 3, c = i & 7;
    const float a = ((part[0][m][c] + part[1][m][c]) + part[2][m][c]) + part[3][m][c];
    const float u = ((part[0][m][c + 8] + part[1][m][c + 8]) + part[2][m][c + 8]) + part[3][m][c + 8];
    const float h = siluf_(a) * u;
    const int col = fblk * 8 + c;
    if (shared) p.Hs[(long long)m * FS + col] = f32_to_bf16(h);
    else p.H[(long long)(slot0 + m) * FR + col] = f32_to_bf16(h);
  }
}

// ---------------------------------------------------------------------------
// Down.  Item i < 4 * D/16: shared expert, output columns 16 (i / 4) .. +15,
// contraction quarter i % 4 of Fs; item >= 4 * D/16: routed expert
// active[(i - 4D/16) / (D/16)] over its own tokens, output columns
// 16 ((i - 4D/16) % (D/16)), whole contraction F.  The 16 weight rows (output
// columns) form one MFMA tile; the 4 waves split the item's contraction and
// their partial tiles are added in LDS in a fixed order.  Results are fp32:
// shared partials in part_sh[quarter][t][n], routed rows in rout[slot][n].
// ---------------------------------------------------------------------------
template <int D, int FR, int FS>
__global__ __launch_bounds__(256) void decode_down_kernel(DecodeArgs p) {
  __shared__ float part[4][64][17];                  // [wave][token][column]
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int fr = lane & 15, g = lane >> 4;
  constexpr int nblk = D / 16, n_sh = 4 * nblk;
  const int item = blockIdx.x;
  const bool shared = item < n_sh;
  int e = 0, cblk, quarter = 0, ntok, slot0 = 0;
  if (shared) {
    cblk = item >> 2;
    quarter = item & 3;
    ntok = p.T;
  } else {
    const int a = (item - n_sh) / nblk;
    if (a >= *p.n_active) return;
    e = p.active[3 * a];
    slot0 = p.active[3 * a + 1];
    ntok = p.active[3 * a + 2];
    cblk = (item - n_sh) - a * nblk;
  }
  const int n = cblk * 16 + fr;                      // this lane's weight row = output column
  // shared: wave w takes chunks [quarter * 8 + 2w, +2) of the 32 chunks of Fs;
  // routed: wave w takes chunks [2w, 2w + 2) of the 8 chunks of F (one scale group)
  constexpr int nch = 2;
  Frag wf[nch];
  uint2 q4[nch];
  uint16_t sc = 0;
  int cbase;
  if (shared) {
    cbase = quarter * (FS * 2 / 128 / 4) + wave * nch;
    const char* wb = reinterpret_cast<const char*>(p.w_sh_down) + (long long)n * FS * 2 + g * 32;
#pragma unroll
    for (int c = 0; c < nch; ++c) {
      wf[c].lo = ld16(wb + (cbase + c) * 128);
      wf[c].hi = ld16(wb + (cbase + c) * 128 + 16);
    }
  } else {
    cbase = wave * nch;
    const long long r = (long long)e * D + n;
    const uint8_t* wq = p.q_down + r * (FR / 2) + g * 8;
#pragma unroll
    for (int c = 0; c < nch; ++c) q4[c] = *reinterpret_cast<const uint2*>(wq + (cbase + c) * 32);
    sc = p.s_down[r * (FR / kGroup) + wave];
  }
  const bf16_t* A = shared ? p.Hs : p.H;
  const int lda = shared ? FS : FR;
  for (int m0 = 0; m0 < ntok; m0 += 16) {
    const int mm = min(m0 + fr, ntok - 1);
    const char* arow = reinterpret_cast<const char*>(A + (long long)(slot0 + mm) * lda) + g * 32;
    Frag ha[nch];
#pragma unroll
    for (int c = 0; c < nch; ++c) {
      ha[c].lo = ld16(arow + (cbase + c) * 128);
      ha[c].hi = ld16(arow + (cbase + c) * 128 + 16);
    }
    f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
    if (shared) {
#pragma unroll
      for (int c = 0; c < nch; ++c) acc = Mma<bf16_t>::run(ha[c], wf[c], acc);
    } else {
      acc = Mma<bf16_t>::run(ha[0], int4x16_to_bf16(q4[0]), acc);
      acc = Mma<bf16_t>::run(ha[1], int4x16_to_bf16(q4[1]), acc);
      const float s = bf16_to_f32(sc);
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[i] *= s;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) part[wave][(m0 + 4 * g + i) & 63][fr] = acc[i];
  }
  __syncthreads();
  float* dst = shared ? p.part_sh + (long long)quarter * p.T * D : p.rout;
  for (int i = tid; i < ntok * 16; i += 256) {
    const int m = i >> 4, c = i & 15;
    const float v = ((part[0][m][c] + part[1][m][c]) + part[2][m][c]) + part[3][m][c];
    dst[(long long)(slot0 + m) * D + cblk * 16 + c] = v;
  }
}

// ---------------------------------------------------------------------------
// y[t, n] = (((sh0 + sh1) + sh2) + sh3)[t, n] + rout[pos[t], n], rounded once
// (top-1: the token's single routed row carries gate 1).
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void decode_combine_kernel(DecodeArgs p) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i >= p.T * D) return;
  const int t = i / D, n = i - t * D;
  const long long q = (long long)p.T * D;
  const float sh = ((p.part_sh[i] + p.part_sh[q + i]) + p.part_sh[2 * q + i]) + p.part_sh[3 * q + i];
  p.y[i] = f32_to_bf16(sh + p.rout[(long long)p.pos[t] * D + n]);
}

}  // namespace

bool decode_shape_supported(int d, int F, int Fs) { return d == kDecodeD && F == kDecodeF && Fs == kDecodeFs; }

void launch_decode(const DecodeArgs& a, hipStream_t s) {
  constexpr int D = kDecodeD, FR = kDecodeF, FS = kDecodeFs;
  if (a.T > 0) hipLaunchKernelGGL(decode_logits_kernel<D>, dim3(16), dim3(256), 0, s, a);
  hipLaunchKernelGGL(decode_select_kernel, dim3(1), dim3(256), 0, s, a);   // also writes the empty routing of T = 0
  if (a.T == 0) return;
  const int max_active = a.T * a.k < a.E ? a.T * a.k : a.E;
  hipLaunchKernelGGL((decode_gate_up_kernel<D, FR, FS>), dim3(FS / 8 + max_active * (FR / 8)), dim3(256), 0, s, a);
  hipLaunchKernelGGL((decode_down_kernel<D, FR, FS>), dim3(4 * (D / 16) + max_active * (D / 16)), dim3(256), 0, s, a);
  hipLaunchKernelGGL(decode_combine_kernel<D>, dim3((a.T * D + 255) / 256), dim3(256), 0, s, a);
}

}  // namespace fgmoe
