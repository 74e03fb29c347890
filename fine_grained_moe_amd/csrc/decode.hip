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
// Three launches for a batch of at most 64 tokens:
//   decode_route      one workgroup: logits (MFMA), top-k, gates, loads,
//                     offsets, dispatch order and the list of active experts;
//   decode_gate_up    H  = silu(x Wg^T) * (x Wu^T) for the shared expert (bf16)
//                     and for each active routed expert over its own tokens
//                     (int4, dequantised in registers);
//   decode_down       y = Hs Wsd^T + H Wd^T, the combine fused in.
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
// Router for a small batch (T <= 64), one workgroup of 4 waves: wave w owns
// tokens 16w..16w+15 and all E <= 64 experts (4 MFMA tiles); then the same
// top-k rule as the large-batch router; then loads, offsets, the stable
// dispatch order and the list of experts with a non-zero load.
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void decode_route_kernel(const uint16_t* __restrict__ x, const uint16_t* __restrict__ wr,
                                                           const float* __restrict__ bias, int T_, int E, int k,
                                                           int32_t* __restrict__ idx, float* __restrict__ gate,
                                                           int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
                                                           int32_t* __restrict__ perm, int32_t* __restrict__ pos,
                                                           int32_t* __restrict__ active, int32_t* __restrict__ n_active) {
  __shared__ float lgp[4][64][65];                   // per-wave partial logits [wave][token][expert]
  __shared__ float lg[64][65];
  __shared__ int ids[64 * 8];
  __shared__ int cnt[64], off[65];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r = lane & 15, g = lane >> 4;
  // wave w multiplies the w-th quarter of d for every token and expert; its
  // quarter of the 128 KiB router matrix is requested before any product
  constexpr int d = D;
  constexpr int nq = D * 2 / 128 / 4;                // 128-byte chunks per quarter
  static_assert(nq >= 1 && nq <= 4, "router quarter of 1..4 chunks");
  const int c0 = wave * nq;
  if (T_ > 0) {
    Frag b[4][4];
#pragma unroll
    for (int ni = 0; ni < 4; ++ni) {
      const char* wrow = reinterpret_cast<const char*>(wr + (long long)min(ni * 16 + r, E - 1) * d) + g * 32;
#pragma unroll
      for (int c = 0; c < 4; ++c)
        if (c < nq) {
          b[ni][c].lo = ld16(wrow + (c0 + c) * 128);
          b[ni][c].hi = ld16(wrow + (c0 + c) * 128 + 16);
        }
    }
    for (int m0 = 0; m0 < T_; m0 += 16) {
      const int t = min(m0 + r, T_ - 1);
      const char* xrow = reinterpret_cast<const char*>(x + (long long)t * d) + g * 32;
      f32x4_t acc[4];
#pragma unroll
      for (int ni = 0; ni < 4; ++ni) acc[ni] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      for (int cb = 0; cb < nq; cb += 4) {
        Frag a[4];
#pragma unroll
        for (int c = 0; c < 4; ++c)
          if (cb + c < nq) {
            a[c].lo = ld16(xrow + (c0 + cb + c) * 128);
            a[c].hi = ld16(xrow + (c0 + cb + c) * 128 + 16);
          }
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          if (cb + c >= nq) break;
#pragma unroll
          for (int ni = 0; ni < 4; ++ni) {
            Frag bb;
            if (cb == 0) bb = b[ni][c];
            else {   // quarters longer than 4 chunks (d > 1024) stream the rest
              const char* wrow = reinterpret_cast<const char*>(wr + (long long)min(ni * 16 + r, E - 1) * d) + g * 32;
              bb.lo = ld16(wrow + (c0 + cb + c) * 128);
              bb.hi = ld16(wrow + (c0 + cb + c) * 128 + 16);
            }
            acc[ni] = Mma<bf16_t>::run(a[c], bb, acc[ni]);
          }
        }
      }
#pragma unroll
      for (int ni = 0; ni < 4; ++ni)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int m = m0 + 4 * g + i;
          if (m < 64) lgp[wave][m][ni * 16 + r] = acc[ni][i];
        }
    }
  }
  __syncthreads();
  for (int i = tid; i < T_ * 64; i += 256) {
    const int t = i >> 6, e = i & 63;
    lg[t][e] = ((lgp[0][t][e] + lgp[1][t][e]) + lgp[2][t][e]) + lgp[3][t][e];
  }
  __syncthreads();

  const float b_e = lane < E ? bias[lane] : 0.f;
  for (int t = wave; t < T_; t += 4) {
    const float l = lane < E ? lg[t][lane] : 0.f;
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
      for (int o = 32; o >= 1; o >>= 1) {
        const uint32_t ohi = __shfl_xor(hi, o), olo = __shfl_xor(lo, o);
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
        idx[t * k + j] = esel[j];
        gate[t * k + j] = ssel[j] / ssum;
        ids[t * k + j] = esel[j];
      }
    }
  }
  __syncthreads();
  const int na = T_ * k;
  if (tid < 64) {
    int c = 0;
    if (tid < E)
      for (int a = 0; a < na; ++a) c += ids[a] == tid ? 1 : 0;
    cnt[tid] = c;
    int incl = c;
    for (int o = 1; o < 64; o <<= 1) {
      const int v = __shfl_up(incl, o);
      if (tid >= o) incl += v;
    }
    off[tid] = incl - c;
    if (tid == 63) off[64] = incl;
    // active experts in ascending order
    const bool act = c > 0;
    const unsigned long long m = __ballot(act);
    const int before = __popcll(m & ((1ull << tid) - 1ull));
    if (act) {   // descriptor of the before-th active expert: (expert, first slot, load)
      active[3 * before] = tid;
      active[3 * before + 1] = incl - c;
      active[3 * before + 2] = c;
    }
    if (tid == 0) *n_active = __popcll(m);
    if (tid < E) {
      counts[tid] = c;
      offsets[tid] = incl - c;
    }
    if (tid == E - 1) offsets[E] = incl;
  }
  __syncthreads();
  for (int a = tid; a < na; a += blockDim.x) {
    const int e = ids[a];
    int rank = 0;
    for (int b = 0; b < a; ++b) rank += ids[b] == e ? 1 : 0;
    const int slot = off[e] + rank;
    perm[slot] = a;
    pos[a] = slot;
  }
}

// ---------------------------------------------------------------------------
// Gate/up GEMV-like products.  Item i < n_sh: shared expert, f-block i of 32;
// item >= n_sh: routed expert active[(i - n_sh) / nfb], f-block (i - n_sh) % nfb.
// Wave w of the block computes h columns f0 + 8w .. f0 + 8w + 7: its 16x16
// MFMA tile has the 8 gate rows in columns 0-7 and the matching 8 up rows in
// columns 8-15, so silu(gate) * up pairs lane l with lane l ^ 8.
// ---------------------------------------------------------------------------
template <int D, int FR, int FS>
__global__ __launch_bounds__(256) void decode_gate_up_kernel(DecodeArgs p) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int fr = lane & 15, g = lane >> 4;
  constexpr int n_sh = FS / 32, nfb = FR / 32;
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
  const int f = fblk * 32 + wave * 8 + (fr & 7);     // this lane's h column
  const int wrow = (fr < 8) ? f : N + f;             // its weight row (gate, then up)
  constexpr int nch = D * 2 / 128;                   // 128-byte chunks of a bf16 row

  // weight row pointers for this lane
  const char* wb = nullptr;
  const uint8_t* wq = nullptr;
  const bf16_t* ws = nullptr;
  if (shared) {
    wb = reinterpret_cast<const char*>(p.w_sh_gate_up) + (long long)wrow * D * 2 + g * 32;
  } else {
    const long long r = (long long)e * 2 * FR + wrow;
    wq = p.q_gate_up + r * (D / 2) + g * 8;
    ws = p.s_gate_up + r * (D / kGroup);
  }

  // this lane's whole weight row slice is requested before any product
  constexpr int MAXCH = nch;
  Frag wbf[MAXCH];
  uint2 wq4[MAXCH];
  uint16_t wsc[MAXCH / 2];
  if (shared) {
#pragma unroll
    for (int c = 0; c < MAXCH; ++c)
      if (c < nch) {
        wbf[c].lo = ld16(wb + c * 128);
        wbf[c].hi = ld16(wb + c * 128 + 16);
      }
  } else {
#pragma unroll
    for (int c = 0; c < MAXCH; ++c)
      if (c < nch) wq4[c] = *reinterpret_cast<const uint2*>(wq + c * 32);
#pragma unroll
    for (int c = 0; c < MAXCH / 2; ++c)
      wsc[c] = ws[c];
  }

  for (int m0 = 0; m0 < ntok; m0 += 16) {
    // this lane's A row: token (shared) or slot's token (routed)
    const int mm = min(m0 + fr, ntok - 1);
    const int tok = shared ? mm : p.perm[slot0 + mm];
    const char* xrow = reinterpret_cast<const char*>(p.x + (long long)tok * D) + g * 32;
    Frag xa[MAXCH];
#pragma unroll
    for (int c = 0; c < MAXCH; ++c)
      if (c < nch) {
        xa[c].lo = ld16(xrow + c * 128);
        xa[c].hi = ld16(xrow + c * 128 + 16);
      }
    f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
    if (shared) {
#pragma unroll
      for (int c = 0; c < MAXCH; ++c)
        if (c < nch) acc = Mma<bf16_t>::run(xa[c], wbf[c], acc);
    } else {
      // one scale group = 2 chunks of 64 elements: fresh accumulator, then scaled
#pragma unroll
      for (int c = 0; c < MAXCH; c += 2) {
        if (c >= nch) break;
        f32x4_t tmp = {0.f, 0.f, 0.f, 0.f};
        tmp = Mma<bf16_t>::run(xa[c], int4x16_to_bf16(wq4[c]), tmp);
        tmp = Mma<bf16_t>::run(xa[c + 1], int4x16_to_bf16(wq4[c + 1]), tmp);
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[i] += tmp[i] * bf16_to_f32(wsc[c / 2]);
      }
    }
    // acc[i]: token row m0 + 4g + i, column fr (gate for fr < 8, up for fr >= 8)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float other = __shfl_xor(acc[i], 8);
      const int m = m0 + 4 * g + i;
      if (fr < 8 && m < ntok) {
        const float h = siluf_(acc[i]) * other;
        if (shared) p.Hs[(long long)m * FS + f] = f32_to_bf16(h);
        else p.H[(long long)(slot0 + m) * FR + f] = f32_to_bf16(h);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Down projections and the combine.  Block b owns output columns
// 16b .. 16b + 15 for every token.  The 4 waves split the shared expert's
// contraction dimension and take the active routed experts in turn; the
// shared partial sums meet in LDS and are added in a fixed order, then the
// token's routed row (slot pos[t]) is added and the sum rounded once.
//   y[t, n] = sum_f Hs[t, f] Wsd[n, f] + sum_f H[pos(t), f] Wd_e(t)[n, f]
// ---------------------------------------------------------------------------
template <int D, int FR, int FS>
__global__ __launch_bounds__(256) void decode_down_kernel(DecodeArgs p) {
  __shared__ float part[4][64][17];                  // shared expert: [wave][token][column]
  __shared__ float rout[64][17];                     // routed expert: [slot][column]
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int fr = lane & 15, g = lane >> 4;
  const int n = blockIdx.x * 16 + fr;                // this lane's weight row = output column
  // independent small loads first: the number of active experts and, for the
  // final sum, the slot of each token this thread will write
  const int na = *p.n_active;
  int my_slot[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int i = tid + 256 * j;
    my_slot[j] = i < p.T * 16 ? p.pos[i >> 4] : 0;
  }

  // shared expert: K = Fs, wave w takes chunks [w*ncs, (w+1)*ncs), its weight
  // slice requested before any product
  {
    constexpr int nch = FS * 2 / 128, ncs = nch / 4, MAXQ = ncs;
    const char* wb = reinterpret_cast<const char*>(p.w_sh_down) + (long long)n * FS * 2 + g * 32 + wave * ncs * 128;
    Frag wf[MAXQ];
#pragma unroll
    for (int c = 0; c < MAXQ; ++c)
      if (c < ncs) {
        wf[c].lo = ld16(wb + c * 128);
        wf[c].hi = ld16(wb + c * 128 + 16);
      }
    for (int m0 = 0; m0 < p.T; m0 += 16) {
      const int tok = min(m0 + fr, p.T - 1);
      const char* hrow = reinterpret_cast<const char*>(p.Hs + (long long)tok * FS) + g * 32 + wave * ncs * 128;
      Frag ha[MAXQ];
#pragma unroll
      for (int c = 0; c < MAXQ; ++c)
        if (c < ncs) {
          ha[c].lo = ld16(hrow + c * 128);
          ha[c].hi = ld16(hrow + c * 128 + 16);
        }
      f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < MAXQ; ++c)
        if (c < ncs) acc = Mma<bf16_t>::run(ha[c], wf[c], acc);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int m = m0 + 4 * g + i;
        if (m < p.T) part[wave][m][fr] = acc[i];
      }
    }
  }
  // routed experts: wave w takes active experts w, w + 4, ... whole (K = F, up
  // to 8 chunks of 64 elements = 4 scale groups), two experts' weights in
  // flight at a time
  {
    constexpr int nch = FR * 2 / 128, ngr = nch / 2, MAXC = nch;
    for (int a0 = wave; a0 < na; a0 += 8) {
      uint2 q[2][MAXC];
      uint16_t sc[2][MAXC / 2];
      int es[2], s0[2], nt[2];
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int a = a0 + 4 * u;
        es[u] = a < na ? p.active[3 * a] : -1;
        s0[u] = a < na ? p.active[3 * a + 1] : 0;
        nt[u] = a < na ? p.active[3 * a + 2] : 0;
        if (es[u] < 0) continue;
        const long long r = (long long)es[u] * D + n;
        const uint8_t* wq = p.q_down + r * (FR / 2) + g * 8;
        const bf16_t* ws = p.s_down + r * ngr;
#pragma unroll
        for (int c = 0; c < MAXC; ++c)
          if (c < nch) q[u][c] = *reinterpret_cast<const uint2*>(wq + c * 32);
#pragma unroll
        for (int c = 0; c < MAXC / 2; ++c)
          sc[u][c] = ws[c];
      }
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        if (es[u] < 0) continue;
        const int ntok = nt[u], slot0 = s0[u];
        for (int m0 = 0; m0 < ntok; m0 += 16) {
          const int mm = min(m0 + fr, ntok - 1);
          const char* hrow = reinterpret_cast<const char*>(p.H + (long long)(slot0 + mm) * FR) + g * 32;
          f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int c = 0; c < MAXC; c += 2) {
            if (c >= nch) break;
            Frag a0f, a1f;
            a0f.lo = ld16(hrow + c * 128);
            a0f.hi = ld16(hrow + c * 128 + 16);
            a1f.lo = ld16(hrow + (c + 1) * 128);
            a1f.hi = ld16(hrow + (c + 1) * 128 + 16);
            f32x4_t tmp = {0.f, 0.f, 0.f, 0.f};
            tmp = Mma<bf16_t>::run(a0f, int4x16_to_bf16(q[u][c]), tmp);
            tmp = Mma<bf16_t>::run(a1f, int4x16_to_bf16(q[u][c + 1]), tmp);
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[i] += tmp[i] * bf16_to_f32(sc[u][c / 2]);
          }
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int m = m0 + 4 * g + i;
            if (m < ntok) rout[slot0 + m][fr] = acc[i];
          }
        }
      }
    }
  }
  __syncthreads();
  // y = shared (its 4 wave partials in order) + the token's routed row (k = 1:
  // slot pos[t]), rounded once
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int i = tid + 256 * j;
    if (i >= p.T * 16) break;
    const int t = i >> 4, c = i & 15;
    const float sh = ((part[0][t][c] + part[1][t][c]) + part[2][t][c]) + part[3][t][c];
    p.y[(long long)t * D + blockIdx.x * 16 + c] = f32_to_bf16(sh + rout[my_slot[j]][c]);
  }
}

}  // namespace

bool decode_shape_supported(int d, int F, int Fs) { return d == kDecodeD && F == kDecodeF && Fs == kDecodeFs; }

void launch_decode(const DecodeArgs& a, hipStream_t s) {
  constexpr int D = kDecodeD, FR = kDecodeF, FS = kDecodeFs;
  hipLaunchKernelGGL(decode_route_kernel<D>, dim3(1), dim3(256), 0, s, a.x, a.w_router, a.bias, a.T, a.E, a.k, a.idx,
                     a.gate, a.counts, a.offsets, a.perm, a.pos, a.active, a.n_active);
  if (a.T == 0) return;
  const int max_active = a.T * a.k < a.E ? a.T * a.k : a.E;
  hipLaunchKernelGGL((decode_gate_up_kernel<D, FR, FS>), dim3(FS / 32 + max_active * (FR / 32)), dim3(256), 0, s, a);
  hipLaunchKernelGGL((decode_down_kernel<D, FR, FS>), dim3(D / 16), dim3(256), 0, s, a);
}

}  // namespace fgmoe
