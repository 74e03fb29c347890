// Expert GEMMs of the MoE layer on gfx950 MFMA, with fused epilogues.
//
// One kernel template serves the four GEMMs of the forward:
//   routed gate/up  (grouped over experts, A rows gathered from x through the
//                    dispatch order, SwiGLU epilogue -> H)
//   routed down     (grouped, rows scaled by their routing weight -> O)
//   shared gate/up  (dense, SwiGLU epilogue -> Hs)
//   shared down     (dense, epilogue adds the token's k routed rows of O -> y)
// The experts are the SwiGLU FFNs of widths 512 (routed) and 2048 (shared) of
// the seventnews article "A relay race of rented GPUs trained NanoColibri's
// 2.7B MoE for $200" (opening section, architecture paragraph).  A launch may
// carry two jobs with the same epilogue (the routed and the shared gate/up):
// their workgroups are interleaved, so the weight-streaming routed tiles and
// the MFMA-bound shared tiles share the chip.
//
// Tiling: a 256-thread workgroup (4 waves, 2 x 2) computes a 128 x 128 tile;
// each wave owns 64 x 64 = 4 x 4 MFMA 16x16 tiles.  K advances in 128-byte
// row chunks (64 bf16 or 32 float) staged through LDS, double-buffered, with
// two stages of global loads in flight.  The 16-byte pieces of each LDS row
// are XOR-swizzled (see swz) so that both the 16-row operand reads and the
// loader's writes are free of bank conflicts.
// B rows are permuted on their way into LDS so that each lane's output
// columns are adjacent and the epilogue writes 4- to 16-byte vectors.
//
// Scheduling: work items are 128-row tiles (dense: row blocks; grouped: the
// tile table the router wrote, in expert order).  Workgroups are dealt to the
// 8 XCDs round-robin by block index, so block b runs on XCD b % 8; XCD x gets
// the contiguous item range [x*q, (x+1)*q).  Grouped jobs run all N tiles of
// an item back to back (an expert's weights and an item's rows stay in that
// XCD's L2); dense jobs run all of the XCD's row blocks for one N tile before
// the next (the XCD's A rows stay in L2 while the large weight matrix streams
// through once).  No host synchronisation: the item count is read on the
// device.
#include "common.h"
#include "kernels.h"

namespace fgmoe {

namespace {

constexpr int BM = 128, BN = 128, NTHR = 256;
constexpr int ROWB = 128;                    // bytes of one row per K stage
constexpr int TILEB = BM * ROWB;             // bytes of one operand tile per stage

// Piece p of LDS row r sits at piece p ^ (r & 7) ^ ((r >> 3) & 1): measured on
// gfx950, 16 consecutive rows read at one piece index then hit distinct banks.
__device__ __forceinline__ int swz(int row, int piece) {
  return row * ROWB + ((piece ^ (row & 7) ^ ((row >> 3) & 1)) << 4);
}

template <int EPI> __device__ __forceinline__ int n_tiles(const GemmJob& j) {
  return EPI == EPI_SWIGLU ? j.N / 64 : j.N / BN;
}
__device__ __forceinline__ int item_count(const GemmJob& j) {
  return j.grouped ? *j.tile_count : (j.M + BM - 1) / BM;
}

template <typename T, int N>
__device__ __forceinline__ void store_vec(T* p, const float (&v)[N]) {
  if constexpr (sizeof(T) == 2) {
    uint32_t w[(N + 1) / 2];
#pragma unroll
    for (int i = 0; i < N; i += 2)
      w[i / 2] = (uint32_t)f32_to_bf16(v[i]) | ((uint32_t)f32_to_bf16(v[i + 1]) << 16);
    if constexpr (N == 2) *reinterpret_cast<uint32_t*>(p) = w[0];
    else *reinterpret_cast<uint2*>(p) = make_uint2(w[0], w[1]);
  } else {
    if constexpr (N == 2) *reinterpret_cast<float2*>(p) = make_float2(v[0], v[1]);
    else *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
  }
}

template <typename T>
__device__ __forceinline__ void load_add4(const T* p, float (&v)[4]) {
  if constexpr (sizeof(T) == 2) {
    const uint2 w = *reinterpret_cast<const uint2*>(p);
    v[0] += bf16_to_f32((bf16_t)(w.x & 0xFFFF));
    v[1] += bf16_to_f32((bf16_t)(w.x >> 16));
    v[2] += bf16_to_f32((bf16_t)(w.y & 0xFFFF));
    v[3] += bf16_to_f32((bf16_t)(w.y >> 16));
  } else {
    const float4 w = *reinterpret_cast<const float4*>(p);
    v[0] += w.x;
    v[1] += w.y;
    v[2] += w.z;
    v[3] += w.w;
  }
}

template <typename T, int EPI>
__global__ __launch_bounds__(NTHR, 2) void gemm_kernel(GemmArgs args) {
  __shared__ __attribute__((aligned(16))) char lds[2 * 2 * TILEB];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;

  // ---- which job: chunks of 8 blocks (one per XCD) alternate between the
  // two jobs while both have chunks left.
  const int chunk = blockIdx.x >> 3;
  const int c0 = args.chunks[0], c1 = args.njobs > 1 ? args.chunks[1] : 0;
  const int both = c0 < c1 ? c0 : c1;
  int jid, jc;
  if (chunk < 2 * both) {
    jid = chunk & 1;
    jc = chunk >> 1;
  } else {
    jid = c0 > c1 ? 0 : 1;
    jc = both + (chunk - 2 * both);
  }
  const GemmJob& p = args.job[jid];
  const int bid = jc * 8 + (blockIdx.x & 7);

  // ---- work item and N tile
  const int count = item_count(p);
  const int q = (count + 7) >> 3;
  const int nbn = n_tiles<EPI>(p);
  const int xcd = bid & 7, local = bid >> 3;
  int pi, nt;
  if (p.grouped) {
    pi = local / nbn;
    nt = local - pi * nbn;
  } else {
    nt = local / (q > 0 ? q : 1);
    pi = local - nt * q;
    if (nt >= nbn) return;
  }
  if (pi >= q) return;
  const int item = xcd * q + pi;
  if (item >= count) return;
  int e = 0, rows, row_base;
  if (p.grouped) {
    e = p.tile_e[item];
    const int m0 = p.tile_m0[item];
    rows = p.counts[e] - m0;
    row_base = p.offsets[e] + m0;
  } else {
    const int m0 = item * BM;
    rows = p.M - m0;
    row_base = m0;
  }
  rows = rows < BM ? rows : BM;

  // ---- global -> LDS assignment: thread writes 16-byte piece c16 of LDS rows
  // r0 + 32 i.  A rows past the item's end re-read its last row: MFMA row r of
  // the result depends only on A row r, and those rows are never stored.
  const int c16 = tid & 7, r0 = tid >> 3;
  const char* a_ptr[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = min(r0 + 32 * i, rows - 1);
    const long long arow = p.a_rows ? (long long)(p.a_rows[row_base + r] / p.a_div) : (long long)(row_base + r);
    a_ptr[i] = reinterpret_cast<const char*>(p.A) + (arow * p.lda) * (long long)sizeof(T) + c16 * 16;
  }
  // LDS B row rho = base + 16 ni + f holds weight row base' + S f + ni (S = 2
  // for SwiGLU halves, 4 otherwise), so lane f's MFMA columns are adjacent
  // output columns.
  const char* bbase = reinterpret_cast<const char*>(p.B) + (long long)e * p.b_estride * (long long)sizeof(T);
  const char* b_ptr[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int rho = r0 + 32 * i;
    long long brow;
    if (EPI == EPI_SWIGLU) {
      const int h = rho & 63, half = rho >> 6;            // gate block, then up block
      const int w32 = h >> 5, ni = (h >> 4) & 1, f = h & 15;
      brow = (long long)(half ? p.up_off : 0) + nt * 64 + w32 * 32 + 2 * f + ni;
    } else {
      const int w64 = rho >> 6, ni = (rho >> 4) & 3, f = rho & 15;
      brow = (long long)nt * BN + w64 * 64 + 4 * f + ni;
    }
    b_ptr[i] = bbase + brow * p.ldb * (long long)sizeof(T) + c16 * 16;
  }

  const int nk = (int)((long long)p.K * sizeof(T) / ROWB);
  // Two register sets: stage s+2 is requested while stage s is multiplied and
  // stage s+1 waits in registers for its LDS buffer.
  u32x4_t ra[2][4], rb[2][4];
  auto gload = [&](int s, u32x4_t (&da)[4], u32x4_t (&db)[4]) {
    const long long off = (long long)s * ROWB;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      da[i] = ld16(a_ptr[i] + off);
      db[i] = ld16(b_ptr[i] + off);
    }
  };
  auto lstore = [&](int buf, const u32x4_t (&da)[4], const u32x4_t (&db)[4]) {
    char* As = lds + buf * 2 * TILEB;
    char* Bs = As + TILEB;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = r0 + 32 * i;
      st16(As + swz(r, c16), da[i]);
      st16(Bs + swz(r, c16), db[i]);
    }
  };

  // ---- LDS -> MFMA operand rows for this wave (16 consecutive LDS rows per tile)
  const int fr = lane & 15, g = lane >> 4;
  int arow_l[4], brow_l[4];
#pragma unroll
  for (int mi = 0; mi < 4; ++mi) arow_l[mi] = wm * 64 + mi * 16 + fr;
#pragma unroll
  for (int ni = 0; ni < 4; ++ni) {
    if (EPI == EPI_SWIGLU)
      brow_l[ni] = (ni < 2 ? wn * 32 + ni * 16 : 64 + wn * 32 + (ni - 2) * 16) + fr;
    else
      brow_l[ni] = wn * 64 + ni * 16 + fr;
  }

  f32x4_t acc[4][4];
#pragma unroll
  for (int mi = 0; mi < 4; ++mi)
#pragma unroll
    for (int ni = 0; ni < 4; ++ni) acc[mi][ni] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  auto compute = [&](int buf) {
    const char* As = lds + buf * 2 * TILEB;
    const char* Bs = As + TILEB;
    Frag fa[4], fb[4];
#pragma unroll
    for (int mi = 0; mi < 4; ++mi) {
      fa[mi].lo = ld16(As + swz(arow_l[mi], 2 * g));
      fa[mi].hi = ld16(As + swz(arow_l[mi], 2 * g + 1));
    }
#pragma unroll
    for (int ni = 0; ni < 4; ++ni) {
      fb[ni].lo = ld16(Bs + swz(brow_l[ni], 2 * g));
      fb[ni].hi = ld16(Bs + swz(brow_l[ni], 2 * g + 1));
    }
#pragma unroll
    for (int mi = 0; mi < 4; ++mi)
#pragma unroll
      for (int ni = 0; ni < 4; ++ni) acc[mi][ni] = Mma<T>::run(fa[mi], fb[ni], acc[mi][ni]);
  };

  gload(0, ra[0], rb[0]);
  if (nk > 1) gload(1, ra[1], rb[1]);
  lstore(0, ra[0], rb[0]);
  __syncthreads();
  // Unrolled by two so that every register-set index is a constant.
  for (int s = 0; s < nk; s += 2) {
    if (s + 2 < nk) gload(s + 2, ra[0], rb[0]);
    compute(0);
    if (s + 1 < nk) lstore(1, ra[1], rb[1]);
    __syncthreads();
    if (s + 1 >= nk) break;
    if (s + 3 < nk) gload(s + 3, ra[1], rb[1]);
    compute(1);
    if (s + 2 < nk) lstore(0, ra[0], rb[0]);
    __syncthreads();
  }

  // ---- epilogue.  acc[mi][ni][i] is row wm*64 + mi*16 + 4g + i; its column
  // is 2f + ni (SwiGLU, ni < 2 gate / ni >= 2 the matching up) or 4f + ni
  // past the wave's column base.
  T* C = reinterpret_cast<T*>(p.C);
  T* aux = reinterpret_cast<T*>(p.aux);
#pragma unroll
  for (int mi = 0; mi < 4; ++mi) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int lr = wm * 64 + mi * 16 + 4 * g + i;
      if (lr >= rows) continue;
      const long long row = row_base + lr;
      if (EPI == EPI_SWIGLU) {
        const int f = nt * 64 + wn * 32 + 2 * fr;
        float h[2], a[2], u[2];
#pragma unroll
        for (int ni = 0; ni < 2; ++ni) {
          a[ni] = acc[mi][ni][i];
          u[ni] = acc[mi][ni + 2][i];
          h[ni] = siluf_(a[ni]) * u[ni];
        }
        store_vec<T, 2>(C + row * p.ldc + f, h);
        if (aux) {
          store_vec<T, 2>(aux + row * p.ldaux + f, a);
          store_vec<T, 2>(aux + row * p.ldaux + p.N + f, u);
        }
      } else if (EPI == EPI_ROWSCALE) {
        const int n = nt * BN + wn * 64 + 4 * fr;
        const float sc = p.gate[p.perm[row]];
        float v[4], raw[4];
#pragma unroll
        for (int ni = 0; ni < 4; ++ni) {
          raw[ni] = acc[mi][ni][i];
          v[ni] = raw[ni] * sc;
        }
        store_vec<T, 4>(C + row * p.ldc + n, v);
        if (aux) store_vec<T, 4>(aux + row * p.ldaux + n, raw);
      } else {  // EPI_COMBINE: row is a token
        const int n = nt * BN + wn * 64 + 4 * fr;
        const T* O = reinterpret_cast<const T*>(p.O);
        float v[4];
#pragma unroll
        for (int ni = 0; ni < 4; ++ni) v[ni] = acc[mi][ni][i];
        for (int j = 0; j < p.k; ++j) load_add4<T>(O + (long long)p.pos[row * p.k + j] * p.ldo + n, v);
        store_vec<T, 4>(C + row * p.ldc + n, v);
      }
    }
  }
}

int job_chunks(const GemmJob& j, int epi) {
  const int nbn = epi == EPI_SWIGLU ? j.N / 64 : j.N / BN;
  const long long groups = (j.max_items + 7) / 8;
  return (int)(groups * nbn);
}

template <typename T>
void launch_dtype(GemmArgs a, hipStream_t s) {
  long long total = 0;
  for (int i = 0; i < a.njobs; ++i) {
    a.chunks[i] = job_chunks(a.job[i], a.epi);
    total += a.chunks[i];
  }
  if (total == 0) return;
  const dim3 grid((unsigned)(total * 8));
  switch (a.epi) {
    case EPI_SWIGLU: hipLaunchKernelGGL((gemm_kernel<T, EPI_SWIGLU>), grid, dim3(NTHR), 0, s, a); break;
    case EPI_ROWSCALE: hipLaunchKernelGGL((gemm_kernel<T, EPI_ROWSCALE>), grid, dim3(NTHR), 0, s, a); break;
    default: hipLaunchKernelGGL((gemm_kernel<T, EPI_COMBINE>), grid, dim3(NTHR), 0, s, a); break;
  }
}

}  // namespace

void launch_gemm(const GemmArgs& a, hipStream_t s) {
  if (a.act == 1) launch_dtype<bf16_t>(a, s);
  else launch_dtype<float>(a, s);
}

}  // namespace fgmoe
