// Expert GEMMs of the MoE layer on gfx950 MFMA, with fused epilogues.
//
// One kernel template serves the four GEMMs of the forward:
//   routed gate/up  (grouped over experts, A rows gathered from x through the
//                    dispatch order, SwiGLU epilogue -> H)
//   routed down     (grouped, rows scaled by their routing weight -> O)
//   shared gate/up  (dense, SwiGLU epilogue -> Hs)
//   shared down     (dense, plain store -> S)
// The experts are the SwiGLU FFNs of widths 512 (routed) and 2048 (shared) of
// the seventnews article "A relay race of rented GPUs trained NanoColibri's
// 2.7B MoE for $200" (opening section, architecture paragraph).  A launch
// carries two jobs with the same B layout (the two gate/up GEMMs, or the two
// down GEMMs): their workgroups are interleaved, so the weight-streaming
// routed tiles and the MFMA-bound shared tiles share the chip.
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
#ifndef FGMOE_GEMM_ROWB
#define FGMOE_GEMM_ROWB 128
#endif
#ifndef FGMOE_GEMM_STAGES
#define FGMOE_GEMM_STAGES 2
#endif
constexpr int kRowB = FGMOE_GEMM_ROWB;       // bytes of one operand row per K stage (64 or 128)
constexpr int kStages = FGMOE_GEMM_STAGES;   // LDS ring depth: kStages * 2 * 128 * kRowB bytes

// LDS swizzle of 16-byte pieces.  gfx950 serves a 16-byte-per-lane LDS read
// 32 lanes at a time over 128 four-byte banks (fitted to measured
// SQ_LDS_BANK_CONFLICT counts of probe access patterns).  An MFMA operand read
// has 16 consecutive rows x 2 piece indices per half-wave; these XORs make
// those 32 pieces hit 32 distinct bank groups.
template <int ROWB>
__device__ __forceinline__ int swz_piece(int row, int piece) {
  if constexpr (ROWB == 128) return piece ^ (row & 7) ^ ((row >> 3) & 1);
  else return piece ^ (((row >> 3) & 1) << 1);
}
template <int ROWB>
__device__ __forceinline__ int swz(int row, int piece) {
  return row * ROWB + (swz_piece<ROWB>(row, piece) << 4);
}

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

__device__ __host__ __forceinline__ int n_tiles(const GemmJob& j) {
  return j.epi == EPI_SWIGLU ? j.N / 64 : j.N / BN;
}
__device__ __forceinline__ int item_count(const GemmJob& j) {
  if (j.kgroup) return j.nexp * ((j.M + BM - 1) / BM);
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
__device__ __forceinline__ void load_vec4(const T* p, float (&v)[4]) {
  if constexpr (sizeof(T) == 2) {
    const uint2 w = *reinterpret_cast<const uint2*>(p);
    v[0] = bf16_to_f32((bf16_t)(w.x & 0xFFFF));
    v[1] = bf16_to_f32((bf16_t)(w.x >> 16));
    v[2] = bf16_to_f32((bf16_t)(w.y & 0xFFFF));
    v[3] = bf16_to_f32((bf16_t)(w.y >> 16));
  } else {
    const float4 w = *reinterpret_cast<const float4*>(p);
    v[0] = w.x;
    v[1] = w.y;
    v[2] = w.z;
    v[3] = w.w;
  }
}

template <typename T, bool SWIGLU, int NS>
__global__ __launch_bounds__(NTHR, 2) void gemm_kernel(GemmArgs args) {
  constexpr int EPI = SWIGLU ? EPI_SWIGLU : EPI_ROWSCALE;   // B-row layout class
  // (the row width is a namespace constant: as a kernel template parameter it
  // made this compiler drop the host-side launch stubs)
  constexpr int ROWB = kRowB;
  constexpr int TILEB = BM * ROWB;                          // one operand tile of one stage
  constexpr int PIECES = ROWB / 16;                         // 16-byte pieces per row and stage
  constexpr int ROWS_PER_DMA = 1024 / ROWB;                 // LDS rows one wave instruction fills
  constexpr int NDMA = 32 / ROWS_PER_DMA;                   // instructions per wave per operand
  __shared__ __attribute__((aligned(16))) char lds[NS * 2 * TILEB];

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
  const int nbn = n_tiles(p);
  const int xcd = bid & 7, local = bid >> 3;
  int pi, nt;
  if (p.grouped || p.kgroup) {
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
  long long kofs = 0;
  int klen = p.K;
  if (p.kgroup) {
    const int mt = (p.M + BM - 1) / BM;
    e = item / mt;
    const int m0 = (item - e * mt) * BM;
    rows = p.M - m0;
    row_base = m0;
    kofs = p.kofs[e];
    klen = p.klen[e];
  } else if (p.grouped) {
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

  // ---- global -> LDS: direct loads (global_load_lds_dwordx4).  Lane i of a
  // wave instruction lands at LDS byte base + 16 i, so instruction j of wave w
  // fills LDS rows w*32 + j*ROWS_PER_DMA + i/PIECES at physical piece
  // i%PIECES; the lane fetches the logical piece the swizzle puts there.  A
  // rows past the item's end re-read its last row: MFMA row r of the result
  // depends only on A row r, and those rows are never stored.
  const int prow = lane / PIECES, ppc = lane % PIECES;
  const char* a_src[NDMA];
  const char* b_src[NDMA];
  const char* bbase = reinterpret_cast<const char*>(p.B) + (long long)e * p.b_estride * (long long)sizeof(T);
#pragma unroll
  for (int j = 0; j < NDMA; ++j) {
    const int R = wave * 32 + j * ROWS_PER_DMA + prow;
    const int c = swz_piece<ROWB>(R, ppc);            // XOR swizzles are their own inverse
    const int ra = min(R, rows - 1);
    const long long arow = p.a_rows ? (long long)(p.a_rows[row_base + ra] / p.a_div) : (long long)(row_base + ra);
    a_src[j] = reinterpret_cast<const char*>(p.A) + (arow * p.lda + kofs) * (long long)sizeof(T) + c * 16;
    // LDS B row rho = base + 16 ni + f holds weight row base' + S f + ni (S = 2
    // for SwiGLU halves, 4 otherwise), so lane f's MFMA columns are adjacent
    // output columns.
    long long brow;
    if (EPI == EPI_SWIGLU) {
      const int h = R & 63, half = R >> 6;           // gate block, then up block
      const int w32 = h >> 5, ni = (h >> 4) & 1, f = h & 15;
      brow = (long long)(half ? p.up_off : 0) + nt * 64 + w32 * 32 + 2 * f + ni;
    } else {
      const int w64 = R >> 6, ni = (R >> 4) & 3, f = R & 15;
      brow = (long long)nt * BN + w64 * 64 + 4 * f + ni;
    }
    b_src[j] = bbase + (brow * p.ldb + kofs) * (long long)sizeof(T) + c * 16;
  }

  const int nk = (int)((long long)klen * sizeof(T) / ROWB);
  // Stage s lives in LDS buffer s % NS; NS - 1 stages are in flight while one
  // is multiplied.  A stage is 2 * NDMA loads per lane.
  auto issue = [&](int s) {
    char* base = lds + (s % NS) * 2 * TILEB + wave * 32 * ROWB;
    const long long off = (long long)s * ROWB;
#pragma unroll
    for (int j = 0; j < NDMA; ++j)
      __builtin_amdgcn_global_load_lds(a_src[j] + off, (lds_ptr_t)(base + j * 1024), 16, 0, 0);
#pragma unroll
    for (int j = 0; j < NDMA; ++j)
      __builtin_amdgcn_global_load_lds(b_src[j] + off, (lds_ptr_t)(base + TILEB + j * 1024), 16, 0, 0);
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
    if constexpr (ROWB == 128) {
      Frag fa[4], fb[4];
#pragma unroll
      for (int mi = 0; mi < 4; ++mi) {
        fa[mi].lo = ld16(As + swz<ROWB>(arow_l[mi], 2 * g));
        fa[mi].hi = ld16(As + swz<ROWB>(arow_l[mi], 2 * g + 1));
      }
#pragma unroll
      for (int ni = 0; ni < 4; ++ni) {
        fb[ni].lo = ld16(Bs + swz<ROWB>(brow_l[ni], 2 * g));
        fb[ni].hi = ld16(Bs + swz<ROWB>(brow_l[ni], 2 * g + 1));
      }
#pragma unroll
      for (int mi = 0; mi < 4; ++mi)
#pragma unroll
        for (int ni = 0; ni < 4; ++ni) acc[mi][ni] = Mma<T>::run(fa[mi], fb[ni], acc[mi][ni]);
    } else {
      u32x4_t fa[4], fb[4];
#pragma unroll
      for (int mi = 0; mi < 4; ++mi) fa[mi] = ld16(As + swz<ROWB>(arow_l[mi], g));
#pragma unroll
      for (int ni = 0; ni < 4; ++ni) fb[ni] = ld16(Bs + swz<ROWB>(brow_l[ni], g));
#pragma unroll
      for (int mi = 0; mi < 4; ++mi)
#pragma unroll
        for (int ni = 0; ni < 4; ++ni) acc[mi][ni] = Mma<T>::run1(fa[mi], fb[ni], acc[mi][ni]);
    }
  };

  for (int s = 0; s < NS - 1 && s < nk; ++s) issue(s);
  for (int s = 0; s < nk; ++s) {
    // This wave's loads of stage s are done once at most the later stages'
    // loads are outstanding; the barrier then covers every wave's loads and
    // every wave's reads of the buffer about to be refilled.
    if (s + NS - 2 < nk) wait_vmcnt<2 * NDMA * (NS - 2)>();
    else wait_vmcnt<0>();
    block_barrier();
    if (s + NS - 1 < nk) issue(s + NS - 1);
    compute(s % NS);
  }

  // ---- epilogue (per job).  acc[mi][ni][i] is row wm*64 + mi*16 + 4g + i; its column
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
      } else if (p.epi == EPI_ROWSCALE) {
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
      } else if (p.epi == EPI_SWIGLU_BWD) {
        // SwiGLU backward: dH = s * acc, then (da, du) from the saved (a, u)
        const int n = nt * BN + wn * 64 + 4 * fr;
        const float sc = p.gate ? p.gate[p.perm[row]] : 1.f;
        const T* au = reinterpret_cast<const T*>(p.aux) + row * p.ldaux;
        float a[4], u[4], da[4], du[4];
        load_vec4<T>(au + n, a);
        load_vec4<T>(au + p.N + n, u);
#pragma unroll
        for (int ni = 0; ni < 4; ++ni) {
          const float dh = acc[mi][ni][i] * sc;
          const float sg = sigmoidf_(a[ni]);
          const float si = a[ni] * sg;
          da[ni] = dh * u[ni] * (sg * (1.f + a[ni] * (1.f - sg)));
          du[ni] = dh * si;
        }
        store_vec<T, 4>(C + row * p.ldc + n, da);
        store_vec<T, 4>(C + row * p.ldc + p.N + n, du);
      } else if (p.epi == EPI_STORE_F32) {
        const int n = nt * BN + wn * 64 + 4 * fr;
        float v[4];
#pragma unroll
        for (int ni = 0; ni < 4; ++ni) v[ni] = acc[mi][ni][i];
        float* Cf = reinterpret_cast<float*>(p.C) + (long long)e * p.c_estride;
        store_vec<float, 4>(Cf + row * p.ldc + n, v);
      } else {  // EPI_STORE
        const int n = nt * BN + wn * 64 + 4 * fr;
        float v[4];
#pragma unroll
        for (int ni = 0; ni < 4; ++ni) v[ni] = acc[mi][ni][i];
        store_vec<T, 4>(C + row * p.ldc + n, v);
      }
    }
  }
}

int job_chunks(const GemmJob& j) {
  const int nbn = n_tiles(j);
  const long long groups = (j.max_items + 7) / 8;
  return (int)(groups * nbn);
}

template <typename T>
void launch_dtype(GemmArgs a, hipStream_t s) {
  long long total = 0;
  for (int i = 0; i < a.njobs; ++i) {
    a.chunks[i] = job_chunks(a.job[i]);
    total += a.chunks[i];
  }
  if (total == 0) return;
  const dim3 grid((unsigned)(total * 8));
  if (a.job[0].epi == EPI_SWIGLU)
    hipLaunchKernelGGL((gemm_kernel<T, true, kStages>), grid, dim3(NTHR), 0, s, a);
  else
    hipLaunchKernelGGL((gemm_kernel<T, false, kStages>), grid, dim3(NTHR), 0, s, a);
}

}  // namespace

void launch_gemm(const GemmArgs& a, hipStream_t s) {
  if (a.act == 1) launch_dtype<bf16_t>(a, s);
  else launch_dtype<float>(a, s);
}

}  // namespace fgmoe
