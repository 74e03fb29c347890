// Expert GEMMs of the MoE layer on gfx950 MFMA, with fused epilogues.
//
// One kernel serves the GEMMs of the forward and of the backward:
//   routed gate/up  (grouped over experts, A rows gathered from x through the
//                    dispatch order, SwiGLU epilogue -> H)
//   routed down     (grouped, rows scaled by their routing weight -> O)
//   shared gate/up  (dense, SwiGLU epilogue -> Hs)
//   shared down     (dense, plain store -> S)
//   backward: SwiGLU-backward epilogue, plain stores, and fp32 weight
//   gradients contracting over each expert's own slot range.
// The experts are the SwiGLU FFNs of widths 512 (routed) and 2048 (shared) of
// the seventnews article "A relay race of rented GPUs trained NanoColibri's
// 2.7B MoE for $200" (opening section, architecture paragraph).  A launch
// carries up to two jobs with the same B layout (the two gate/up GEMMs, or the
// two down GEMMs): their workgroups are interleaved, so the weight-streaming
// routed tiles and the MFMA-bound shared tiles share the chip.
//
// Workgroup: 4 waves (2 x 2), two workgroups per CU.  Every wave owns a
// 64 x 128 piece of a 128 x 256 output tile (4 x 8 MFMA 16x16x32 tiles).  K
// advances in 64-byte row chunks through a 3-deep LDS ring (24 KiB stages:
// the tile's 128 A rows then its 256 B rows) filled by direct global->LDS
// loads (global_load_lds_dwordx4), each wave loading a quarter of a stage.
// Measured on gfx950: a CU's address unit takes global->LDS loads at about
// 64 bytes per clock, so a 128 x 128 x 32 step (16 KiB per MFMA-MFLOP) would
// need all of it to keep the MFMA pipes busy, 128 x 256 about three
// quarters; and a wave that issues its stage's loads as one burst stalls
// behind the other waves' loads for about as long as its MFMAs take, so the
// loads of the next stage but one are spread between the current stage's
// MFMAs instead.
//
// The 16-byte pieces of each LDS row are XOR-swizzled (see swz) so that the
// 16-row operand reads are free of bank conflicts.  B rows are permuted on
// their way into LDS so that each lane's output columns are adjacent and the
// epilogue writes 8- to 32-byte vectors.  Rows past an item's end re-read its
// last row and columns past N re-read row N - 1; neither is stored.
//
// Scheduling: work items are 128-row tiles (dense: row blocks; grouped: the
// tile table the router wrote, in expert order).  Workgroups are
// dealt to the 8 XCDs round-robin by block index, so block b runs on XCD
// b % 8; XCD x gets the contiguous item range [x*q, (x+1)*q).  Grouped jobs
// run all N tiles of an item back to back (an expert's weights and an item's
// rows stay in that XCD's L2); dense jobs run all of the XCD's row blocks for
// one N tile before the next.  No host synchronisation: the item count of a
// grouped job is read on the device.
#include <type_traits>

#include "gemm_tile.h"

namespace fgmoe {

namespace {

constexpr int NTHR = 256;                    // 4 waves
constexpr int BM = 128, BN = 256;            // workgroup tile
constexpr int WM = 64, WN = 128, NI = WN / 16, HN = NI / 2;   // one wave's output piece
constexpr int kStages = 3;                   // LDS ring depth
constexpr int ATILE = BM * kRowB, BTILE = BN * kRowB;        // one stage of each operand
constexpr int kStageBytes = ATILE + BTILE;
constexpr int NDA = BM / 4 / 16, NDB = BN / 4 / 16;          // loads per wave and stage: A 2, B 4
constexpr int kLoads = NDA + NDB;

// SwiGLU tiles hold BN / 2 gate and the matching BN / 2 up rows of B.
__device__ __host__ __forceinline__ int n_tiles(const GemmJob& j) {
  const int w = j.epi == EPI_SWIGLU ? BN / 2 : BN;
  return (j.N + w - 1) / w;
}
__device__ __forceinline__ int item_count(const GemmJob& j) {
  if (j.kgroup) return j.nexp * ((j.M + BM - 1) / BM);
  return j.grouped ? *j.tile_count : (j.M + BM - 1) / BM;
}
// Upper bound of item_count, on the host.
inline long long max_item_count(const GemmJob& j) {
  if (j.kgroup) return (long long)j.nexp * ((j.M + BM - 1) / BM);
  return j.grouped ? j.max_items : (j.M + BM - 1) / BM;
}

template <typename T, bool SWIGLU>
__global__ __launch_bounds__(NTHR, 2) void gemm_kernel(GemmArgs args) {
  // One LDS object (the ring, then the row scales): with a second __shared__
  // array the compiler could no longer tell which LDS reads the direct loads
  // feed and waited for every load in flight before each stage.
  __shared__ __attribute__((aligned(16))) char lds[kStages * kStageBytes + BM * 4];
  float* const row_scale = reinterpret_cast<float*>(lds + kStages * kStageBytes);

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;

  // ---- which job
  int jid, bid;
  select_job(args, blockIdx.x, jid, bid);
  const GemmJob& p = args.job[jid];

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

  // Row scales of the gate-scaled epilogues: thread r < 128 fetches perm of
  // row r now (it lands with the first stage), the gate itself after the
  // main loop, and the scales reach the waves through LDS.
  const bool scaled = p.gate != nullptr && (p.epi == EPI_ROWSCALE || p.epi == EPI_SWIGLU_BWD);
  int my_perm = 0;
  if (scaled && tid < BM) my_perm = p.perm[row_base + min(tid, rows - 1)];

  // ---- global -> LDS.  A stage holds the A tile (128 rows) then the B tile
  // (256 rows).  Lane i of a wave instruction lands at LDS byte base + 16 i,
  // so A load j of wave w fills A rows 32w + 16j + i/4 and B load j fills B
  // rows 64w + 16j + i/4, at physical piece i%4; the lane fetches the logical
  // piece the swizzle puts there.  LDS B row wn*128 + ni*16 + f holds output
  // column (tile base) + wn*128 + 8f + ni, so lane f's MFMA columns are 8
  // adjacent output columns; for SwiGLU the first 128 B rows are gate rows
  // and the next 128 the matching up rows, with h column (tile base) +
  // wn*64 + 4f + ni.
  const char* a_src[NDA];
  const char* b_src[NDB];
  const char* bbase = reinterpret_cast<const char*>(p.B) + (long long)e * p.b_estride * (long long)sizeof(T);
#pragma unroll
  for (int j = 0; j < NDA; ++j) {
    const int R = wave * (BM / 4) + j * 16 + (lane >> 2);
    const int c = swz_piece(R, lane & 3);            // XOR swizzles are their own inverse
    const int ra = min(R, rows - 1);
    const long long arow = p.a_rows ? (long long)(p.a_rows[row_base + ra] / p.a_div) : (long long)(row_base + ra);
    a_src[j] = reinterpret_cast<const char*>(p.A) + (arow * p.lda + kofs) * (long long)sizeof(T) + c * 16;
  }
#pragma unroll
  for (int j = 0; j < NDB; ++j) {
    const int R = wave * (BN / 4) + j * 16 + (lane >> 2);
    const int c = swz_piece(R, lane & 3);
    long long brow;
    if (SWIGLU) {
      const int half = R >> 7, h = R & 127;
      const int w = h >> 6, ni = (h >> 4) & 3, f = h & 15;
      const int col = min(nt * (BN / 2) + w * 64 + 4 * f + ni, p.N - 1);
      brow = (long long)(half ? p.up_off : 0) + col;
    } else {
      const int w = R >> 7, ni = (R >> 4) & 7, f = R & 15;
      brow = min(nt * BN + w * 128 + 8 * f + ni, p.N - 1);
    }
    b_src[j] = bbase + (brow * p.ldb + kofs) * (long long)sizeof(T) + c * 16;
  }
  const int nk = (int)((long long)klen * sizeof(T) / kRowB);
  // load j of this wave for stage s (j < NDA: A, else B)
  auto issue_one = [&](int s, int j) {
    char* st = lds + (s % kStages) * kStageBytes;
    const long long off = (long long)s * kRowB;
    if (j < NDA)
      __builtin_amdgcn_global_load_lds(a_src[j] + off, (lds_ptr_t)(st + wave * (BM / 4) * kRowB + j * 1024), 16, 0, 0);
    else
      __builtin_amdgcn_global_load_lds(b_src[j - NDA] + off,
                                       (lds_ptr_t)(st + ATILE + wave * (BN / 4) * kRowB + (j - NDA) * 1024), 16, 0, 0);
  };
  auto issue = [&](int s) {
#pragma unroll
    for (int j = 0; j < kLoads; ++j) issue_one(s, j);
  };

  // ---- LDS -> MFMA operand rows of this wave (16 consecutive LDS rows per tile)
  const int fr = lane & 15, g = lane >> 4;
  int arow_l[4], brow_l[NI];
#pragma unroll
  for (int mi = 0; mi < 4; ++mi) arow_l[mi] = wm * WM + mi * 16 + fr;
#pragma unroll
  for (int ni = 0; ni < NI; ++ni)
    brow_l[ni] = (SWIGLU ? (ni < HN ? wn * 64 + ni * 16 : BN / 2 + wn * 64 + (ni - HN) * 16) : wn * WN + ni * 16) + fr;

  f32x4_t acc[4][NI];
#pragma unroll
  for (int mi = 0; mi < 4; ++mi)
#pragma unroll
    for (int ni = 0; ni < NI; ++ni) acc[mi][ni] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // One stage: lane group g owns 16-byte piece g of each 64-byte row chunk
  // (the same for both operands, so the products pair up whatever the order
  // of K inside).  With loads, this wave's loads of stage snext go after
  // MFMAs 4, 9, 14, 19, 24 and 29.
  constexpr int SP = 4 * NI / kLoads;                      // MFMAs between two loads (5)
  auto compute = [&](int s, int snext, auto with_loads) {
    const char* As = lds + (s % kStages) * kStageBytes;
    const char* Bs = As + ATILE;
    u32x4_t fa[4], fb[NI];
#pragma unroll
    for (int mi = 0; mi < 4; ++mi) fa[mi] = ld16(As + swz(arow_l[mi], g));
#pragma unroll
    for (int ni = 0; ni < NI; ++ni) fb[ni] = ld16(Bs + swz(brow_l[ni], g));
#pragma unroll
    for (int mi = 0; mi < 4; ++mi)
#pragma unroll
      for (int ni = 0; ni < NI; ++ni) {
        acc[mi][ni] = Mma<T>::run1(fa[mi], fb[ni], acc[mi][ni]);
        if constexpr (decltype(with_loads)::value) {
          const int qq = mi * NI + ni;
          if (qq % SP == SP - 1 && qq / SP < kLoads) {
            issue_one(snext, qq / SP);
            __builtin_amdgcn_sched_barrier(0);   // keep the loads spread out
          }
        }
      }
  };

  // ---- main loop.  Stage s is waited for with the next stage's loads still
  // in flight; the barrier then covers every wave's loads of stage s and
  // every wave's reads of stage s-1, whose buffer stage s+2 refills.  The
  // last two stages have nothing left to load.
  for (int s = 0; s < kStages - 1 && s < nk; ++s) issue(s);
  int s = 0;
  for (; s + kStages - 1 < nk; ++s) {
    wait_vmcnt<kLoads>();
    block_barrier();
    compute(s, s + kStages - 1, std::true_type{});
  }
  for (; s < nk; ++s) {
    if (s + 1 < nk) wait_vmcnt<kLoads>();
    else wait_vmcnt<0>();
    block_barrier();
    compute(s, 0, std::false_type{});
  }

  if (scaled) {
    if (tid < BM) row_scale[tid] = p.gate[my_perm];
    __syncthreads();
  }
  // ---- epilogue (per job).  acc[mi][ni][i] is tile row wm*64 + mi*16 + 4g + i.
  // Its column, past the wave's base, is 8f + ni (f = lane % 16); for SwiGLU,
  // blocks ni < 4 are gate columns 4f + ni and ni >= 4 the matching up.
  T* C = reinterpret_cast<T*>(p.C);
  T* aux = reinterpret_cast<T*>(p.aux);
  const int n = nt * BN + wn * WN + NI * fr;               // first column of this lane (not SwiGLU)
  const int fh = nt * (BN / 2) + wn * (WN / 2) + HN * fr;  // first h column of this lane (SwiGLU)
  if (SWIGLU ? fh >= p.N : n >= p.N) return;
#pragma unroll
  for (int mi = 0; mi < 4; ++mi) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int lr = wm * WM + mi * 16 + 4 * g + i;
      if (lr >= rows) continue;
      const long long row = row_base + lr;
      if (SWIGLU) {
        float h[HN], a[HN], u[HN];
#pragma unroll
        for (int ni = 0; ni < HN; ++ni) {
          a[ni] = acc[mi][ni][i];
          u[ni] = acc[mi][ni + HN][i];
          h[ni] = siluf_(a[ni]) * u[ni];
        }
        store_vec<T, HN>(C + row * p.ldc + fh, h);
        if (aux) {
          store_vec<T, HN>(aux + row * p.ldaux + fh, a);
          store_vec<T, HN>(aux + row * p.ldaux + p.N + fh, u);
        }
      } else if (p.epi == EPI_ROWSCALE) {
        const float sc = row_scale[lr];
        float v[NI], raw[NI];
#pragma unroll
        for (int ni = 0; ni < NI; ++ni) {
          raw[ni] = acc[mi][ni][i];
          v[ni] = raw[ni] * sc;
        }
        store_vec<T, NI>(C + row * p.ldc + n, v);
        if (aux) store_vec<T, NI>(aux + row * p.ldaux + n, raw);
      } else if (p.epi == EPI_SWIGLU_BWD) {
        // SwiGLU backward: dH = s * acc, then (da, du) from the saved (a, u)
        const float sc = p.gate ? row_scale[lr] : 1.f;
        const T* au = reinterpret_cast<const T*>(p.aux) + row * p.ldaux;
        float a[NI], u[NI], da[NI], du[NI];
        load_vec<T, NI>(au + n, a);
        load_vec<T, NI>(au + p.N + n, u);
#pragma unroll
        for (int ni = 0; ni < NI; ++ni) {
          const float dh = acc[mi][ni][i] * sc;
          const float sg = sigmoidf_(a[ni]);
          const float si = a[ni] * sg;
          da[ni] = dh * u[ni] * (sg * (1.f + a[ni] * (1.f - sg)));
          du[ni] = dh * si;
        }
        store_vec<T, NI>(C + row * p.ldc + n, da);
        store_vec<T, NI>(C + row * p.ldc + p.N + n, du);
      } else if (p.epi == EPI_STORE_F32) {
        float v[NI];
#pragma unroll
        for (int ni = 0; ni < NI; ++ni) v[ni] = acc[mi][ni][i];
        float* Cf = reinterpret_cast<float*>(p.C) + (long long)e * p.c_estride;
        store_vec<float, NI>(Cf + row * p.ldc + n, v);
      } else {  // EPI_STORE
        float v[NI];
#pragma unroll
        for (int ni = 0; ni < NI; ++ni) v[ni] = acc[mi][ni][i];
        store_vec<T, NI>(C + row * p.ldc + n, v);
      }
    }
  }
}

int job_chunks(const GemmJob& j) {
  const int nbn = n_tiles(j);
  const long long groups = (max_item_count(j) + 7) / 8;
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
    hipLaunchKernelGGL((gemm_kernel<T, true>), grid, dim3(NTHR), 0, s, a);
  else
    hipLaunchKernelGGL((gemm_kernel<T, false>), grid, dim3(NTHR), 0, s, a);
}

}  // namespace

void launch_gemm(const GemmArgs& a, hipStream_t s) {
  if (a.act == 1) launch_dtype<bf16_t>(a, s);
  else launch_dtype<float>(a, s);
}

}  // namespace fgmoe
