// Expert GEMMs of the MoE layer in bf16 on gfx950 MFMA: 256 x 256 output
// tiles, one workgroup of 8 waves per CU.
//
// The two forward launches of a bf16 layer run here:
//   gate/up: routed (grouped over experts, A rows gathered from x through the
//            dispatch order) + shared (dense), SwiGLU epilogue -> H, Hs
//   down:    routed (grouped, rows scaled by their routing weight) + shared
//            (dense, two contraction slices, plain store) -> O, S
// and the two input-gradient launches of the backward:
//   dH:      routed (A rows of dy gathered, rows scaled by their gate) +
//            shared, SwiGLU-backward epilogue -> dA|dU, dAs|dUs
//   dX:      routed + shared, plain store -> dXp, dXs
// The experts are the SwiGLU FFNs of widths 512 (routed) and 2048 (shared) of
// the seventnews article "A relay race of rented GPUs trained NanoColibri's
// 2.7B MoE for $200" (opening section, architecture paragraph).
//
// Why a second tile shape next to gemm.hip's 128 x 256 pair of workgroups:
// a CU's operand traffic per MFMA flop falls by a third (32 KiB per 4.2 MFLOP
// of K step instead of 2 x 24 KiB per 2 x 2.1 MFLOP), which is the resource
// that bounds the smaller tiles.  A grouped item is
// up to 256 rows of one expert, so an expert of up to 256 rows streams its
// weights once; the waves whose 64-row band lies past the item's rows skip
// their operand reads and MFMAs (they still load their share of the stage).
//
// Workgroup: 8 waves (4 x 2), each owning a 64 x 128 piece (4 x 8 MFMA
// 16x16x32 tiles).  K advances in 64-byte row chunks through a 5-deep LDS
// ring of 32 KiB stages (256 A rows, then 256 B rows; 160 KiB, all of a
// CU's LDS), filled by direct global->LDS loads (global_load_lds_dwordx4)
// spread between the MFMAs; a stage's loads have three K steps to land.
// Measured on gfx950 with per-workgroup clock stamps: with the operands read
// from LDS right after each K step's barrier, the MFMA pipes waited about a
// third of the loop for those reads; here each K step's MFMAs run from
// registers while the next step's operands are read behind them.  The LDS
// rows are XOR-swizzled (swz) and B rows permuted so that each lane's output
// columns are adjacent, as in gemm.hip.
//
// Scheduling.  Items are 256-row tiles (dense: row blocks, times the
// contraction slices of a split dense job; grouped: the 256-row tile table
// the router wrote).  Block b runs on XCD b % 8.  Grouped jobs: XCD x gets
// the contiguous item range [x*q, (x+1)*q) and runs all N tiles of an item
// back to back (an expert's weights are read once); so do dense jobs with
// xcd_cols = -1 (an item's A rows are read once).  Other dense jobs: the XCDs
// split the (row block, N tile) grid into an (8 / gc) x gc grid of ranges,
// gc chosen by the caller so that the L2 misses of the two operands,
// (M rows x gc + N rows x 8 / gc) x K, are smallest; measured with
// FETCH_SIZE, gc = 1 on the 4096-token shared gate/up fetched the 8 MiB
// weight matrix once per XCD.
#include <algorithm>
#include <type_traits>

#include "gemm_tile.h"

namespace fgmoe {

namespace {

constexpr int NTHR = 512;                    // 8 waves
constexpr int BM = kTileMFwd, BN = 256;      // workgroup tile
constexpr int WM = 64;                       // rows of one wave's output piece
constexpr int kStages = 5;                   // LDS ring depth (5 x 32 KiB: all of a CU's LDS)
constexpr int ATILE = BM * kRowB, BTILE = BN * kRowB;        // one stage of each operand
constexpr int kStageBytes = ATILE + BTILE;
constexpr int NDA = BM / 8 / 16, NDB = BN / 8 / 16;          // loads per wave and stage: A 2, B 2
constexpr int kLoads = NDA + NDB;
static_assert(BM == 256, "the wave layout covers 256 rows");

__device__ __host__ __forceinline__ int n_tiles(const GemmJob& j) {
  const int w = j.epi == EPI_SWIGLU ? BN / 2 : BN;
  return (j.N + w - 1) / w;
}
// The weight row that LDS B row R of N tile nt holds (before clamping to the
// last row): SwiGLU tiles put 128 gate rows, then the matching 128 up rows,
// ordered so that each lane's output columns are adjacent; other tiles 256
// rows in the same interleaved order.  The stage-major layout stores rows in
// this LDS order.
__device__ __host__ __forceinline__ long long b_tile_row(bool swiglu, int R, int nt, int up_off) {
  if (swiglu) {
    const int half = R >> 7, h = R & 127;
    const int w = h >> 6, ni = (h >> 4) & 3, f = h & 15;
    return (long long)(half ? up_off : 0) + nt * (BN / 2) + w * 64 + 4 * f + ni;
  }
  const int w = R >> 7, ni = (R >> 4) & 7, f = R & 15;
  return (long long)nt * BN + w * 128 + 8 * f + ni;
}
// 8 int4 codes (one 32-bit word, element 2i in the low nibble of byte i),
// each times its row's scale and rounded once to bf16, in MFMA operand order:
// the same bits as the int4 prefill's separate dequantisation.
__device__ __forceinline__ u32x4_t dq_int4x8(uint32_t w, float sc) {
  u32x4_t r;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const float lo = (float)(((int)(w << (28 - 8 * j))) >> 28);
    const float hi = (float)(((int)(w << (24 - 8 * j))) >> 28);
    r[j] = pack_bf16x2(lo * sc, hi * sc);
  }
  return r;
}
// Segment swizzle of K-major stage rows (see the K-major loader).
__device__ __forceinline__ int ksw(int r) { return (((r >> 3) & 3) << 2) | (r & 3); }
typedef int i32x4_t __attribute__((ext_vector_type(4)));
// Four consecutive int32 of a read-only table at a wave-uniform address:
// through the constant address space the compiler emits a scalar load and
// tracks its completion itself.
typedef const __attribute__((address_space(4))) i32x4_t __attribute__((aligned(4)))* const_i32x4_ptr;
__device__ __forceinline__ i32x4_t sload4(const int32_t* q) {
  const unsigned long long a = (unsigned long long)q;
  const unsigned lo = __builtin_amdgcn_readfirstlane((unsigned)a), hi = __builtin_amdgcn_readfirstlane((unsigned)(a >> 32));
  return *reinterpret_cast<const_i32x4_ptr>(((unsigned long long)hi << 32) | lo);
}

// One K-major MFMA fragment: two transposing 8-byte LDS reads, 4 K rows
// apart.  Issued as inline asm: the compiler's builtin for this read makes
// it wait for every direct-to-LDS load in flight first (it cannot tell them
// apart), which would drain the load pipeline at each fragment.  The
// compiler does not see these reads either, so the results are used only
// after lds_wait_frags, and this relies on each read writing straight into
// the fragment's registers: a copy the compiler placed between a read and
// the wait would take the registers before the data arrives (the backward
// parity tests, which run this path, would show it).
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ u32x4_t ds_read_tr_frag(const char* p) {
  const uint32_t a = (uint32_t)(uintptr_t)(lds_ptr_t)p;
  u32x2_t lo{0, 0}, hi{0, 0};
#if defined(__HIP_DEVICE_COMPILE__)
  asm volatile("ds_read_b64_tr_b16 %0, %1" : "=v"(lo) : "v"(a));
  asm volatile("ds_read_b64_tr_b16 %0, %1 offset:2048" : "=v"(hi) : "v"(a));
#endif
  return u32x4_t{lo[0], lo[1], hi[0], hi[1]};
}
// Waits for every LDS and scalar-cache access in flight; the fragments pass
// through, so nothing reads them before the wait.
template <int NA, int NB>
__device__ __forceinline__ void lds_wait_frags(u32x4_t (&a)[NA], u32x4_t (&b)[NB]) {
  static_assert(NA == 4 && NB == 8, "one wave's fragments");
#if defined(__HIP_DEVICE_COMPILE__)
  asm volatile("s_waitcnt lgkmcnt(0)"
               : "+v"(a[0]), "+v"(a[1]), "+v"(a[2]), "+v"(a[3]), "+v"(b[0]), "+v"(b[1]), "+v"(b[2]), "+v"(b[3]),
                 "+v"(b[4]), "+v"(b[5]), "+v"(b[6]), "+v"(b[7]));
#endif
}

// contraction slices of a dense job
__device__ __host__ __forceinline__ int k_slices(const GemmJob& j) { return j.ksplit > 1 ? j.ksplit : 1; }
// items: grouped jobs the router's tile table; per-expert-contraction jobs
// (kgroup) every (expert, row block); dense jobs row blocks x contraction slices
__device__ __forceinline__ int item_count(const GemmJob& j) {
  if (j.kgroup) return j.nexp * ((j.M + BM - 1) / BM);
  return j.grouped ? *j.tile_count : (j.M + BM - 1) / BM * k_slices(j);
}
inline long long max_item_count(const GemmJob& j) {
  if (j.kgroup) return (long long)j.nexp * ((j.M + BM - 1) / BM);
  return j.grouped ? j.max_items : (long long)(j.M + BM - 1) / BM * k_slices(j);
}
// XCD grid of a dense job: gc column groups (N-tile ranges) x 8 / gc row groups
__device__ __host__ __forceinline__ int xcd_cols(const GemmJob& j) {
  return j.xcd_cols == 2 || j.xcd_cols == 4 || j.xcd_cols == 8 ? j.xcd_cols : 1;
}

// I4: the launch has a job with int4 B (the int4 prefill); the bf16-only
// instantiations carry none of that code.  KM: 1 every job has both
// operands K-major (the weight gradients), 2 every job has a row-major A and
// a K-major B (the input gradients, B the weights as stored), 0 neither.
template <bool SWIGLU, bool I4, int KM>
__global__ __launch_bounds__(NTHR, 1) void gemm256_kernel(GemmArgs args) {
  typedef bf16_t T;
  // The ring; after the main loop its first buffer holds the row scales.
  __shared__ __attribute__((aligned(16))) char lds[kStages * kStageBytes];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

  int jid, bid;
  select_job(args, blockIdx.x, jid, bid);
  const GemmJob& p = args.job[jid];
  constexpr bool KA = KM == 1, KB = KM != 0;   // A, B K-major (KB: transposing B reads, N fragment first)

  // ---- work item and N tile.  Grouped: XCD x takes items [x*q, (x+1)*q),
  // each with all its N tiles back to back.  Dense: XCD x takes row-item
  // range xr and N-tile range xc of an (8 / gc) x gc grid, N tiles outer.
  const int count = item_count(p);
  const int nbn = n_tiles(p);
  const int xcd = bid & 7, local = bid >> 3;
  int item, nt;
  if (p.grouped || p.kgroup || p.xcd_cols < 0) {
    const int q = (count + 7) >> 3;
    const int pi = local / nbn;
    nt = local - pi * nbn;
    if (pi >= q) return;
    item = xcd * q + pi;
  } else {
    const int gc = xcd_cols(p), gr = 8 / gc;
    const int qr = (count + gr - 1) / gr, qc = (nbn + gc - 1) / gc;
    const int ntl = local / (qr > 0 ? qr : 1), pi = local - ntl * qr;
    if (ntl >= qc) return;
    nt = (xcd % gc) * qc + ntl;
    item = (xcd / gc) * qr + pi;
    if (nt >= nbn) return;
  }
  if (item >= count) return;
  int e = 0, rows, row_base, kz = 0;
  if (p.grouped) {
    e = p.tile_e[item];
    const int m0 = p.tile_m0[item];
    rows = p.counts[e] - m0;
    row_base = p.offsets[e] + m0;
  } else if (p.kgroup) {
    // (expert, row block): dense rows, the expert's own contraction range
    const int nrb = (p.M + BM - 1) / BM;
    e = item / nrb;
    const int m0 = (item - e * nrb) * BM;
    rows = p.M - m0;
    row_base = m0;
  } else {
    // dense items: row blocks of contraction slice 0, then of slice 1, ...
    const int nrb = (p.M + BM - 1) / BM;
    kz = item / nrb;
    const int m0 = (item - kz * nrb) * BM;
    rows = p.M - m0;
    row_base = m0;
  }
  const int klen = p.kgroup ? p.klen[e] : p.K / k_slices(p);
  const long long kofs = p.kgroup ? (long long)p.kofs[e] : (long long)kz * klen;
  // K-major: the expert's rows that exist (the rest of its last stage reads zeros)
  const int kcnt = KA ? max(0, min(klen, p.K - (int)kofs)) : klen;
  rows = rows < BM ? rows : BM;

  // Row scales of the gate-scaled epilogue: thread r < 256 fetches perm of
  // row r now and the gate two K steps before the end (after the wait that
  // drains every stage load, so no stage wait counts it); the scales reach
  // the waves through LDS.
  const bool scaled = p.gate != nullptr && (p.epi == EPI_ROWSCALE || p.epi == EPI_SWIGLU_BWD);
  int my_perm = 0;
  if (scaled && tid < BM) my_perm = p.perm[row_base + min(tid, rows - 1)];

  // ---- global -> LDS.  Lane i of a wave instruction lands at LDS byte
  // base + 16 i, so A load j of wave w fills A rows 32w + 16j + i/4 and B
  // load j fills B rows 32w + 16j + i/4, at physical piece i%4; the lane
  // fetches the logical piece the swizzle puts there.  LDS B row
  // wn*128 + ni*16 + f holds output column (tile base) + wn*128 + 8f + ni; for
  // SwiGLU the first 128 B rows are gate rows and the next 128 the matching
  // up rows, with h column (tile base) + wn*64 + 4f + ni.
  // int4 B (routed experts of the int4 prefill): a stage of B row r is its
  // 16 bytes (32 nibbles) at LDS byte 16 r, fetched as four 4-byte pieces by
  // four consecutive lanes, so a wave instruction still covers 16 rows and
  // every wave issues the same loads per stage as on the bf16 path.
  const bool b4 = I4 && p.b_int4 != 0;
  const char* a_src[NDA];
  const char* b_src[NDB];
  const char* bbase = reinterpret_cast<const char*>(p.B) +
                      (long long)e * p.b_estride * (b4 ? 1LL : (long long)sizeof(T));
  // the weight row that LDS B row R of this tile holds
  auto b_row = [&](int R) -> long long {
    if (SWIGLU) {
      const long long col = min(b_tile_row(true, R, nt, 0), (long long)p.N - 1);
      return (R >> 7 ? p.up_off : 0) + col;
    }
    return min(b_tile_row(false, R, nt, 0), (long long)p.N - 1);
  };
#pragma unroll
  for (int j = 0; j < NDA; ++j) {
    const int R = wave * (BM / 8) + j * 16 + (lane >> 2);
    const int c = swz_piece(R, lane & 3);            // XOR swizzles are their own inverse
    const int ra = min(R, rows - 1);
    const long long arow = p.a_rows ? (long long)(p.a_rows[row_base + ra] / p.a_div) : (long long)(row_base + ra);
    a_src[j] = reinterpret_cast<const char*>(p.A) + (arow * p.lda + kofs) * (long long)sizeof(T) + c * 16;
  }
#pragma unroll
  for (int j = 0; j < NDB; ++j) {
    const int R = wave * (BN / 8) + j * 16 + (lane >> 2);
    const int c = swz_piece(R, lane & 3);
    if (b4) {
      b_src[j] = bbase + b_row(R) * p.ldb + kofs / 2 + (lane & 3) * 4;
    } else if (p.b_staged) {
      // stage s of this tile: 256 rows x 64 bytes, contiguous, in LDS row order
      b_src[j] = bbase + (long long)nt * p.K * BN * (long long)sizeof(T) + R * kRowB + c * 16;
    } else {
      b_src[j] = bbase + (b_row(R) * p.ldb + kofs) * (long long)sizeof(T) + c * 16;
    }
  }
  const long long b_step = b4 ? 16LL : p.b_staged ? (long long)BN * kRowB : (long long)kRowB;
  const int nk = KA ? (kcnt + 31) >> 5 : (int)((long long)klen * sizeof(T) / kRowB);

  // ---- K-major operands (KM = 1: both, KM = 2: B only, A row-major as
  // above).  A stage holds 32 K rows of 256 columns (512 bytes) of each
  // K-major operand; load j of wave w fills K rows 4w + 2j + h,
  // h = lane / 32, 16 bytes per lane.  The 32-byte segment q of K row r sits
  // at segment q ^ ksw(r), which spreads the 16 rows x 32 bytes of one
  // transposing fragment read over all the banks.  A lane's piece is clamped
  // into the tile's columns (the extra columns feed only outputs that are
  // not stored); rows past the expert's count read zeros.  A gathered
  // operand's K rows come from its token map, four entries per wave and
  // stage, fetched by a scalar load one main-loop trip ahead (the vector
  // memory counter, which the stage waits use, never counts them).
  int km_col[NDA + NDB];   // byte offset of the lane's piece in its operand row
  const int kh = lane >> 5, kp = lane & 31;
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  const char* const km_base[2] = {reinterpret_cast<const char*>(p.A),
                                  reinterpret_cast<const char*>(p.B) + (long long)e * p.b_estride * 2};
  const long long km_ld2[2] = {p.lda * 2, p.ldb * 2};
  const int32_t* const km_map[2] = {p.a_krow, p.b_krow};
  const char* const km_zero = reinterpret_cast<const char*>(p.zrow) + 16 * kp;
  const int km_ofs = (int)kofs;
  if constexpr (KB) {
    const int ncols = min(p.N - nt * BN, BN);
#pragma unroll
    for (int j = KA ? 0 : NDA; j < NDA + NDB; ++j) {
      const int r = 4 * wave + 2 * (j & 1) + kh;
      const int lp = ((((kp >> 1) ^ ksw(r)) << 1) | (kp & 1)) * 8;
      km_col[j] = j < NDA ? (row_base + min(lp, rows - 8)) * 2 : (nt * BN + min(lp, ncols - 8)) * 2;
    }
  }
  // The map entries of the next stage to issue, per operand (scalar loads
  // started one main-loop trip ahead), and this lane's K rows of the stage
  // being issued (km_sel, at the top of a trip, right after the barrier:
  // no LDS read is in flight there, so the wait for the scalar loads that the
  // compiler puts before their first use costs only what is left of them).
  i32x4_t km_rows[2] = {i32x4_t{0, 0, 0, 0}, i32x4_t{0, 0, 0, 0}};
  int km_r[2][2] = {{0, 0}, {0, 0}};
  auto km_fetch = [&](int s) {
#pragma unroll
    for (int op = 0; op < 2; ++op)
      if (km_map[op]) km_rows[op] = sload4(km_map[op] + km_ofs + 32 * s + 4 * wave_u);
  };
  auto km_sel = [&](int s) {
#pragma unroll
    for (int op = 0; op < 2; ++op)
#pragma unroll
      for (int jj = 0; jj < 2; ++jj)
        km_r[op][jj] = km_map[op] ? (kh ? km_rows[op][2 * jj + 1] : km_rows[op][2 * jj])
                                  : km_ofs + 32 * s + 4 * wave + 2 * jj + kh;
  };
  // KM = 2: B has every K row (K a multiple of 32) and no map, so its source
  // is a fixed pointer advanced by 32 rows per stage, as in the row-major path
  const char* kb_src[NDB];
  if constexpr (KM == 2) {
#pragma unroll
    for (int j = 0; j < NDB; ++j)
      kb_src[j] = km_base[1] + (long long)(km_ofs + 4 * wave + 2 * j + kh) * km_ld2[1] + km_col[NDA + j];
  }
  auto km_src = [&](int s, int j) -> const char* {
    if constexpr (KM == 2) {
      return kb_src[j - NDA] + (long long)s * 32 * km_ld2[1];
    } else {
      const int op = j < NDA ? 0 : 1, jj = j & 1;
      const int kk = 32 * s + 4 * wave + 2 * jj + kh;
      return kk < kcnt ? km_base[op] + (long long)km_r[op][jj] * km_ld2[op] + km_col[j] : km_zero;
    }
  };
  auto issue_one = [&](int s, int j) {
    char* st = lds + (s % kStages) * kStageBytes;
    const long long off = (long long)s * kRowB;
    if (KA || (KB && j >= NDA)) {
      const char* src = km_src(s, j);
      __builtin_amdgcn_global_load_lds(src, (lds_ptr_t)(st + (j < NDA ? 0 : ATILE) + (wave * 2 + (j & 1)) * 1024), 16, 0,
                                       0);
    } else {
      if (j < NDA)
        __builtin_amdgcn_global_load_lds(a_src[j] + off, (lds_ptr_t)(st + wave * (BM / 8) * kRowB + j * 1024), 16, 0, 0);
      else if (b4)
        __builtin_amdgcn_global_load_lds(b_src[j - NDA] + (long long)s * b_step,
                                         (lds_ptr_t)(st + ATILE + wave * (BN / 8) * 16 + (j - NDA) * 256), 4, 0, 0);
      else
        __builtin_amdgcn_global_load_lds(b_src[j - NDA] + (long long)s * b_step,
                                         (lds_ptr_t)(st + ATILE + wave * (BN / 8) * kRowB + (j - NDA) * 1024), 16, 0,
                                         0);
    }
  };
  auto issue = [&](int s) {
#pragma unroll
    for (int j = 0; j < kLoads; ++j) issue_one(s, j);
  };

  // int4 B: the tile's bf16 scales, [K / 128 groups][256 LDS rows], in ring
  // buffer 0's B space past the 4 KiB its int4 stage uses (never a load
  // target), filled before the ring and made visible by a barrier.
  const uint16_t* scl = reinterpret_cast<const uint16_t*>(lds + ATILE + 4096);
  if (b4) {
    const int G = p.K / 128;
    const uint16_t* sg = reinterpret_cast<const uint16_t*>(p.b_scales) + (long long)e * p.b_sestride;
    uint16_t* dst = reinterpret_cast<uint16_t*>(lds + ATILE + 4096);
    for (int i = tid; i < G * BN; i += NTHR) {
      const int gi = i / BN, R = i - gi * BN;
      dst[i] = sg[b_row(R) * G + gi];
    }
    __syncthreads();
  }
  // ---- LDS -> MFMA operand rows of this wave (16 consecutive LDS rows per
  // tile).  Wave layouts (WC: column groups of waves): 2 (4 row bands x 2,
  // a wave 64 x 128, eight fragments), 4 (2 x 4, 64 x 64, four) and 8 (1 x 8,
  // 64 x 32, two).  The LDS layout of B and the stage loads are the same in
  // every layout: a wave of layout WC takes NI of the eight fragments of
  // wave group wn2 of layout 2 (sub-block sub), so a lane's NI output columns
  // stay adjacent.  With args.small_layouts, tiles of at most 128 rows take
  // layout 4 and SwiGLU tiles of at most 64 rows layout 8 (the other
  // instantiations' registers do not hold a third layout): every wave then
  // has rows to multiply, two per SIMD instead of one or none.
  const int fr = lane & 15, g = lane >> 4;
  auto tile_body = [&](auto wc_tag) {
  constexpr int WC = decltype(wc_tag)::value;
  static_assert(WC == 2 || KM == 0, "K-major operands use the 4 x 2 layout");
  constexpr int NI = 16 / WC, HN = NI / 2, NSUB = WC / 2;
  const int wm = wave / WC, wn = wave % WC;
  const int wn2 = wn / NSUB, sub = wn % NSUB;
  const bool active = wm * WM < rows;
  int arow_l[4], brow_l[NI];
#pragma unroll
  for (int mi = 0; mi < 4; ++mi) arow_l[mi] = wm * WM + mi * 16 + fr;
#pragma unroll
  for (int li = 0; li < NI; ++li) {
    // the fragment's index in layout 2
    const int ni = SWIGLU ? (li < HN ? sub * HN + li : 4 + sub * HN + (li - HN)) : sub * NI + li;
    brow_l[li] = (SWIGLU ? (ni < 4 ? wn2 * 64 + ni * 16 : BN / 2 + wn2 * 64 + (ni - 4) * 16) : wn2 * 128 + ni * 16) + fr;
  }

  f32x4_t acc[4][NI];
#pragma unroll
  for (int mi = 0; mi < 4; ++mi)
#pragma unroll
    for (int ni = 0; ni < NI; ++ni) acc[mi][ni] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // Lane (fr, g)'s int4 operand of LDS B row r: the 8 nibbles of elements
  // 8g .. 8g + 7 of the stage, and the row's scale for stage s's group.
  auto qword = [&](const char* Bs, int r) { return *reinterpret_cast<const uint32_t*>(Bs + r * 16 + 4 * g); };
  auto qscale = [&](int s, int r) { return bf16_to_f32(scl[(s >> 2) * BN + r]); };

  // Operands of one stage: lane group g owns 16-byte piece g of each 64-byte
  // row chunk.  The MFMAs of stage s run from registers (fa, fb) while the
  // operands of stage s + 1 are read from LDS behind them: fb[ni] is reloaded
  // as soon as the four MFMAs that use it are issued, the A pieces go to a
  // second set (fa of the next stage).  This wave's global loads of stage
  // s + kStages - 1 go between the MFMAs (after blocks ni = 1, 3, 5, 7).
  // int4 B: the raw code word and scale of each B fragment (expanded to
  // bf16 right before its MFMAs)
  u32x4_t fa0[4], fa1[4], fb[NI];
  uint32_t qb[NI];
  float qs[NI];
  // K-major fragment at tile column 16 c16: lane (fr, g) needs K rows 8g ..
  // 8g + 7 of column 16 c16 + fr.  A transposing read gives lane i of each
  // 16-lane group the four values at column c0 + i of four consecutive rows
  // when lane j of the group points at row (first) + j / 4, columns c0 +
  // 4 (j % 4) .. + 3; two reads (rows 8g and 8g + 4) make the fragment.
  const int km_lane = (8 * g + (fr >> 2)) * 512 + 8 * (fr & 3);
  const int km_f = (g << 2) | (fr >> 2);   // ksw of every row this lane reads
  auto km_frag = [&](const char* X, int c16) -> u32x4_t {
    return ds_read_tr_frag(X + km_lane + 32 * (c16 ^ km_f));
  };
  auto read_a = [&](int s, u32x4_t (&fa)[4]) {
    const char* As = lds + (s % kStages) * kStageBytes;
#pragma unroll
    for (int mi = 0; mi < 4; ++mi) {
      if constexpr (KA) fa[mi] = km_frag(As, 4 * wm + mi);
      else fa[mi] = ld16(As + swz(arow_l[mi], g));
    }
  };
  auto read_b = [&](int s, auto b4c) {
    const char* Bs = lds + (s % kStages) * kStageBytes + ATILE;
#pragma unroll
    for (int ni = 0; ni < NI; ++ni) {
      if constexpr (KB) {
        fb[ni] = km_frag(Bs, 8 * wn + ni);
      } else if constexpr (decltype(b4c)::value) {
        qb[ni] = qword(Bs, brow_l[ni]);
        qs[ni] = qscale(s, brow_l[ni]);
      } else {
        fb[ni] = ld16(Bs + swz(brow_l[ni], g));
      }
    }
  };
  // stage s from (fa, fb); prefetch: read stage s + 1 into (fn, fb); loads:
  // issue stage s + kStages - 1
  // ACT: this wave's row band holds rows (compile-time, so the loop below is
  // instantiated once per case and its LDS waits stay exact).  B4: int4 B.
  auto compute = [&](int s, u32x4_t (&fa)[4], u32x4_t (&fn)[4], auto act, auto prefetch, auto with_loads,
                     auto b4c) {
    if constexpr (!decltype(act)::value) {
      if constexpr (decltype(with_loads)::value) issue(s + kStages - 1);
      return;
    }
    constexpr bool B4 = decltype(b4c)::value;
    const char* An = lds + ((s + 1) % kStages) * kStageBytes;
    const char* Bn = An + ATILE;
#pragma unroll
    for (int ni = 0; ni < NI; ++ni) {
      u32x4_t bv;
      if constexpr (B4) bv = dq_int4x8(qb[ni], qs[ni]);
      else bv = fb[ni];
      // K-major: the N fragment is the MFMA's first operand, so a lane's four
      // results are four adjacent output columns of one output row
#pragma unroll
      for (int mi = 0; mi < 4; ++mi) {
        if constexpr (KB) acc[mi][ni] = Mma<T>::run1(bv, fa[mi], acc[mi][ni]);
        else acc[mi][ni] = Mma<T>::run1(fa[mi], bv, acc[mi][ni]);
      }
      if constexpr (decltype(prefetch)::value) {
        if constexpr (KB) {
          fb[ni] = km_frag(Bn, 8 * wn + ni);
          if (ni < 4) {
            if constexpr (KA) fn[ni] = km_frag(An, 4 * wm + ni);
            else fn[ni] = ld16(An + swz(arow_l[ni], g));
          }
        } else {
          if constexpr (B4) {
            qb[ni] = qword(Bn, brow_l[ni]);
            qs[ni] = qscale(s + 1, brow_l[ni]);
          } else {
            fb[ni] = ld16(Bn + swz(brow_l[ni], g));
          }
          if constexpr (NI >= 4) {
            if (ni < 4) fn[ni] = ld16(An + swz(arow_l[ni], g));
          } else {
#pragma unroll
            for (int q = 0; q < 4 / NI; ++q) fn[ni * (4 / NI) + q] = ld16(An + swz(arow_l[ni * (4 / NI) + q], g));
          }
        }
      }
      if constexpr (decltype(with_loads)::value) {
        if constexpr (NI == 8) {
          if (ni & 1) issue_one(s + kStages - 1, ni >> 1);
        } else {
#pragma unroll
          for (int q = 0; q < kLoads / NI; ++q) issue_one(s + kStages - 1, ni * (kLoads / NI) + q);
        }
      }
      __builtin_amdgcn_sched_barrier(0);   // keep the reads and loads spread out
    }
    if constexpr (KB && decltype(prefetch)::value) lds_wait_frags(fn, fb);
  };

  // ---- main loop.  Iteration s waits for stage s + 1 (its loads went out
  // two iterations earlier) and passes a barrier, so stage s + 1 is complete
  // in LDS for the prefetch, and every wave has finished the MFMAs of stage
  // s - 1, whose operands it read in iteration s - 2: buffer (s - 1) % 5 is
  // free for the loads of stage s + 4.
  static_assert(kStages == 5, "the waits below assume a 5-deep ring");
  for (int s = 0; s < kStages - 1 && s < nk; ++s) {
    if constexpr (KA) {
      km_fetch(s);
      km_sel(s);
    }
    issue(s);
  }
  if (KA && kStages - 1 < nk) km_fetch(kStages - 1);
  if (nk >= 4) wait_vmcnt<3 * kLoads>();
  else if (nk == 3) wait_vmcnt<2 * kLoads>();
  else if (nk == 2) wait_vmcnt<kLoads>();
  else wait_vmcnt<0>();
  block_barrier();
  float my_gate = 0.f;
  auto run = [&](auto act, auto b4c) {
    using A = decltype(act);
    using B4 = decltype(b4c);
    if constexpr (A::value) {
      read_a(0, fa0);
      read_b(0, B4{});
      if constexpr (KB) lds_wait_frags(fa0, fb);
    }
    // Stages issued before iteration s: min(nk, s + 4); in flight after stage
    // s + 1: that minus s + 2.  Two K steps per trip, so the two A sets swap
    // roles without a copy (a copy would wait for every LDS read in flight
    // before each barrier).
    int s = 0;
    for (; s + kStages - 1 < nk; ++s) {
      wait_vmcnt<2 * kLoads>();
      block_barrier();
      if constexpr (KA) km_sel(s + kStages - 1);
      compute(s, fa0, fa1, A{}, std::true_type{}, std::true_type{}, B4{});
      if (KA && s + kStages < nk) km_fetch(s + kStages);
#pragma unroll
      for (int mi = 0; mi < 4; ++mi) fa0[mi] = fa1[mi];
    }
    for (; s + 1 < nk; ++s) {
      if (nk - s - 2 >= 2) wait_vmcnt<2 * kLoads>();
      else if (nk - s - 2 == 1) wait_vmcnt<kLoads>();
      else wait_vmcnt<0>();
      block_barrier();
      if (scaled && s == nk - 2 && tid < BM) my_gate = p.gate[my_perm];
      compute(s, fa0, fa1, A{}, std::true_type{}, std::false_type{}, B4{});
#pragma unroll
      for (int mi = 0; mi < 4; ++mi) fa0[mi] = fa1[mi];
    }
    compute(s, fa0, fa1, A{}, std::false_type{}, std::false_type{}, B4{});
  };
  // an expert with an empty contraction range (no tokens) stores zeros
  if (nk > 0) {
    if (!active) run(std::false_type{}, std::false_type{});   // loads only (issue_one picks the B form)
    else if constexpr (I4) {
      if (b4) run(std::true_type{}, std::true_type{});
      else run(std::true_type{}, std::false_type{});
    } else {
      run(std::true_type{}, std::false_type{});
    }
  }

  // Row scales, staged in ring buffer 0 once every wave is past its last
  // read of the ring.
  float* const row_scale = reinterpret_cast<float*>(lds);
  if (scaled) {
    __syncthreads();
    if (tid < BM) row_scale[tid] = nk >= 2 ? my_gate : p.gate[my_perm];
    __syncthreads();
  }
  if constexpr (KM == 2) __syncthreads();            // the ring is reused below
  if (!active) return;
  if constexpr (KM == 2) {
    // acc[mi][ni][i] is tile row wm*64 + 16 mi + fr, column wn*128 + 16 ni +
    // 4g + i.  Re-laid through LDS (this wave's 32 x 144 fp32 block, past the
    // row scales), two 16-row blocks at a time, into the layout of the
    // row-major mode (row wm*64 + 16 mi + 4g + i, column wn*128 + 8 fr + ni),
    // so that the epilogue below stores 8 adjacent columns per lane.  Rows
    // 144 floats apart put both directions at two cycles per 1 KiB access.
    constexpr int XS = 144;
    float* const xb = reinterpret_cast<float*>(lds + 4096) + wave * (32 * XS);
#pragma unroll
    for (int half = 0; half < 2; ++half) {
#pragma unroll
      for (int m2 = 0; m2 < 2; ++m2)
#pragma unroll
        for (int ni = 0; ni < NI; ++ni)
          *reinterpret_cast<f32x4_t*>(xb + (16 * m2 + fr) * XS + 16 * ni + 4 * g) = acc[2 * half + m2][ni];
#pragma unroll
      for (int m2 = 0; m2 < 2; ++m2)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float* src = xb + (16 * m2 + 4 * g + i) * XS + 8 * fr;
          const f32x4_t lo = *reinterpret_cast<const f32x4_t*>(src), hi = *reinterpret_cast<const f32x4_t*>(src + 4);
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            acc[2 * half + m2][c][i] = lo[c];
            acc[2 * half + m2][c + 4][i] = hi[c];
          }
        }
    }
  } else if constexpr (KM == 1) {
    // acc[mi][ni][i]: tile row wm*64 + 16 mi + fr, column wn*128 + 16 ni + 4g + i
    float* const Ck = reinterpret_cast<float*>(p.C) + (long long)e * p.c_estride;
#pragma unroll
    for (int mi = 0; mi < 4; ++mi) {
      const int lr = wm * WM + 16 * mi + fr;
      if (lr >= rows) continue;
#pragma unroll
      for (int ni = 0; ni < NI; ++ni) {
        const int n = nt * BN + wn * 128 + 16 * ni + 4 * g;
        if (n < p.N)
          *reinterpret_cast<f32x4_t*>(Ck + (long long)(row_base + lr) * p.ldc + n) = acc[mi][ni];
      }
    }
    return;
  }
  // ---- epilogue.  acc[mi][ni][i] is tile row wm*64 + mi*16 + 4g + i.  Its
  // column, past the wave's base, is 8f + ni (f = lane % 16); for SwiGLU,
  // blocks ni < 4 are gate columns 4f + ni and ni >= 4 the matching up.
  T* C = reinterpret_cast<T*>(p.C) + kz * p.c_kstride;
  float* const Cf = reinterpret_cast<float*>(p.C) + (long long)e * p.c_estride;   // EPI_STORE_F32 (kgroup)
  T* aux = reinterpret_cast<T*>(p.aux);
  const int n = nt * BN + wn2 * 128 + 8 * fr + sub * NI;         // first column of this lane (not SwiGLU)
  const int fh = nt * (BN / 2) + wn2 * 64 + 4 * fr + sub * HN;   // first h column of this lane (SwiGLU)
  if (SWIGLU ? fh >= p.N : n >= p.N) return;
  if (WC == 2 && !SWIGLU && KM != 1 && p.epi == EPI_SWIGLU_BWD) {
    // SwiGLU backward: dH = s * acc, then (da, du) from the saved (a, u).
    // The saved rows of the next 16-row block are requested before this
    // block's arithmetic (a row per (mi, i); rows past the item re-read its
    // last row, so no load sits under a lane condition and waits where the
    // condition ends): the loads of one block overlap the math and stores of
    // the one before instead of a round trip per row.
    const T* const aub = reinterpret_cast<const T*>(p.aux);
    u32x4_t ra[2][4], ru[2][4];
    auto load_block = [&](int mi, u32x4_t (&xa)[4], u32x4_t (&xu)[4]) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int lr = min(wm * WM + mi * 16 + 4 * g + i, rows - 1);
        const T* au = aub + (long long)(row_base + lr) * p.ldaux;
        xa[i] = ld16(au + n);
        xu[i] = ld16(au + p.N + n);
      }
    };
    load_block(0, ra[0], ru[0]);
#pragma unroll
    for (int mi = 0; mi < 4; ++mi) {
      if (mi + 1 < 4) load_block(mi + 1, ra[(mi + 1) & 1], ru[(mi + 1) & 1]);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int lr = wm * WM + mi * 16 + 4 * g + i;
        if (lr >= rows) continue;
        const long long row = row_base + lr;
        const float sc = p.gate ? row_scale[lr] : 1.f;
        float da[NI], du[NI], hs[NI];
#pragma unroll
        for (int ni = 0; ni < NI; ++ni) {
          const uint32_t wa = ra[mi & 1][i][ni >> 1], wu = ru[mi & 1][i][ni >> 1];
          const float a = bf16_to_f32((bf16_t)((ni & 1) ? (wa >> 16) : (wa & 0xFFFFu)));
          const float u = bf16_to_f32((bf16_t)((ni & 1) ? (wu >> 16) : (wu & 0xFFFFu)));
          const float dh = acc[mi][ni][i] * sc;
          const float sg = sigmoidf_(a);
          const float si = a * sg;
          da[ni] = dh * u * (sg * (1.f + a * (1.f - sg)));
          du[ni] = dh * si;
          hs[ni] = sc * (si * u);
        }
        store_vec<T, NI>(C + row * p.ldc + n, da);
        store_vec<T, NI>(C + row * p.ldc + p.N + n, du);
        if (p.hg) store_vec<T, NI>(reinterpret_cast<T*>(p.hg) + row * p.N + n, hs);
      }
    }
    return;
  }
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
      } else if (p.epi == EPI_STORE_F32) {
        float v[NI];
#pragma unroll
        for (int ni = 0; ni < NI; ++ni) v[ni] = acc[mi][ni][i];
        store_vec<float, NI>(Cf + row * p.ldc + n, v);
      } else {  // EPI_STORE
        float v[NI];
#pragma unroll
        for (int ni = 0; ni < NI; ++ni) v[ni] = acc[mi][ni][i];
        store_vec<T, NI>(C + row * p.ldc + n, v);
      }
    }
  }
  };
  // the wave layout of this tile (row-major jobs: by the rows it holds)
  if constexpr (KM == 0) {
    if (SWIGLU && args.small_layouts && rows <= 64) {
      tile_body(std::integral_constant<int, 8>{});
      return;
    }
    if (args.small_layouts && rows <= 128) {
      tile_body(std::integral_constant<int, 4>{});
      return;
    }
  }
  tile_body(std::integral_constant<int, 2>{});
}

// chunks of 8 blocks (one per XCD) a job needs: the blocks one XCD runs
int job_chunks(const GemmJob& j) {
  const int nbn = n_tiles(j);
  if (j.grouped || j.kgroup || j.xcd_cols < 0) return (int)((max_item_count(j) + 7) / 8 * nbn);
  const int gc = xcd_cols(j), gr = 8 / gc;
  return (int)((max_item_count(j) + gr - 1) / gr * ((nbn + gc - 1) / gc));
}

// One 16-byte piece per thread: piece u of the stage-major array is piece
// (u % 4) of the 64-byte chunk s of weight row b_tile_row(R, nt), where
// u / 4 = ((e * ntiles + nt) * nstages + s) * 256 + R.
__global__ __launch_bounds__(256) void pack_routed_kernel(const char* __restrict__ w, char* __restrict__ out,
                                                          long long units, int K, int ntiles, int up_off,
                                                          int swiglu) {
  const int nstages = K * 2 / kRowB;
  for (long long u = (long long)blockIdx.x * 256 + threadIdx.x; u < units; u += (long long)gridDim.x * 256) {
    const int piece = (int)(u & 3);
    const long long rowu = u >> 2;
    const int R = (int)(rowu % BN);
    const long long t = rowu / BN;
    const int st = (int)(t % nstages);
    const long long en = t / nstages;
    const int nt = (int)(en % ntiles);
    const long long e = en / ntiles;
    const long long row = b_tile_row(swiglu != 0, R, nt, up_off);
    const long long rows_e = (long long)ntiles * BN;
    const char* src = w + ((e * rows_e + row) * K) * 2 + st * kRowB + piece * 16;
    *reinterpret_cast<uint4*>(out + u * 16) = *reinterpret_cast<const uint4*>(src);
  }
}

}  // namespace

void launch_pack_routed(const void* w_gate_up, const void* w_down, int E, int d, int F, void* out_gate_up,
                        void* out_down, hipStream_t s) {
  // gate/up: [E, 2F, d] in tiles of 128 h columns (256 rows); down: [E, d, F]
  // in tiles of 256 output columns
  const long long u_gu = (long long)E * 2 * F * d * 2 / 16, u_d = (long long)E * d * F * 2 / 16;
  if (u_gu > 0)
    hipLaunchKernelGGL(pack_routed_kernel, dim3((unsigned)std::min<long long>((u_gu + 255) / 256, 16384)), dim3(256),
                       0, s, (const char*)w_gate_up, (char*)out_gate_up, u_gu, d, F / (BN / 2), F, 1);
  if (u_d > 0)
    hipLaunchKernelGGL(pack_routed_kernel, dim3((unsigned)std::min<long long>((u_d + 255) / 256, 16384)), dim3(256),
                       0, s, (const char*)w_down, (char*)out_down, u_d, F, d / BN, 0, 0);
}

// bf16 operands only: epilogues SwiGLU, row scale, SwiGLU backward, plain
// store (bf16) or fp32 store (the weight gradients, with per-expert
// contraction ranges: klen[e] a multiple of 32, possibly 0, or K-major
// operands, both jobs then); K / ksplit a multiple of 32 (checked by the
// caller); a split job's slices each write their own output.
void launch_gemm_fwd256(const GemmArgs& in, hipStream_t s) {
  GemmArgs a = in;
  long long total = 0;
  for (int i = 0; i < a.njobs; ++i) {
    a.chunks[i] = job_chunks(a.job[i]);
    total += a.chunks[i];
  }
  if (total == 0) return;
  const dim3 grid((unsigned)(total * 8));
  const bool i4 = a.job[0].b_int4 || (a.njobs > 1 && a.job[1].b_int4);
  if (a.job[0].kmaj == 1) {
    hipLaunchKernelGGL((gemm256_kernel<false, false, 1>), grid, dim3(NTHR), 0, s, a);
  } else if (a.job[0].kmaj == 2) {
    hipLaunchKernelGGL((gemm256_kernel<false, false, 2>), grid, dim3(NTHR), 0, s, a);
  } else if (a.job[0].epi == EPI_SWIGLU) {
    if (i4) hipLaunchKernelGGL((gemm256_kernel<true, true, 0>), grid, dim3(NTHR), 0, s, a);
    else hipLaunchKernelGGL((gemm256_kernel<true, false, 0>), grid, dim3(NTHR), 0, s, a);
  } else {
    if (i4) hipLaunchKernelGGL((gemm256_kernel<false, true, 0>), grid, dim3(NTHR), 0, s, a);
    else hipLaunchKernelGGL((gemm256_kernel<false, false, 0>), grid, dim3(NTHR), 0, s, a);
  }
}

}  // namespace fgmoe
