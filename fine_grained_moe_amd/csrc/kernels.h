// Host-side launchers of the gfx950 kernels (internal to the library).
#pragma once

#include <algorithm>

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fgmoe {

// Rows of one grouped-GEMM tile: gemm.hip (fp32 forward, backward) and
// gemm_fwd.hip (bf16 forward).  The router writes a tile table for each.
constexpr int kTileM = 128;
constexpr int kTileMFwd = 256;

// Tokens owned by one router workgroup: 16, or 64 for bf16 batches of more
// than 4096 tokens with d a multiple of 256 (above one round of 16-token
// workgroups on 256 CUs; the router matrix is then read a quarter as often).
// The per-block loads and ranks of launch_route_topk are per tpb tokens.
inline int route_tpb(int T, int act, int d) { return (act == 1 && d % 256 == 0 && T > 4096) ? 64 : 16; }
inline int route_blocks(int T, int tpb) { return (T + tpb - 1) / tpb; }
// Upper bound of sum_e ceil(count_e / kTileM) over any routing of T*k slots.
inline long long max_group_tiles(long long slots, int E, int tm = kTileM) {
  return (slots + (long long)E * (tm - 1)) / tm;
}

// (expert, first row) of every tm rows of each expert, in expert order, and
// the number of entries.
struct TileTable {
  int32_t* e;
  int32_t* m0;
  int32_t* count;
};

// act: 0 = float32, 1 = bfloat16 (moe_dtype values).
void launch_route_topk(int act, const void* x, const void* w_router, const float* bias, int T, int d, int E,
                       int k, int32_t* idx, float* gate, int32_t* block_counts, int32_t* rank, hipStream_t s);
// tiles: kTileM rows per entry; tiles_fwd: kTileMFwd rows (may be null).
// bias (may be null): once the loads are known, the bias step with gamma on
// bias (in place) and, if stats is not null, the balance figures (as
// launch_bias_update with total T * k).
// tpb: route_tpb of the batch (the router's block size).
void launch_route_dispatch(const int32_t* block_counts, const int32_t* idx, const int32_t* rank, int tpb, int T,
                           int E, int k, int32_t* counts, int32_t* offsets, TileTable tiles, TileTable tiles_fwd,
                           int32_t* perm, int32_t* pos, float gamma, float* bias, float* stats, hipStream_t s);
// stats (may be null): [4] expert-balance figures of the batch
void launch_bias_update(int E, long long total, const int32_t* counts, float gamma, float* bias, float* stats,
                        hipStream_t s);

enum Epilogue {
  EPI_SWIGLU = 0,       // C[row, f] = silu(acc_gate) * acc_up; aux = (gate | up) pre-activations
  EPI_ROWSCALE = 1,     // C[row, n] = gate[perm[row]] * acc; aux = acc
  EPI_STORE = 2,        // C[row, n] = acc (operand dtype)
  EPI_SWIGLU_BWD = 3,   // dH = s * acc (s = gate[perm[row]] or 1); from a = aux[row, n], u = aux[row, N + n]:
                        //   C[row, n] = dH * u * silu'(a), C[row, N + n] = dH * silu(a)
  EPI_STORE_F32 = 4     // C[row, n] = acc as float32
};

// One GEMM problem C = A . B^T on MFMA with a fused epilogue.  Element offsets
// are in elements of the launch's dtype.
struct GemmJob {
  int epi;                 // Epilogue; both jobs of a launch are SwiGLU or both are not
  // A: rows of length >= K.  Row of output row `slot`: a_rows ? a_rows[slot] / a_div : slot.
  const void* A;
  long long lda;
  const int32_t* a_rows;
  int a_div;
  // B: [N_rows, K] per expert, expert e at B + e * b_estride.
  const void* B;
  long long ldb;
  long long b_estride;
  // launch_gemm_fwd256 only: B in the stage-major layout of
  // launch_pack_routed (whole 256-row tiles; ldb unused)
  int b_staged;
  // launch_gemm_fwd256 only, grouped jobs: B holds int4 rows (two nibbles
  // per byte, element 2i in the low nibble; ldb and b_estride in bytes) with
  // one bf16 scale per 128 elements of a row in b_scales (row r of expert e
  // at b_scales + e * b_sestride + r * K / 128); the operand is bf16(q *
  // scale).  K / 128 <= kInt4MaxGroups.
  int b_int4;
  const void* b_scales;
  long long b_sestride;
  int K;
  int N;                   // output columns (SwiGLU: h columns; B then has gate rows 0..N-1 and up rows up_off..)
  int up_off;
  // rows: grouped (tile table over experts) or dense [M]
  int grouped;
  int M;
  const int32_t* tile_e;
  const int32_t* tile_m0;
  const int32_t* tile_count;
  const int32_t* offsets;
  const int32_t* counts;
  int max_items;           // grouped jobs: upper bound of the tile count (sizes the grid)
  // per-expert contraction ranges (weight gradients): item = (expert, row
  // tile of M); expert e contracts over K elements [kofs[e], kofs[e] + klen[e])
  // of every A and B row and writes C + e * c_estride.  klen[e] % (64 bytes) == 0.
  int kgroup;
  int nexp;
  const int32_t* kofs;
  const int32_t* klen;
  long long c_estride;
  // launch_gemm_fwd256 only.  kmaj = 1, kgroup jobs with the fp32 store (the
  // weight gradients): A and B are K-major, element (m, k) of A at
  // A[krow(k) * lda + m] and (n, k) of B at B[krow(k) * ldb + n], krow(k) =
  // a_krow ? a_krow[k] : k (b_krow likewise), over expert e's rows kofs[e] +
  // [0, min(klen[e], K - kofs[e])) (klen[e] any count).  The maps are readable
  // 32 entries past every range, zrow points at 512 zero bytes, M and N are
  // multiples of 8 and lda, ldb multiples of 8 elements.  kmaj = 2, grouped
  // or dense jobs with the plain store or the SwiGLU-backward epilogue (the
  // input gradients): A as usual, B K-major, (n, k) of expert e at B +
  // e * b_estride + k * ldb + n; K a multiple of 32, N of 8.  Both jobs of a
  // launch have the same kmaj.
  int kmaj;
  const int32_t* a_krow;
  const int32_t* b_krow;
  const void* zrow;
  // dense jobs of launch_gemm_fwd256: the contraction is cut into ksplit
  // equal slices (K / ksplit a multiple of 32); slice z writes C + z * c_kstride.
  int ksplit;
  long long c_kstride;
  // dense jobs of launch_gemm_fwd256: the 8 XCDs take a (8 / xcd_cols) x
  // xcd_cols grid of (row-block, N-tile) ranges (1, 2, 4 or 8; 0 means 1), N
  // tiles outer; -1: XCD x takes a contiguous range of row items and runs
  // each item's N tiles back to back (as grouped jobs)
  int xcd_cols;
  // outputs
  void* C;
  long long ldc;
  void* aux;               // SwiGLU: pre-activations [rows, 2N] (gate | up); ROWSCALE: unscaled rows
  long long ldaux;
  const float* gate;       // ROWSCALE: row scale gate[perm[slot]]
  const int32_t* perm;
  // launch_gemm_fwd256, SwiGLU-backward epilogue: also the row-scaled
  // activation s * silu(a) * u, [rows, N] (unused when null)
  void* hg;
};

// A launch: one or two jobs sharing the dtype.
struct GemmArgs {
  int act;                 // dtype of A, B, C, aux
  int njobs;
  int order;               // two jobs: 0 = chunks alternate, 1 = job 0's chunks first, 2 = job 1's first
  int chunks[2];           // filled by launch_gemm
  GemmJob job[2];
  // launch_gemm_fwd256, row-major operands: tiles of at most 128 rows (64,
  // SwiGLU) spread their 64-row band(s) over all eight waves
  int small_layouts;
};
void launch_gemm(const GemmArgs& a, hipStream_t s);
// bf16 jobs with the SwiGLU, row-scale, SwiGLU-backward or store epilogue
// (K % 32 == 0) on 256 x 256 tiles; grouped jobs index the kTileMFwd tile
// table.
void launch_gemm_fwd256(const GemmArgs& a, hipStream_t s);
// Scale groups of an int4 B operand that a launch_gemm_fwd256 tile keeps in
// LDS (K / 128 of them): K up to 3072.
constexpr int kInt4MaxGroups = 24;
// Routed bf16 weights into the stage-major layout that launch_gemm_fwd256
// reads with b_staged: gate/up [E, 2F, d] (F % 128 == 0) and down [E, d, F]
// (d % 256 == 0) to arrays of the same sizes.
void launch_pack_routed(const void* w_gate_up, const void* w_down, int E, int d, int F, void* out_gate_up,
                        void* out_down, hipStream_t s);

// Top-1 serving with int4 routed experts, T <= 64 tokens (decode.hip), built
// for the NanoColibri layer shape.
constexpr int kDecodeMaxT = 64;
constexpr int kDecodeD = 1024, kDecodeF = 512, kDecodeFs = 2048;
bool decode_shape_supported(int d, int F, int Fs);
struct DecodeArgs {
  int T, d, E, F, Fs, k;
  const uint16_t* x;                 // [T, d] bf16
  const uint16_t* w_router;          // [E, d] bf16
  const float* bias;                 // [E]
  const uint16_t* w_sh_gate_up;      // [2Fs, d] bf16
  const uint16_t* w_sh_down;         // [d, Fs] bf16
  const uint8_t* q_gate_up;          // [E, 2F, d/2] int4 pairs
  const uint16_t* s_gate_up;         // [E, 2F, d/128] bf16
  const uint8_t* q_down;             // [E, d, F/2]
  const uint16_t* s_down;            // [E, d, F/128]
  int32_t* idx;
  float* gate;
  int32_t* counts;
  int32_t* offsets;
  int32_t* perm;
  int32_t* pos;
  int32_t* active;                   // [E][3] (expert, first slot, load) of each expert with a load, ascending
  int32_t* n_active;                 // [1]
  uint64_t* rkey;                    // [4][64] per expert tile: each token's largest selection key (workspace)
  float* rscore;                     // [4][64] the sigmoid score that goes with it (workspace)
  uint16_t* Hs;                      // [T, Fs] bf16 (workspace)
  uint16_t* H;                       // [T*k, F] bf16 (workspace)
  float* part_sh;                    // [4, T, d] fp32 shared down partials (workspace)
  uint16_t* y;                       // [T, d] bf16
  const uint16_t* resid;             // [T, d] bf16 residual added to y, or null
  // MoE block, at most 16 tokens: x holds h, which stage 1 normalises (x =
  // bf16(h / rms(h) * gamma)); the normalised rows go to xn for stage 2.
  // gamma null (required above 16 tokens): x is used as it is.
  const float* gamma;                // [d] float32, or null
  float eps;
  uint16_t* xn;                      // [T, d] bf16 (workspace)
  // Expert streaming: the routed weights above hold n_slots slots, and expert
  // e's weights sit in slot slot[e] (clamped to the slots), or null: slot e.
  const int32_t* slot;               // [E] int32, or null
  int n_slots;
  // the bias step, taken by stage 2 once the loads are known (null: none)
  float* step_bias;                  // [E] in/out (the bias the router read)
  float step_gamma;
  float* step_stats;                 // [4] balance figures, or null
  // the next layer's router and shared gate/up (the same shapes), read into
  // the L2 caches by stage 3, or null
  const uint16_t* pf_router;
  const uint16_t* pf_sh_gate_up;
};
void launch_decode(const DecodeArgs& a, hipStream_t s);

// Backward helpers (backward.hip).  Contraction ranges of the weight-gradient
// GEMMs are padded to kPadK elements with zero columns.
constexpr int kPadK = 64;
inline long long pad_k(long long n) { return (n + kPadK - 1) / kPadK * kPadK; }

// dst[b][r][c] = scale * src[b][row(c)][r]; see transpose_kernel.
struct TransposeArgs {
  const void* src;
  long long ld_src;
  long long src_bstride;
  void* dst;
  long long ld_dst;
  long long dst_bstride;
  int R, C, batch;
  int n_in;                  // without map1: columns >= n_in are zero
  const int32_t* map1;       // column -> index (or -1 for a zero column)
  const int32_t* map2;       // index -> source index; source row = map2[...] / div
  int div;
  const float* scale;        // optional, indexed by the source index before division
};
void launch_fill_zero(void* p, size_t bytes, hipStream_t s);   // bytes % 4 == 0
// int4 export (quant.hip): w [rows, K] (act 1 = bf16, else fp32), K % 128 == 0
// -> packed [rows, K/2] bytes and bf16 scales [rows, K/128].
void launch_quant_int4(int act, const void* w, long long rows, int K, uint8_t* packed, void* scales,
                       hipStream_t s);
// Inverse for the int4 prefill: packed [E, rows_e, K/2] + scales [E, rows_e,
// K/128] -> bf16 [E, rows_e, K] for the experts with counts[e] > 0.
void launch_dequant_int4(const void* packed, const void* scales, int E, int rows_e, int K, const int32_t* counts,
                         void* out, hipStream_t s);
void launch_bwd_prep(const int32_t* counts, const int32_t* offsets, int E, int Pmax, int Tp, int S, int step,
                     int32_t* kofs, int32_t* klen, int32_t* ksh, int32_t* pcol, int32_t* krow_pad, int32_t* zrow,
                     hipStream_t s);
// Contraction slices of the shared expert's weight gradients (a function of
// the padded token count Tp): S slices of `step` columns, step % kPadK == 0.
constexpr int kMaxSplitK = 4;
inline int splitk_count(long long Tp) { return (int)std::max(1LL, std::min<long long>(kMaxSplitK, Tp / 4096)); }
inline long long splitk_step(long long Tp) { return pad_k((Tp + splitk_count(Tp) - 1) / splitk_count(Tp)); }
void launch_splitk_reduce(const float* part, long long n, int S, float* out, hipStream_t s);   // n % 4 == 0
void launch_transpose(int act, const TransposeArgs& a, hipStream_t s);
void launch_bwd_gate(int act, const void* dy, const void* ou, const void* x, const void* wr, const int32_t* idx,
                     const float* gate, const int32_t* pos, int T, int d, int k, float* dl, int32_t* krow,
                     hipStream_t s);
void launch_bwd_dwr(int act, const void* x, const float* dl, const int32_t* perm, const int32_t* pcol, int P,
                    const int32_t* kofs, const int32_t* klen, int E, int d, int k, float* part, float* dwr,
                    hipStream_t s);
void launch_bwd_dx(int act, const void* dxs, const void* dxp, const void* wr, const float* dl, const int32_t* idx,
                   const int32_t* pos, int T, int d, int k, void* dx, hipStream_t s);

// y[t] = S_0[t] + ... + S_{nS-1}[t] + sum_j O[pos[t*k + j]] (+ resid[t]) in
// that order, rounded once.  The S_z ([T, d] each, consecutive) are the
// contraction slices of the shared down; resid (may be null) is the MoE
// block's residual input.
void launch_combine(int act, const void* S, int nS, const void* O, const int32_t* pos, int T, int d, int k,
                    const void* resid, void* y, hipStream_t s);

// x = bf16(h / sqrt(mean(h^2) + eps) * gamma) per row (block.hip); bf16 h and
// x [T, d], gamma [d] float32, d a multiple of 8 and at most 8 * 64 *
// kNormMaxVec.
constexpr int kNormMaxVec = 16;
void launch_rmsnorm(const void* h, const float* gamma, float eps, int T, int d, void* x, hipStream_t s);

}  // namespace fgmoe
