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
// 2.7B MoE for $200" (opening section, architecture paragraph).
//
// Tiling: a 256-thread workgroup (4 waves, 2 x 2) computes a 128 x 128 tile;
// each wave owns 64 x 64 = 4 x 4 MFMA 16x16 tiles.  K advances in 128-byte
// row chunks (64 bf16 or 32 float) staged through LDS, double-buffered, with
// the 16-byte pieces of each row XOR-swizzled by (row & 7) against bank
// conflicts.  Each lane's MFMA operand is 32 contiguous bytes of its row.
//
// Scheduling: work items are 128-row tiles (dense: row blocks; grouped: the
// tile table the router wrote, in expert order).  Workgroups are dealt to the
// 8 XCDs round-robin by block index, so block b runs on XCD b % 8; XCD x gets
// the contiguous item range [x*q, (x+1)*q) and runs all N tiles of an item
// back to back, keeping an item's A rows and an expert's weights in that
// XCD's L2.  No host synchronisation: the item count is read on the device.
#include "common.h"
#include "kernels.h"

namespace fgmoe {

namespace {

constexpr int BM = 128, BN = 128, NTHR = 256;
constexpr int ROWB = 128;                    // bytes of one row per K stage
constexpr int TILEB = BM * ROWB;             // bytes of one operand tile per stage

__device__ __forceinline__ int swz(int row, int piece) { return row * ROWB + ((piece ^ (row & 7)) << 4); }

template <typename T, int EPI, bool GATHER>
__global__ __launch_bounds__(NTHR, 2) void gemm_kernel(GemmArgs p) {
  __shared__ __attribute__((aligned(16))) char lds[2 * 2 * TILEB];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;

  // ---- work item
  const int count = p.grouped ? *p.tile_count : (p.M + BM - 1) / BM;
  const int q = (count + 7) >> 3;
  const int nbn = (EPI == EPI_SWIGLU) ? p.N / 64 : p.N / BN;
  const int bid = blockIdx.x;
  const int xcd = bid & 7, local = bid >> 3;
  const int pi = local / nbn, nt = local - pi * nbn;
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

  // ---- global -> LDS assignment: thread loads 16-byte piece c16 of rows r0 + 32 i
  const int c16 = tid & 7, r0 = tid >> 3;
  const char* a_ptr[4];
  bool a_ok[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = r0 + 32 * i;
    a_ok[i] = r < rows;
    long long arow = 0;
    if (a_ok[i]) arow = GATHER ? (long long)(p.a_rows[row_base + r] / p.a_div) : (long long)(row_base + r);
    a_ptr[i] = reinterpret_cast<const char*>(p.A) + (arow * p.lda) * (long long)sizeof(T) + c16 * 16;
  }
  const char* bbase = reinterpret_cast<const char*>(p.B) + (long long)e * p.b_estride * (long long)sizeof(T);
  const char* b_ptr[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int n = r0 + 32 * i;
    long long brow;
    if (EPI == EPI_SWIGLU)
      brow = n < 64 ? (long long)nt * 64 + n : (long long)p.up_off + nt * 64 + (n - 64);
    else
      brow = (long long)nt * BN + n;
    b_ptr[i] = bbase + brow * p.ldb * (long long)sizeof(T) + c16 * 16;
  }

  const int nk = (int)((long long)p.K * sizeof(T) / ROWB);
  const u32x4_t z = {0u, 0u, 0u, 0u};
  u32x4_t ra[4], rb[4];
  auto gload = [&](int s) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      ra[i] = a_ok[i] ? ld16(a_ptr[i] + (long long)s * ROWB) : z;
      rb[i] = ld16(b_ptr[i] + (long long)s * ROWB);
    }
  };
  auto lstore = [&](int buf) {
    char* As = lds + buf * 2 * TILEB;
    char* Bs = As + TILEB;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = r0 + 32 * i;
      st16(As + swz(r, c16), ra[i]);
      st16(Bs + swz(r, c16), rb[i]);
    }
  };

  // ---- LDS -> MFMA operand rows for this wave
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

  gload(0);
  lstore(0);
  __syncthreads();
  for (int s = 0; s < nk; ++s) {
    const int buf = s & 1;
    if (s + 1 < nk) gload(s + 1);
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
    if (s + 1 < nk) lstore(buf ^ 1);
    __syncthreads();
  }

  // ---- epilogue.  acc[mi][ni][i] is row wm*64 + mi*16 + 4g + i, column (wave
  // column base) + ni*16 + fr.
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
#pragma unroll
        for (int ni = 0; ni < 2; ++ni) {
          const int f = nt * 64 + wn * 32 + ni * 16 + fr;
          const float a = acc[mi][ni][i], u = acc[mi][ni + 2][i];
          C[row * p.ldc + f] = from_f32<T>(siluf_(a) * u);
          if (aux) {
            aux[row * p.ldaux + f] = from_f32<T>(a);
            aux[row * p.ldaux + p.N + f] = from_f32<T>(u);
          }
        }
      } else if (EPI == EPI_ROWSCALE) {
        const float sc = p.gate[p.perm[row]];
#pragma unroll
        for (int ni = 0; ni < 4; ++ni) {
          const int n = nt * BN + wn * 64 + ni * 16 + fr;
          C[row * p.ldc + n] = from_f32<T>(acc[mi][ni][i] * sc);
          if (aux) aux[row * p.ldaux + n] = from_f32<T>(acc[mi][ni][i]);
        }
      } else {  // EPI_COMBINE: row is a token
        const T* O = reinterpret_cast<const T*>(p.O);
        int slot[8];
#pragma unroll
        for (int j = 0; j < 8; ++j)
          if (j < p.k) slot[j] = p.pos[row * p.k + j];
#pragma unroll
        for (int ni = 0; ni < 4; ++ni) {
          const int n = nt * BN + wn * 64 + ni * 16 + fr;
          float v = acc[mi][ni][i];
#pragma unroll
          for (int j = 0; j < 8; ++j)
            if (j < p.k) v += to_f32<T>(O[(long long)slot[j] * p.ldo + n]);
          C[row * p.ldc + n] = from_f32<T>(v);
        }
      }
    }
  }
}

template <typename T, int EPI, bool GATHER>
void launch_t(const GemmArgs& a, hipStream_t s) {
  const int nbn = (EPI == EPI_SWIGLU) ? a.N / 64 : a.N / BN;
  const long long groups = (a.max_items + 7) / 8;
  const long long blocks = groups * 8 * nbn;
  if (blocks == 0) return;
  hipLaunchKernelGGL((gemm_kernel<T, EPI, GATHER>), dim3((unsigned)blocks), dim3(NTHR), 0, s, a);
}

template <typename T>
void launch_dtype(const GemmArgs& a, hipStream_t s) {
  const bool gather = a.a_rows != nullptr;
  switch (a.epi) {
    case EPI_SWIGLU:
      if (gather) launch_t<T, EPI_SWIGLU, true>(a, s);
      else launch_t<T, EPI_SWIGLU, false>(a, s);
      break;
    case EPI_ROWSCALE: launch_t<T, EPI_ROWSCALE, false>(a, s); break;
    default: launch_t<T, EPI_COMBINE, false>(a, s); break;
  }
}

}  // namespace

void launch_gemm(const GemmArgs& a, hipStream_t s) {
  if (a.act == 1) launch_dtype<bf16_t>(a, s);
  else launch_dtype<float>(a, s);
}

}  // namespace fgmoe
