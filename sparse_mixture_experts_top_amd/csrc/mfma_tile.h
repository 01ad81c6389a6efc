// bf16 MFMA tile engine for gfx950: C[BM x BN] += A[BM x K] * B[BN x K]^T.
//
// One workgroup = 4 waves in a 2 x 2 grid; each wave owns a (BM/2) x (BN/2)
// sub-tile made of 16 x 16 fragments computed with v_mfma_f32_16x16x32_bf16.
// K advances in steps of 64: each step stages A and B through LDS (double
// buffered: the next step's global loads are in flight while the current
// step's MFMAs run), rows padded by 16 bytes to spread LDS banks.
//
// Fragment layout of the 16x16x32 bf16 MFMA: lane l supplies row (l % 16) of
// the A fragment and row (l % 16) of the B fragment (= column of B^T), each
// as 8 consecutive k values starting at 8 * (l / 16); it receives the four
// results C[4 * (l / 16) + i][l % 16], i = 0..3.
#pragma once

#include "common.h"

namespace moe {

template <int BM_, int BN_>
struct TileCfg {
  static constexpr int BM = BM_;
  static constexpr int BN = BN_;
  static constexpr int BK = 64;
  static constexpr int THREADS = 256;
  static constexpr int LDS_STRIDE = BK + 8;            // bf16 per LDS row
  static constexpr int FM = BM / 32;                   // fragments per wave along M
  static constexpr int FN = BN / 32;                   // fragments per wave along N
  static constexpr int CHUNKS_PER_ROW = BK / 8;        // 16-byte chunks per K-row
  static constexpr int ROWS_PER_PASS = THREADS / CHUNKS_PER_ROW;  // 32
  static constexpr int A_LOADS = BM / ROWS_PER_PASS;   // 16-byte loads per thread
  static constexpr int B_LOADS = BN / ROWS_PER_PASS;
  static constexpr int A_ELEMS = BM * LDS_STRIDE;
  static constexpr int B_ELEMS = BN * LDS_STRIDE;
  static constexpr int SMEM_BYTES = 2 * (A_ELEMS + B_ELEMS) * 2;
  // NN variant of B (B stored [K][N]): chunks of 8 consecutive n for one k.
  static constexpr int NN_CHUNKS_PER_K = BN / 8;
  static constexpr int NN_K_PER_PASS = THREADS / NN_CHUNKS_PER_K;
  static constexpr int NN_B_LOADS = BK / NN_K_PER_PASS;
  static_assert(BM % 32 == 0 && BN % 32 == 0, "tile must split over 2x2 waves of 16x16 fragments");
  static_assert(BM % ROWS_PER_PASS == 0 && BN % ROWS_PER_PASS == 0, "tile rows vs loader");
  static_assert(NN_K_PER_PASS > 0 && BK % NN_K_PER_PASS == 0, "NN loader");
};

template <class Cfg>
struct Acc {
  f32x4 v[Cfg::FM][Cfg::FN];
  __device__ __forceinline__ void zero() {
#pragma unroll
    for (int i = 0; i < Cfg::FM; ++i)
#pragma unroll
      for (int j = 0; j < Cfg::FN; ++j) v[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
};

// Row (within the tile) of value r of fragment (i, j) for this lane.
template <class Cfg>
__device__ __forceinline__ int frag_row(int wm, int i, int lane, int r) {
  return wm * (Cfg::BM / 2) + i * 16 + (lane >> 4) * 4 + r;
}
template <class Cfg>
__device__ __forceinline__ int frag_col(int wn, int j, int lane) {
  return wn * (Cfg::BN / 2) + j * 16 + (lane & 15);
}

template <class Cfg>
__device__ __forceinline__ void mfma_step(const bf16_t* As, const bf16_t* Bs, Acc<Cfg>& acc,
                                          int wm, int wn, int lane) {
#pragma unroll
  for (int kk = 0; kk < Cfg::BK / 32; ++kk) {
    bf16x8 a[Cfg::FM], b[Cfg::FN];
    const int koff = kk * 32 + (lane >> 4) * 8;
#pragma unroll
    for (int i = 0; i < Cfg::FM; ++i)
      a[i] = *reinterpret_cast<const bf16x8*>(
          &As[(wm * (Cfg::BM / 2) + i * 16 + (lane & 15)) * Cfg::LDS_STRIDE + koff]);
#pragma unroll
    for (int j = 0; j < Cfg::FN; ++j)
      b[j] = *reinterpret_cast<const bf16x8*>(
          &Bs[(wn * (Cfg::BN / 2) + j * 16 + (lane & 15)) * Cfg::LDS_STRIDE + koff]);
#pragma unroll
    for (int i = 0; i < Cfg::FM; ++i)
#pragma unroll
      for (int j = 0; j < Cfg::FN; ++j)
        acc.v[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[i], b[j], acc.v[i][j], 0, 0, 0);
  }
}

// 16 bytes as a native vector (HIP's uint4 is a struct, which keeps arrays of
// it from being promoted to registers).
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Global -> register staging of one K step (16-byte loads).
template <int N>
__device__ __forceinline__ void gload_rows(u32x4 (&r)[N], const bf16_t* const (&rows)[N], int k0) {
#pragma unroll
  for (int i = 0; i < N; ++i) r[i] = *reinterpret_cast<const u32x4*>(rows[i] + k0);
}

// Register -> LDS store of one K step; `lds` is the buffer base, rows of the
// tile are ROWS_PER_PASS apart for consecutive loads.
template <class Cfg, int N>
__device__ __forceinline__ void sstore_rows(bf16_t* lds, const u32x4 (&r)[N], int lrow, int lcol) {
#pragma unroll
  for (int i = 0; i < N; ++i)
    *reinterpret_cast<u32x4*>(&lds[(lrow + i * Cfg::ROWS_PER_PASS) * Cfg::LDS_STRIDE + lcol]) = r[i];
}

// Main loop with both operands K-contiguous ("NT"): a_rows[i] / b_rows[i] are
// the row starts (already offset by this thread's 8-element column chunk) of
// the rows this thread loads; rows past the valid range must point at some
// valid row (their results are discarded by the caller). K % 64 == 0.
// LDS holds [A0 | A1 | B0 | B1]; buffers are addressed by integer offsets so
// every access stays an LDS (ds_*) instruction.
template <class Cfg>
__device__ __forceinline__ void mainloop_nt(const bf16_t* const (&a_rows)[Cfg::A_LOADS],
                                            const bf16_t* const (&b_rows)[Cfg::B_LOADS], int K,
                                            Acc<Cfg>& acc, bf16_t* smem) {
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int lrow = tid / Cfg::CHUNKS_PER_ROW;
  const int lcol = (tid % Cfg::CHUNKS_PER_ROW) * 8;
  bf16_t* const A0 = smem;
  bf16_t* const B0 = smem + 2 * Cfg::A_ELEMS;
  u32x4 ra[Cfg::A_LOADS], rb[Cfg::B_LOADS];
  const int nk = K / Cfg::BK;

  gload_rows(ra, a_rows, 0);
  gload_rows(rb, b_rows, 0);
  sstore_rows<Cfg>(A0, ra, lrow, lcol);
  sstore_rows<Cfg>(B0, rb, lrow, lcol);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    const bool more = kt + 1 < nk;
    if (more) {
      gload_rows(ra, a_rows, (kt + 1) * Cfg::BK);
      gload_rows(rb, b_rows, (kt + 1) * Cfg::BK);
    }
    mfma_step<Cfg>(A0 + cur * Cfg::A_ELEMS, B0 + cur * Cfg::B_ELEMS, acc, wm, wn, lane);
    if (more) {
      sstore_rows<Cfg>(A0 + (cur ^ 1) * Cfg::A_ELEMS, ra, lrow, lcol);
      sstore_rows<Cfg>(B0 + (cur ^ 1) * Cfg::B_ELEMS, rb, lrow, lcol);
    }
    __syncthreads();
  }
}

// B stored [K][N] ("NN"): load 8 consecutive n of one k per 16-byte chunk;
// columns at or past n_valid are clamped to the last valid column.
template <class Cfg>
__device__ __forceinline__ void gload_nn(u32x4 (&r)[Cfg::NN_B_LOADS], const bf16_t* b_base,
                                         int64_t ldb, int k0, int nk_row, int nn_col, int n_valid,
                                         bool chunk_ok) {
#pragma unroll
  for (int i = 0; i < Cfg::NN_B_LOADS; ++i) {
    const bf16_t* src = b_base + (int64_t)(k0 + nk_row + i * Cfg::NN_K_PER_PASS) * ldb;
    if (chunk_ok) {
      r[i] = *reinterpret_cast<const u32x4*>(src + nn_col);
    } else {
      uint32_t t[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) t[u] = src[min(nn_col + u, n_valid - 1)];
      r[i] = u32x4{t[0] | t[1] << 16, t[2] | t[3] << 16, t[4] | t[5] << 16, t[6] | t[7] << 16};
    }
  }
}

// Transposing store: element (k, n) of the chunk goes to LDS row n, column k.
template <class Cfg>
__device__ __forceinline__ void sstore_nn(bf16_t* lds, const u32x4 (&r)[Cfg::NN_B_LOADS],
                                          int nk_row, int nn_col) {
#pragma unroll
  for (int i = 0; i < Cfg::NN_B_LOADS; ++i) {
    const int kr = nk_row + i * Cfg::NN_K_PER_PASS;
    const uint32_t w[4] = {r[i][0], r[i][1], r[i][2], r[i][3]};
#pragma unroll
    for (int u = 0; u < 8; ++u)
      lds[(nn_col + u) * Cfg::LDS_STRIDE + kr] = static_cast<bf16_t>(w[u >> 1] >> ((u & 1) * 16));
  }
}

// Main loop with A K-contiguous and B stored [K][N] ("NN"): b_base points at
// B[0][n0] (row stride ldb); columns n0 + c for c >= n_valid are clamped to
// column n0 + n_valid - 1. B is transposed into the same LDS layout as NT.
template <class Cfg>
__device__ __forceinline__ void mainloop_nn(const bf16_t* const (&a_rows)[Cfg::A_LOADS],
                                            const bf16_t* b_base, int64_t ldb, int n_valid,
                                            int K, Acc<Cfg>& acc, bf16_t* smem) {
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int lrow = tid / Cfg::CHUNKS_PER_ROW;
  const int lcol = (tid % Cfg::CHUNKS_PER_ROW) * 8;
  const int nk_row = tid / Cfg::NN_CHUNKS_PER_K;
  const int nn_col = (tid % Cfg::NN_CHUNKS_PER_K) * 8;
  const bool chunk_ok = nn_col + 8 <= n_valid;
  bf16_t* const A0 = smem;
  bf16_t* const B0 = smem + 2 * Cfg::A_ELEMS;
  u32x4 ra[Cfg::A_LOADS], rb[Cfg::NN_B_LOADS];
  const int nk = K / Cfg::BK;

  gload_rows(ra, a_rows, 0);
  gload_nn<Cfg>(rb, b_base, ldb, 0, nk_row, nn_col, n_valid, chunk_ok);
  sstore_rows<Cfg>(A0, ra, lrow, lcol);
  sstore_nn<Cfg>(B0, rb, nk_row, nn_col);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    const bool more = kt + 1 < nk;
    if (more) {
      gload_rows(ra, a_rows, (kt + 1) * Cfg::BK);
      gload_nn<Cfg>(rb, b_base, ldb, (kt + 1) * Cfg::BK, nk_row, nn_col, n_valid, chunk_ok);
    }
    mfma_step<Cfg>(A0 + cur * Cfg::A_ELEMS, B0 + cur * Cfg::B_ELEMS, acc, wm, wn, lane);
    if (more) {
      sstore_rows<Cfg>(A0 + (cur ^ 1) * Cfg::A_ELEMS, ra, lrow, lcol);
      sstore_nn<Cfg>(B0 + (cur ^ 1) * Cfg::B_ELEMS, rb, nk_row, nn_col);
    }
    __syncthreads();
  }
}

// Workgroup -> work item with the XCD-aware order: the hardware hands
// consecutive workgroup ids to the 8 XCDs in turn, so id b runs on XCD b % 8.
// Giving each XCD a contiguous range of items keeps items that share operands
// (neighbouring ids) inside one XCD's L2. Returns the first item of this
// workgroup and the stride to its next one, for `items` items and a grid that
// is a multiple of 8.
struct XcdSplit {
  int first, end, stride;
};
__device__ __forceinline__ XcdSplit xcd_split(int items) {
  const int xcd = blockIdx.x & 7;
  const int j = blockIdx.x >> 3;
  const int per_xcd = gridDim.x >> 3;
  const int chunk = (items + 7) >> 3;
  XcdSplit s;
  s.first = xcd * chunk + j;
  s.end = min(items, (xcd + 1) * chunk);
  s.stride = per_xcd;
  return s;
}

}  // namespace moe
