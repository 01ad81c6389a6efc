// bf16 MFMA tile engine for gfx950: C[BM x BN] += A[BM x K] * B[BN x K]^T.
//
// One workgroup = 4 waves in a 2 x 2 grid; each wave owns a (BM/2) x (BN/2)
// sub-tile made of 16 x 16 fragments computed with v_mfma_f32_16x16x32_bf16.
// K advances in steps of 64: each step stages A and B through LDS (two
// buffers, plus two register stages of global loads in flight), rows padded
// by 16 bytes to spread LDS banks.
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

// Staging registers and loaders for one K step of A (K-contiguous rows) and
// of B, either K-contiguous rows ("NT") or stored [K][N] ("NN", transposed
// into the same LDS layout while it is stored).
template <class Cfg>
struct RegsNT {
  u32x4 a[Cfg::A_LOADS];
  u32x4 b[Cfg::B_LOADS];
};

// a[i] / b[i]: start (already offset by this thread's 8-element column chunk)
// of the i-th row this thread loads; rows past the valid range point at some
// valid row, their results are discarded by the epilogue.
template <class Cfg>
struct LoaderNT {
  typedef RegsNT<Cfg> Regs;
  const bf16_t* a[Cfg::A_LOADS];
  const bf16_t* b[Cfg::B_LOADS];
  __device__ __forceinline__ void load(Regs& r, int kt) const {
    const int k0 = kt * Cfg::BK;
    gload_rows(r.a, a, k0);
    gload_rows(r.b, b, k0);
  }
  __device__ __forceinline__ void store(bf16_t* As, bf16_t* Bs, const Regs& r) const {
    const int lrow = threadIdx.x / Cfg::CHUNKS_PER_ROW, lcol = (threadIdx.x % Cfg::CHUNKS_PER_ROW) * 8;
    sstore_rows<Cfg>(As, r.a, lrow, lcol);
    sstore_rows<Cfg>(Bs, r.b, lrow, lcol);
  }
};

// B stored [K][N]: load 8 consecutive n of one k per 16-byte chunk; columns
// at or past n_valid are clamped to the last valid column.
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

template <class Cfg>
struct RegsNN {
  u32x4 a[Cfg::A_LOADS];
  u32x4 b[Cfg::NN_B_LOADS];
};

template <class Cfg>
struct LoaderNN {
  typedef RegsNN<Cfg> Regs;
  const bf16_t* a[Cfg::A_LOADS];
  const bf16_t* b_base;  // B[0][n0]
  int64_t ldb;
  int n_valid;
  __device__ __forceinline__ void load(Regs& r, int kt) const {
    const int k0 = kt * Cfg::BK;
    const int nk_row = threadIdx.x / Cfg::NN_CHUNKS_PER_K;
    const int nn_col = (threadIdx.x % Cfg::NN_CHUNKS_PER_K) * 8;
    gload_rows(r.a, a, k0);
    gload_nn<Cfg>(r.b, b_base, ldb, k0, nk_row, nn_col, n_valid, nn_col + 8 <= n_valid);
  }
  __device__ __forceinline__ void store(bf16_t* As, bf16_t* Bs, const Regs& r) const {
    const int lrow = threadIdx.x / Cfg::CHUNKS_PER_ROW, lcol = (threadIdx.x % Cfg::CHUNKS_PER_ROW) * 8;
    sstore_rows<Cfg>(As, r.a, lrow, lcol);
    sstore_nn<Cfg>(Bs, r.b, threadIdx.x / Cfg::NN_CHUNKS_PER_K, (threadIdx.x % Cfg::NN_CHUNKS_PER_K) * 8);
  }
};

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

// Persistent GEMM driver with register-staged loads (used where B must be
// transposed on its way into LDS). The workgroup's items (XCD-aware split,
// see xcd_split) are walked as one flat sequence of K steps, so the pipeline
// never drains between items: while the MFMAs of step g run from one LDS
// buffer, step g+1 is in flight into registers; when step g closes an item,
// its epilogue runs while the next item's first step is loading.
//   Prob::setup(item, loader)   row pointers of an item
//   Prob::epilogue(item, acc)   consume one finished tile
template <class Cfg, class Loader, class Prob>
__device__ __forceinline__ void persistent_gemm(Prob& pb, int items, int nk, bf16_t* smem) {
  const XcdSplit sp = xcd_split(items);
  if (sp.first >= sp.end || nk <= 0) return;
  const int n_mine = (sp.end - sp.first + sp.stride - 1) / sp.stride;
  const int total = n_mine * nk;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  bf16_t* const A0 = smem;
  bf16_t* const B0 = smem + 2 * Cfg::A_ELEMS;
  Loader ld;
  typename Loader::Regs r0;
  int l_ord = 0, l_kt = 0;  // load cursor: item ordinal and K step
  pb.setup(sp.first, ld);
  ld.load(r0, 0);
  ld.store(A0, B0, r0);
  if (++l_kt == nk) {
    l_kt = 0;
    if (++l_ord < n_mine) pb.setup(sp.first + l_ord * sp.stride, ld);
  }
  __syncthreads();
  Acc<Cfg> acc;
  acc.zero();
  int c_kt = 0, c_ord = 0;  // compute cursor
  for (int g = 0; g < total; ++g) {
    const int cur = g & 1;
    const bool more = g + 1 < total;
    if (more) ld.load(r0, l_kt);
    mfma_step<Cfg>(A0 + cur * Cfg::A_ELEMS, B0 + cur * Cfg::B_ELEMS, acc, wm, wn, lane);
    if (more) {
      ld.store(A0 + (cur ^ 1) * Cfg::A_ELEMS, B0 + (cur ^ 1) * Cfg::B_ELEMS, r0);
      if (++l_kt == nk) {
        l_kt = 0;
        if (++l_ord < n_mine) pb.setup(sp.first + l_ord * sp.stride, ld);
      }
    }
    __syncthreads();
    if (++c_kt == nk) {
      pb.epilogue(sp.first + c_ord * sp.stride, acc);
      acc.zero();
      c_kt = 0;
      ++c_ord;
    }
  }
}

// ===================================================== LDS-DMA pipeline ===
//
// For operands that are K-contiguous rows (A and B "NT"), global memory is
// copied straight into LDS with global_load_lds_dwordx4 (each lane moves 16
// bytes; the 64 lanes of one instruction fill 1 KB of LDS in lane order), so
// no registers hold tiles in transit and several K steps can be in flight.
//
// K step = 32. A stage holds A [BM][32] and B [BN][32] bf16 (64-byte rows,
// 16 rows per DMA instruction). To keep the MFMA fragment reads (16 rows x one
// 16-byte chunk per instruction) free of bank conflicts, the 16-byte chunk c
// of row r is stored at slot c ^ chunk_key(r): among any 8 consecutive rows
// (one 128-byte bank line holds two rows) the (row parity, slot) pairs are
// all distinct, and among any 16 consecutive rows the (row mod 4, slot)
// pairs are, so the read is conflict-free whether the LDS serves 8 or 16
// lanes of a 16-byte read per cycle.
// STAGES stages form a ring in one LDS array; stage g's slot is g % STAGES and
// STAGES - 1 stages are in flight while one is consumed.

typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(1))) void glb_void_t;

template <int BM_, int BN_, int STAGES_ = 4>
struct DmaCfg {
  static constexpr int BM = BM_;
  static constexpr int BN = BN_;
  static constexpr int BK = 32;
  static constexpr int STAGES = STAGES_;  // ring slots; STAGES - 1 stages in flight
  static constexpr int FM = BM / 32;  // fragments per wave along M (2 x 2 waves)
  static constexpr int FN = BN / 32;
  static constexpr int A_DMA = BM / 64;  // DMA instructions per wave per stage (16 rows each, 4 waves)
  static constexpr int B_DMA = BN / 64;
  static constexpr int DMA_PER_STAGE = A_DMA + B_DMA;
  static constexpr int A_ELEMS = BM * BK;
  static constexpr int B_ELEMS = BN * BK;
  static constexpr int STAGE_ELEMS = A_ELEMS + B_ELEMS;
  static_assert(BM % 64 == 0 && BN % 64 == 0, "DMA tiles are multiples of 64 rows");
  static_assert(STAGES >= 3 && (STAGES - 2) * DMA_PER_STAGE <= 63, "ring depth vs vmcnt");
};

// Per-thread source rows of one item: a[i] / b[i] point at the logical chunk
// this lane fetches ((lane & 3) ^ chunk_key(lane / 4)) of row 16 * (wave * X_DMA + i)
// + lane / 4 of the tile; set by Prob::setup.
// a_kstep / b_kstep: elements between consecutive K steps of one operand
// (32 for a row-major operand; one whole 8 KB tile for a packed one).
template <class Cfg>
struct DmaLoader {
  const bf16_t* a[Cfg::A_DMA];
  const bf16_t* b[Cfg::B_DMA];
  int a_kstep = Cfg::BK;
  int b_kstep = Cfg::BK;
};

// Swizzle key of tile row r (only r mod 16 matters): bit 0 = bit 2 of r,
// bit 1 = bit 1 ^ bit 3 of r. XOR with it maps chunk -> slot and back.
__host__ __device__ __forceinline__ int chunk_key(int r) {
  return ((r >> 2) & 1) | ((((r >> 1) ^ (r >> 3)) & 1) << 1);
}

// Row of the tile whose chunk this thread fetches in DMA instruction i, and
// the element offset of that chunk inside the row: lane l writes slot l % 4
// of row l / 4 of its 16-row group, so it fetches chunk (l % 4) ^ key.
__device__ __forceinline__ int dma_row(int x_dma, int i) {
  return 16 * ((int)(threadIdx.x >> 6) * x_dma + i) + ((threadIdx.x & 63) >> 2);
}
__device__ __forceinline__ int dma_chunk_elem() {
  const int lane = threadIdx.x & 63;
  return ((lane & 3) ^ chunk_key(lane >> 2)) * 8;
}

// One 16-byte-per-lane DMA: global -> LDS at lds + 16 * lane. Issued as
// inline assembly so the compiler's wait-count pass does not treat it as an
// LDS store: with many DMAs in flight it would otherwise make every LDS read
// wait for all of them. Completion is tracked explicitly instead
// (dma_wait_stage + barrier before a stage is read). M0 carries the LDS
// base; nothing else in these kernels uses M0.
__device__ __forceinline__ void dma16(const void* g, const bf16_t* lds) {
  const uint32_t a = (uint32_t)(uintptr_t)(lds_void_t*)lds;
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(g), "s"(a) : "memory");
}

template <class Cfg>
__device__ __forceinline__ void dma_issue(const DmaLoader<Cfg>& ld, int kt, bf16_t* As, bf16_t* Bs) {
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int64_t ka = (int64_t)kt * ld.a_kstep, kb = (int64_t)kt * ld.b_kstep;
#pragma unroll
  for (int i = 0; i < Cfg::A_DMA; ++i) dma16(ld.a[i] + ka, As + 16 * (wave * Cfg::A_DMA + i) * Cfg::BK);
#pragma unroll
  for (int i = 0; i < Cfg::B_DMA; ++i) dma16(ld.b[i] + kb, Bs + 16 * (wave * Cfg::B_DMA + i) * Cfg::BK);
}

// Packed B operand: the weight tile of one (n block, K step) stored as the
// exact image of its LDS stage (BN rows x 32, chunks swizzled as above), so
// a DMA instruction copies 1 KB of contiguous memory. Pointer for this lane's
// chunk of DMA instruction i, K step 0, given the tile's base.
template <class Cfg>
__device__ __forceinline__ const bf16_t* packed_b_ptr(const bf16_t* tile0, int i) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  return tile0 + (int64_t)(wave * Cfg::B_DMA + i) * 16 * Cfg::BK + lane * 8;
}
constexpr int kPackTileElems = 128 * 32;  // one packed weight tile: 128 rows x 32 (8 KB)

// One K step of 32 from a swizzled stage. The MFMA is fed (B, A) so that it
// produces C^T fragments: lane l then holds output row (l % 16) and the four
// consecutive output columns 4 * (l / 16) .. +3 of a 16 x 16 fragment, which
// the epilogues write as one 8- or 16-byte store instead of four scattered
// 2-byte ones (see dma_out_row / dma_out_col).
template <class Cfg>
__device__ __forceinline__ void dma_mfma(const bf16_t* As, const bf16_t* Bs, Acc<Cfg>& acc, int wm,
                                         int wn, int lane) {
  const int r = lane & 15;
  const int slot = (lane >> 4) ^ chunk_key(r);
  bf16x8 a[Cfg::FM], b[Cfg::FN];
#pragma unroll
  for (int i = 0; i < Cfg::FM; ++i)
    a[i] = *reinterpret_cast<const bf16x8*>(&As[(wm * (Cfg::BM / 2) + i * 16 + r) * Cfg::BK + slot * 8]);
#pragma unroll
  for (int j = 0; j < Cfg::FN; ++j)
    b[j] = *reinterpret_cast<const bf16x8*>(&Bs[(wn * (Cfg::BN / 2) + j * 16 + r) * Cfg::BK + slot * 8]);
#pragma unroll
  for (int i = 0; i < Cfg::FM; ++i)
#pragma unroll
    for (int j = 0; j < Cfg::FN; ++j)
      acc.v[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(b[j], a[i], acc.v[i][j], 0, 0, 0);
}

// Output coordinates (within the tile) of acc.v[i][j][r] for the DMA driver:
// row dma_out_row(i), column dma_out_col(j) + r, r = 0..3.
template <class Cfg>
__device__ __forceinline__ int dma_out_row(int wm, int i, int lane) {
  return wm * (Cfg::BM / 2) + i * 16 + (lane & 15);
}
template <class Cfg>
__device__ __forceinline__ int dma_out_col(int wn, int j, int lane) {
  return wn * (Cfg::BN / 2) + j * 16 + (lane >> 4) * 4;
}

// s_waitcnt with vmcnt = n (n < 64) and the other counters left alone: vmcnt
// lives in bits [3:0] and [15:14], expcnt [6:4], lgkmcnt [11:8]. The count
// must be an immediate, hence the table.
#define MOE_VMCNT(n) \
  case n: __builtin_amdgcn_s_waitcnt(((n) & 15) | (((n) >> 4) << 14) | (7 << 4) | (15 << 8)); break;
#define MOE_VMCNT8(b) MOE_VMCNT(b) MOE_VMCNT(b + 1) MOE_VMCNT(b + 2) MOE_VMCNT(b + 3) \
  MOE_VMCNT(b + 4) MOE_VMCNT(b + 5) MOE_VMCNT(b + 6) MOE_VMCNT(b + 7)
__device__ __forceinline__ void wait_vmcnt(int n) {
  switch (n) {
    MOE_VMCNT8(0) MOE_VMCNT8(8) MOE_VMCNT8(16) MOE_VMCNT8(24)
    MOE_VMCNT8(32) MOE_VMCNT8(40) MOE_VMCNT8(48) MOE_VMCNT8(56)
    default: __builtin_amdgcn_s_waitcnt((7 << 4) | (15 << 8)); break;  // vmcnt(0)
  }
}
#undef MOE_VMCNT8
#undef MOE_VMCNT
template <int N>
__device__ __forceinline__ void wait_vmcnt_imm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Before reading stage g: wait until this wave's DMAs of stage g have landed.
// Vector-memory operations complete in order for the counter's purposes only
// among loads; the operations issued after stage g's DMAs are the DMAs of the
// younger stages in flight plus the epilogue stores of the last three steps
// (stores share the counter on this GPU). Allowing exactly that many keeps the
// stores from draining the pipeline; any count that is not exactly known
// (younger_stores < 0) or does not fit the counter falls back to counting the
// DMAs only, which waits longer and is always safe. Both arguments are
// wave-uniform; the steady state (full ring, no recent stores) takes one
// immediate wait, the rest a scalar branch table.
template <class Cfg>
__device__ __forceinline__ void dma_wait_stage(int younger_stages, int younger_stores) {
  if (younger_stages == Cfg::STAGES - 2 && younger_stores == 0) {
    wait_vmcnt_imm<(Cfg::STAGES - 2) * Cfg::DMA_PER_STAGE>();
    return;
  }
  int n = younger_stages * Cfg::DMA_PER_STAGE;
  if (younger_stores > 0 && n + younger_stores <= 63) n += younger_stores;
  wait_vmcnt(n);
}

// Persistent driver on the DMA ring. Same contract as persistent_gemm, with
// Prob::setup filling a DmaLoader and Prob::epilogue returning the number of
// vector-memory store instructions the calling wave issued (-1 if not exactly
// known, e.g. when the epilogue also loads). The ring has STAGES slots in one
// LDS array; stage g lives in slot g % STAGES. Step g:
//   wait for own DMAs of stage g, barrier (everyone's DMAs of g landed, and
//   everyone finished reading slot (g-1) % STAGES), issue stage
//   g + STAGES - 1 into that slot, MFMAs of stage g, epilogue if g closes an
//   item.
// The barrier is a bare s_barrier: the explicit vmcnt wait before it already
// orders this wave's DMA writes, and a fenced barrier would wait for every
// stage in flight.
template <class Cfg, class Prob>
__device__ __forceinline__ void persistent_gemm_dma(Prob& pb, int items, int nk) {
  constexpr int S = Cfg::STAGES;
  __shared__ __align__(16) bf16_t ring[S * Cfg::STAGE_ELEMS];
  const XcdSplit sp = xcd_split(items);
  if (sp.first >= sp.end || nk <= 0) return;
  const int n_mine = (sp.end - sp.first + sp.stride - 1) / sp.stride;
  const int total = n_mine * nk;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  DmaLoader<Cfg> ld;
  int l_ord = 0, l_kt = 0;  // load cursor
  int l_slot = 0;           // ring slot of the next stage to load
  pb.setup(sp.first, ld);

#define MOE_DMA_NEXT()                                                         \
  {                                                                            \
    bf16_t* st_ = ring + l_slot * Cfg::STAGE_ELEMS;                            \
    dma_issue<Cfg>(ld, l_kt, st_, st_ + Cfg::A_ELEMS);                         \
    l_slot = (l_slot + 1 == S) ? 0 : l_slot + 1;                               \
    if (++l_kt == nk) {                                                        \
      l_kt = 0;                                                                \
      if (++l_ord < n_mine) pb.setup(sp.first + l_ord * sp.stride, ld);        \
    }                                                                          \
  }

  // prologue: stages 0 .. S-2 in flight
  for (int p = 0; p < S - 1 && p < total; ++p) MOE_DMA_NEXT();
  Acc<Cfg> acc;
  acc.zero();
  int c_kt = 0, c_ord = 0, c_slot = 0;
  // store instructions issued by the epilogues of the last S-1 steps (< 0:
  // not exactly known); they were issued after the DMAs of the stage awaited
  int st_hist[S - 1];
#pragma unroll
  for (int i = 0; i < S - 1; ++i) st_hist[i] = 0;
  for (int g = 0; g < total; ++g) {
    int ys = 0;
#pragma unroll
    for (int i = 0; i < S - 1; ++i) ys = (ys < 0 || st_hist[i] < 0) ? -1 : ys + st_hist[i];
    dma_wait_stage<Cfg>(min(S - 2, total - 1 - g), ys);
    __builtin_amdgcn_s_barrier();
    if (g + S - 1 < total) MOE_DMA_NEXT();
    const bf16_t* st = ring + c_slot * Cfg::STAGE_ELEMS;
    dma_mfma<Cfg>(st, st + Cfg::A_ELEMS, acc, wm, wn, lane);
    c_slot = (c_slot + 1 == S) ? 0 : c_slot + 1;
#pragma unroll
    for (int i = S - 2; i > 0; --i) st_hist[i] = st_hist[i - 1];
    st_hist[0] = 0;
    if (++c_kt == nk) {
      // the count is wave-uniform; keep it (and the wait it selects) scalar
      st_hist[0] = __builtin_amdgcn_readfirstlane(pb.epilogue(sp.first + c_ord * sp.stride, acc));
      acc.zero();
      c_kt = 0;
      ++c_ord;
    }
  }
#undef MOE_DMA_NEXT
}

}  // namespace moe
