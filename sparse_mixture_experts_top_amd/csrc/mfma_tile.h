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

#include <type_traits>

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
// Wave roles. A workgroup has compute waves and producer waves (counts in
// DmaCfg). The producers issue every DMA of the ring and never store; the compute waves
// read LDS, run the MFMAs and write the results. On this GPU stores share
// the vector-memory counter with loads and the counter retires in issue
// order, so in a wave that both loads and stores, every load issued after an
// epilogue's stores could only be waited for once those stores were
// acknowledged - a bubble of a full write latency after every output tile.
// With the roles split, a producer's waits count its own DMAs only (a
// constant in the steady state) and the compute waves never wait on memory
// counters. Several producers share each stage's DMAs: one wave alone issues
// them too slowly to keep the memory system busy.
//
// K step = 32. A stage holds A [BM][32] and B [BN][32] bf16 (64-byte rows,
// 16 rows per DMA instruction). To keep the MFMA fragment reads (lane l reads
// 16-byte chunk l / 16 of row l % 16) free of bank conflicts, the chunk c of
// row r is stored at slot c ^ chunk_key(r) with chunk_key(r) = bits 1..2 of
// r. On gfx950 a ds_read_b128 of this pattern then runs at the LDS's full
// rate, 4 cycles (256 bytes per cycle) with no bank-conflict cycles, as the
// SQ_LDS_BANK_CONFLICT / SQ_LDS_IDX_ACTIVE counters show; unswizzled rows, or
// keys that are a permutation within every 4 rows of equal r mod 4, take 8
// cycles (2-way conflicts).
// STAGES stages form a ring in one LDS array; stage g's slot is g % STAGES and
// STAGES - 1 stages are in flight while one is consumed. With SB > 0 the two
// operands have rings of their own: A keeps STAGES slots, B gets SB slots and
// is fetched SB - STAGES stages further ahead (see persistent_gemm_dma).

typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(1))) void glb_void_t;


// Tile BM x BN, STAGES ring slots, CW compute waves (waves 0 .. CW-1) in a
// WM x (CW / WM) grid over the tile and PW producer waves (waves CW ..
// CW+PW-1; producer p issues the DMAs i with i % PW == p). A workgroup runs
// alone on its CU (THREADS = 64 (CW + PW)); the occupancy hint WAVES_PER_SIMD
// caps the registers per wave at 512 / WAVES_PER_SIMD. SB_ > 0 splits the
// ring: A in STAGES slots, B in SB_ slots.
template <int BM_, int BN_, int STAGES_ = 4, int WM_ = 2, int CW_ = 4, int PW_ = 4, int BK_ = 32, int SB_ = 0>
struct DmaCfg {
  static constexpr int BM = BM_;
  static constexpr int BN = BN_;
  static constexpr int BK = BK_;           // K values per stage: 32 or 64
  static constexpr int CPR = BK / 8;       // 16-byte chunks per LDS row
  static constexpr int RPD = 64 / CPR;     // rows per DMA instruction (1 KB)
  static constexpr int KSUB = BK / 32;     // MFMA K steps per stage
  static constexpr int STAGES = STAGES_;  // ring slots; STAGES - 1 stages in flight
  static constexpr int CW = CW_;
  static constexpr int PW = PW_;  // 0: symmetric, every wave computes and issues DMAs
  static constexpr int DW = PW_ > 0 ? PW_ : CW_;  // waves sharing the DMAs of a stage
  static constexpr int THREADS = 64 * (CW + PW);
  static constexpr int WAVES_PER_SIMD = (CW + PW + 3) / 4;
  static constexpr int WM = WM_;          // the compute waves form a WM x WN grid over the tile
  static constexpr int WN = CW_ / WM_;
  static constexpr int FM = BM / (16 * WM);  // 16 x 16 fragments per wave along M
  static constexpr int FN = BN / (16 * WN);
  static constexpr int A_DMA = BM / RPD;  // DMA instructions per stage (RPD rows each)
  static constexpr int B_DMA = BN / RPD;
  static constexpr int DMA_PER_STAGE = A_DMA + B_DMA;
  static constexpr int A_ELEMS = BM * BK;
  static constexpr int B_ELEMS = BN * BK;
  static constexpr int STAGE_ELEMS = A_ELEMS + B_ELEMS;
  static_assert(WM == 1 || WM == 2 || WM == 4, "wave grid");
  static_assert(FM >= 1 && FN >= 1 && FM * 16 * WM == BM && FN * 16 * WN == BN, "fragments");
  static_assert(BK == 32 || BK == 64, "stage depth");
  static_assert(BM % 16 == 0 && BN % 16 == 0, "fragments are 16 rows");
  // B instructions per DMA wave and stage: with B_DMA % DW != 0 (symmetric
  // drivers only) the last round's missing instructions repeat instruction
  // B_DMA - 1 (the same rows into the same LDS rows; see b_inst)
  static constexpr int B_Q = (B_DMA + DW - 1) / DW;
  static constexpr int DMA_PER_PRODUCER = A_DMA / DW + B_Q;  // per stage and DMA wave
  static_assert(A_DMA % DW == 0 && (B_DMA % DW == 0 || PW_ == 0), "DMA split");
  static_assert(CW % WM == 0, "wave grid");
  static_assert(STAGES >= 2 && (STAGES - 2) * DMA_PER_PRODUCER <= 63, "ring depth vs vmcnt");
  // split ring: B slots, the lead of B over A in stages, LDS elements
  static constexpr int SB = SB_;
  static constexpr bool SPLIT = SB_ > 0;
  static constexpr int B_LEAD = SPLIT ? SB_ - STAGES_ : 0;
  static constexpr int A_PER = A_DMA / DW, B_PER = B_Q;  // per stage and producer
  static constexpr int RING_ELEMS = SPLIT ? STAGES * A_ELEMS + SB * B_ELEMS : STAGES * STAGE_ELEMS;
  static_assert(!SPLIT || (SB_ > STAGES_ && PW_ > 0 && STAGES_ >= 2), "split ring: producers, B ring deeper");
  static_assert(!SPLIT || (STAGES_ - 1) * A_PER + (SB_ - 1) * B_PER <= 63, "split ring vs vmcnt");
};

// Lane pointers of one producer for one item: a[q] / b[q] belong to the
// producer's q-th DMA instruction of each operand, i = q * DW + part,
// and point at the logical chunk this lane fetches ((lane & 3) ^
// chunk_key(lane / 4)) of tile row 16 i + lane / 4; set by
// Prob::setup(item, ld, part).
// a_kstep / b_kstep: elements between consecutive K steps of one operand
// (32 for a row-major operand; one whole packed tile for a packed one).
// b_stream: every B line is read by this item only (streamed weight tiles),
// so B is fetched with the non-temporal hint (see dma16_nt).
template <class Cfg>
struct DmaLoader {
  const bf16_t* a[Cfg::A_DMA / Cfg::DW];
  const bf16_t* b[Cfg::B_Q];
  int a_kstep = Cfg::BK;
  int b_kstep = Cfg::BK;
  bool b_stream = false;
};

// Swizzle key of tile row r for 64-byte rows (4 chunks; BK = 32, also the
// packed weight layout): bits 1..2 of r. XOR with it maps chunk -> slot and
// back.
__host__ __device__ __forceinline__ int chunk_key(int r) { return (r >> 1) & 3; }
// For 128-byte rows (8 chunks; BK = 64): bits 0..2 of r. The fragment read of
// either K half (chunks 0..3 or 4..7 of rows r = lane % 16) is then
// conflict-free on gfx950 as well (4 LDS cycles per ds_read_b128, measured).
template <class Cfg>
__device__ __forceinline__ int lds_key(int r) {
  return Cfg::CPR == 4 ? chunk_key(r) : (r & 7);
}

// Tile row whose chunk this (producer) lane fetches in DMA instruction i, and
// the element offset of that chunk inside the row: lane l writes slot
// l % CPR of row l / CPR of the instruction's RPD-row group, so it fetches
// chunk (l % CPR) ^ key.
template <class Cfg>
__device__ __forceinline__ int dma_row(int i) {
  return Cfg::RPD * i + (int)(threadIdx.x & 63) / Cfg::CPR;
}
template <class Cfg>
__device__ __forceinline__ int dma_chunk_elem() {
  const int lane = threadIdx.x & 63;
  return ((lane % Cfg::CPR) ^ lds_key<Cfg>(lane / Cfg::CPR)) * 8;
}

// One 16-byte-per-lane DMA: global -> LDS at lds + 16 * lane. Issued as
// inline assembly so the compiler's wait-count pass does not treat it as an
// LDS store: with many DMAs in flight it would otherwise make every LDS read
// wait for all of them. Completion is tracked explicitly instead (the
// producer's vmcnt wait + the barrier before a stage is read). M0 carries the
// LDS base; nothing else in these kernels uses M0.
__device__ __forceinline__ void dma16(const void* g, const bf16_t* lds) {
  const uint32_t a = (uint32_t)(uintptr_t)(lds_void_t*)lds;
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(g), "s"(a) : "memory");
}

// The same with the non-temporal hint, for an operand every line of which is
// read by one workgroup only (streamed weight tiles): the L2 then evicts those
// lines first and keeps the operand tiles that neighbouring CUs share (a
// 320-row expert tile's token rows, read by all its column blocks), which
// the streamed weights otherwise push out (ep64 gate/up 119 -> 110 us).
__device__ __forceinline__ void dma16_nt(const void* g, const bf16_t* lds) {
  const uint32_t a = (uint32_t)(uintptr_t)(lds_void_t*)lds;
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off nt" ::"v"(g), "s"(a) : "memory");
}

// Producer `part`'s share of the DMA instructions of K step kt: A
// instructions i with i % DW == part into the A part of a stage at a_dst, B
// ones into the B part at b_dst; dma_issue does both, A first.
template <class Cfg>
__device__ __forceinline__ void dma_issue_a(const DmaLoader<Cfg>& ld, int kt, bf16_t* a_dst, int part) {
  const int64_t ka = (int64_t)kt * ld.a_kstep;
#pragma unroll
  for (int q = 0; q < Cfg::A_DMA / Cfg::DW; ++q)
    dma16(ld.a[q] + ka, a_dst + Cfg::RPD * (q * Cfg::DW + part) * Cfg::BK);
}
// B instruction of round q for DMA wave `part` (repeats the last one when
// the waves do not split B evenly).
template <class Cfg>
__device__ __forceinline__ int b_inst(int q, int part) {
  return Cfg::B_DMA % Cfg::DW == 0 ? q * Cfg::DW + part : min(q * Cfg::DW + part, Cfg::B_DMA - 1);
}
template <class Cfg>
__device__ __forceinline__ void dma_issue_b(const DmaLoader<Cfg>& ld, int kt, bf16_t* b_dst, int part) {
  const int64_t kb = (int64_t)kt * ld.b_kstep;
  if (ld.b_stream) {  // wave-uniform
#pragma unroll
    for (int q = 0; q < Cfg::B_Q; ++q)
      dma16_nt(ld.b[q] + kb, b_dst + Cfg::RPD * b_inst<Cfg>(q, part) * Cfg::BK);
  } else {
#pragma unroll
    for (int q = 0; q < Cfg::B_Q; ++q)
      dma16(ld.b[q] + kb, b_dst + Cfg::RPD * b_inst<Cfg>(q, part) * Cfg::BK);
  }
}
template <class Cfg>
__device__ __forceinline__ void dma_issue(const DmaLoader<Cfg>& ld, int kt, bf16_t* stage, int part) {
  dma_issue_a<Cfg>(ld, kt, stage, part);
  dma_issue_b<Cfg>(ld, kt, stage + Cfg::A_ELEMS, part);
}

// Packed B operand: a weight tile of 128 rows x one K step stored as the
// exact image of its part of an LDS stage (chunks swizzled as above), so a
// DMA instruction copies 1 KB of contiguous memory. A B stage of BN rows
// spans BN / 128 such tiles. Pointer for this lane's chunk of DMA
// instruction i (rows 16 i .. 16 i + 15 of the stage) at K step 0, given the
// base of the stage's first tile and the element distance between the tiles
// of consecutive 128-row blocks.
constexpr int kPackTileRows = 128;
constexpr int kPackTileElems = kPackTileRows * 32;  // one packed weight tile (8 KB)
__device__ __forceinline__ const bf16_t* packed_b_ptr(const bf16_t* tile0, int i, int64_t block_stride) {
  constexpr int per_tile = kPackTileRows / 16;  // DMA instructions per tile
  return tile0 + (i / per_tile) * block_stride + (int64_t)(i % per_tile) * 16 * 32 + (threadIdx.x & 63) * 8;
}

// First tile row of row fragment i of wave row wm. Row fragments are
// interleaved over the wave rows (wave row wm holds fragments wm, wm + WM,
// ...), so when a partly filled row tile skips its padding fragments, the
// remaining work stays spread over all wave rows.
template <class Cfg>
__device__ __forceinline__ int frag_row0(int wm, int i) {
  return 16 * (i * Cfg::WM + wm);
}

// Operand fragments of one K step for one compute wave: FN B fragments and
// all FM A fragments (padding rows included; they are in bounds).
template <class Cfg>
struct Frags {
  bf16x8 a[Cfg::FM], b[Cfg::FN];
};

// LDS reads of the wave's fragments of a stage whose A and B parts are at
// As and Bs (read_frags: one slot of the joint ring at `st`).
template <class Cfg>
__device__ __forceinline__ void read_frags_ab(Frags<Cfg>& fr, const bf16_t* As, const bf16_t* Bs, int wm, int wn,
                                              int lane, int sub = 0) {
  const int r = lane & 15;
  const int slot = ((lane >> 4) + 4 * sub) ^ lds_key<Cfg>(r);
#pragma unroll
  for (int j = 0; j < Cfg::FN; ++j)
    fr.b[j] = *reinterpret_cast<const bf16x8*>(&Bs[(wn * (Cfg::BN / Cfg::WN) + j * 16 + r) * Cfg::BK + slot * 8]);
#pragma unroll
  for (int i = 0; i < Cfg::FM; ++i)
    fr.a[i] = *reinterpret_cast<const bf16x8*>(&As[(frag_row0<Cfg>(wm, i) + r) * Cfg::BK + slot * 8]);
}
template <class Cfg>
__device__ __forceinline__ void read_frags(Frags<Cfg>& fr, const bf16_t* st, int wm, int wn, int lane,
                                           int sub = 0) {
  read_frags_ab<Cfg>(fr, st, st + Cfg::A_ELEMS, wm, wn, lane, sub);
}

// Read cursor of the compute waves over the ring: the A and B parts of the
// next stage to read, advanced one stage at a time.
template <class Cfg>
struct RingCursor {
  const bf16_t* ring;
  int sa = 1 % Cfg::STAGES, sb = 1 % (Cfg::SPLIT ? Cfg::SB : 1);
  __device__ __forceinline__ const bf16_t* a() const {
    return Cfg::SPLIT ? ring + sa * Cfg::A_ELEMS : ring + sa * Cfg::STAGE_ELEMS;
  }
  __device__ __forceinline__ const bf16_t* b() const {
    return Cfg::SPLIT ? ring + Cfg::STAGES * Cfg::A_ELEMS + sb * Cfg::B_ELEMS : a() + Cfg::A_ELEMS;
  }
  __device__ __forceinline__ void advance() {
    sa = (sa + 1 == Cfg::STAGES) ? 0 : sa + 1;
    if (Cfg::SPLIT) sb = (sb + 1 == Cfg::SB) ? 0 : sb + 1;
  }
};

// Workgroup barrier without a memory fence (see persistent_gemm_dma), with
// compiler-level memory clobbers on both sides: the s_barrier intrinsic is
// not a memory operation to the optimiser, which could otherwise move LDS
// reads across it.
__device__ __forceinline__ void ring_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// s_waitcnt lgkmcnt(0) with the other counters left alone.
__device__ __forceinline__ void wait_lgkm0() { __builtin_amdgcn_s_waitcnt((15) | (7 << 4) | (0 << 8) | (3 << 14)); }

// One compute step of the software pipeline: barrier g (stage g + 1 has
// landed), LDS reads of stage g + 1 into `nxt` (unless g is the last step),
// then the MFMAs of stage g from `cur` (read during the previous step) over
// the wave's first nf row fragments - the rest, padding of a partly filled
// row tile, is skipped behind wave-uniform branches with the accumulators
// updated in place. The reads are issued ahead of the MFMAs so their latency
// hides behind the matrix work; the caller completes them before the next
// barrier, after which the producers may refill their slot. The MFMA is fed
// (B, A) so that it produces C^T fragments: lane l then holds output row
// (l % 16) and the four consecutive output columns 4 * (l / 16) .. +3 of a
// 16 x 16 fragment, which the epilogues write as one 8- or 16-byte store
// instead of four scattered 2-byte ones (see dma_out_row / dma_out_col).
template <class Cfg>
__device__ __forceinline__ void mma_pp_step(int g, int total, int nf, RingCursor<Cfg>& rc,
                                            const Frags<Cfg>& cur, Frags<Cfg>& nxt, Acc<Cfg>& acc,
                                            int wm, int wn, int lane) {
  ring_barrier();
  if (g + 1 < total) {
    read_frags_ab<Cfg>(nxt, rc.a(), rc.b(), wm, wn, lane);
    rc.advance();
  }
#pragma unroll
  for (int i = 0; i < Cfg::FM; ++i) {
    if (i < nf) {
#pragma unroll
      for (int j = 0; j < Cfg::FN; ++j)
        acc.v[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(cur.b[j], cur.a[i], acc.v[i][j], 0, 0, 0);
    }
  }
}

// Row fragments of wave row wm that hold some of the tile's first `valid`
// rows: fragments i with frag_row0(wm, i) < valid.
template <class Cfg>
__device__ __forceinline__ int dma_active_frags(int wm, int valid) {
  const int used = (valid + 15) >> 4;  // 16-row blocks holding valid rows
  const int n = (used - wm + Cfg::WM - 1) / Cfg::WM;
  return n <= 0 ? 0 : min(Cfg::FM, n);
}

// Output coordinates (within the tile) of acc.v[i][j][r] for the DMA driver:
// row dma_out_row(i), column dma_out_col(j) + r, r = 0..3. Compute wave w is
// at (wm, wn) = (w / WN, w % WN) of the wave grid.
template <class Cfg>
__device__ __forceinline__ int dma_out_row(int wm, int i, int lane) {
  return frag_row0<Cfg>(wm, i) + (lane & 15);
}
template <class Cfg>
__device__ __forceinline__ int dma_out_col(int wn, int j, int lane) {
  return wn * (Cfg::BN / Cfg::WN) + j * 16 + (lane >> 4) * 4;
}

// Two output fragments side by side (columns c .. c+15 in `lo`, c+16 .. c+31
// in `hi`, each lane holding its four columns 4 (l / 16) .. +3 of both) as
// bf16, moved across the lanes of the same output row so that lane l holds
// the eight consecutive columns c + pair_col(l) .. +7: one 16-byte store per
// lane instead of two 8-byte ones, and every output row written in 64-byte
// runs per store (two 32-byte runs before). The row fragment's 16 rows keep
// their lanes (l % 16): v_permlane32_swap exchanges the upper half-wave of
// its first operand with the lower half-wave of its second, and
// v_permlane16_swap the odd 16-lane groups of its first operand with the
// even groups of its second. All 64 lanes must execute it (a lane that
// stores nothing still passes its values through).
__device__ __forceinline__ uint4 pair_cols_bf16(const float (&lo)[4], const float (&hi)[4]) {
  const uint2 x = pack4_bf16(lo[0], lo[1], lo[2], lo[3]);
  const uint2 y = pack4_bf16(hi[0], hi[1], hi[2], hi[3]);
  // lane groups (16 lanes) of x: columns 0-3 | 4-7 | 8-11 | 12-15, of y: 16-19 | ... | 28-31
  const auto a0 = __builtin_amdgcn_permlane32_swap(x.x, y.x, false, false);
  const auto a1 = __builtin_amdgcn_permlane32_swap(x.y, y.y, false, false);
  // a[0]: 0-3 | 4-7 | 16-19 | 20-23, a[1]: 8-11 | 12-15 | 24-27 | 28-31
  const auto b0 = __builtin_amdgcn_permlane16_swap(a0[0], a0[1], false, false);
  const auto b1 = __builtin_amdgcn_permlane16_swap(a1[0], a1[1], false, false);
  // b[0]: 0-3 | 8-11 | 16-19 | 24-27, b[1]: 4-7 | 12-15 | 20-23 | 28-31
  return make_uint4(b0[0], b1[0], b0[1], b1[1]);
}
__device__ __forceinline__ int pair_col(int lane) { return (lane >> 4) * 8; }
// The same move for fp32 values: out[k] = column c + pair_col(l) + k. (The
// conversions go through values: __builtin_bit_cast of a vector element such
// as lo[q] or b[1] reads element 0 with this compiler.)
__device__ __forceinline__ void pair_cols_f32(const f32x4& lo, const f32x4& hi, float (&out)[8]) {
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(lo[q]), __float_as_uint(hi[q]), false, false);
    const auto b = __builtin_amdgcn_permlane16_swap(a[0], a[1], false, false);
    out[q] = __uint_as_float(b[0]);
    out[4 + q] = __uint_as_float(b[1]);
  }
}

// s_waitcnt with vmcnt = n (n < 64) and the other counters left alone: vmcnt
// lives in bits [3:0] and [15:14], expcnt [6:4], lgkmcnt [11:8].
template <int N>
__device__ __forceinline__ void wait_vmcnt_imm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}
// Producer wait before stage g is read, with `younger` stages (0 .. STAGES-2)
// issued after it: at most younger * DMA_PER_PRODUCER DMAs may still be out.
// The steady state (younger = STAGES - 2) is one immediate wait; the ring's
// last steps select theirs from a short scalar chain.
template <class Cfg, int Y = Cfg::STAGES - 2>
__device__ __forceinline__ void dma_wait_stage(int younger) {
  if constexpr (Y == 0) {
    wait_vmcnt_imm<0>();
  } else {
    if (younger >= Y)
      wait_vmcnt_imm<Y * Cfg::DMA_PER_PRODUCER>();
    else
      dma_wait_stage<Cfg, Y - 1>(younger);
  }
}

// Producer wait with a run-time count: vmcnt <= the largest immediate <= n.
template <int N>
__device__ __forceinline__ void wait_vmcnt_le(int n) {
  if constexpr (N == 0) {
    wait_vmcnt_imm<0>();
  } else {
    if (n >= N)
      wait_vmcnt_imm<N>();
    else
      wait_vmcnt_le<N - 1>(n);
  }
}

// Split ring (Cfg::SPLIT): a producer issues its DMAs in steps, step j being
// A of stage j then B of stage j + B_LEAD (steps past the last stage issue
// nothing for that operand), after B_LEAD B-only steps at the start. When it
// waits for stage j, steps up to j + STAGES - 2 have been issued, and since
// loads complete in issue order, stage j (both parts) has landed once at most
// these are still out: B of step j and both parts of steps j + 1 ..
// j + STAGES - 2, as far as they exist (rem = stages left from j on).
template <class Cfg>
__device__ __forceinline__ int split_younger(int rem) {
  int c = Cfg::B_LEAD < rem ? Cfg::B_PER : 0;
#pragma unroll
  for (int m = 1; m <= Cfg::STAGES - 2; ++m) c += (m < rem ? Cfg::A_PER : 0) + (m + Cfg::B_LEAD < rem ? Cfg::B_PER : 0);
  return c;
}
template <class Cfg>
__device__ __forceinline__ void split_wait_stage(int rem) {
  constexpr int steady = Cfg::B_PER + (Cfg::STAGES - 2) * (Cfg::A_PER + Cfg::B_PER);
  if (rem > Cfg::STAGES - 2 + Cfg::B_LEAD)
    wait_vmcnt_imm<steady>();
  else
    wait_vmcnt_le<steady>(split_younger<Cfg>(rem));
}

// Extra K steps a problem appends to each item (Prob::kExtra, default 0):
// stages whose operands come from a second loader filled by
// Prob::setup_extra(item, ld, part), e.g. a rank-r adapter term carried
// through the matrix cores after the item's nk main steps.
template <class P, class = void>
struct ExtraSteps {
  static constexpr int value = 0;
};
template <class P>
struct ExtraSteps<P, std::void_t<decltype(P::kExtra)>> {
  static constexpr int value = P::kExtra;
};


// Persistent warp-specialised driver on the DMA ring. Items are processed in
// order; Prob::rows(item) gives an item's valid tile rows (row fragments past
// them skip their MFMAs), Prob::setup(item, ld, part) fills producer part's
// DmaLoader, Prob::epilogue(item, acc) writes an item's result (compute
// waves). K steps are numbered g = 0 .. total-1 over the workgroup's items
// (nk = nk_main + extra steps per item). Barrier "-1" publishes stage 0; barrier g then
// publishes stage g + 1 and tells the producers that slot g % STAGES (stage
// g, read by the compute waves during step g - 1) is free:
//   producers: wait until their DMAs of stage g + 1 landed; barrier g; issue
//              stage g + STAGES into slot g % STAGES.
//   compute:   barrier g; read stage g + 1 into one register set while the
//              MFMAs of stage g run from the other; epilogue if g closes an
//              item; finish the reads before the next barrier.
// The register sets alternate per step; an item with an odd step count
// hands the next item's first stage over from the second set to the first.
// Barriers are bare s_barrier: the producers' explicit vmcnt waits already
// order their DMA writes, and a fenced barrier would wait for every stage in
// flight.
// Split ring (Cfg::SB > 0): A stays in STAGES slots, B gets SB slots of its
// own, so barrier g frees A slot g % STAGES and B slot g % SB, and the
// producers refill them with A of stage g + STAGES and B of stage g + SB.
// B then has SB - 1 stages in flight where A has STAGES - 1: for streamed
// weights, whose lines come from HBM once, against token rows that the
// column blocks of an expert share through the L2.
template <class Cfg, class Prob>
__device__ __forceinline__ void persistent_gemm_dma(Prob& pb, int items, int nk_main) {
  static_assert(Cfg::KSUB == 1, "one MFMA K step per stage");
  constexpr int S = Cfg::STAGES;
  constexpr int NX = ExtraSteps<Prob>::value;
  __shared__ __align__(16) bf16_t ring[Cfg::RING_ELEMS];
  const XcdSplit sp = xcd_split(items);
  if (sp.first >= sp.end || nk_main <= 0) return;
  const int nk = nk_main + NX;  // K steps per item
  const int n_mine = (sp.end - sp.first + sp.stride - 1) / sp.stride;
  const int total = n_mine * nk;
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));

  if constexpr (Cfg::SPLIT) {
    if (wave >= Cfg::CW) {
      const int part = wave - Cfg::CW;
      // separate cursors (item, K step, slot) for the A and the B stream
      struct Cursor {
        int ord = 0, kt = 0, slot = 0, n = 0;  // n: stages issued
        DmaLoader<Cfg> ld, ldx;
      };
      Cursor ca, cb;
      pb.setup(sp.first, ca.ld, part);
      pb.setup(sp.first, cb.ld, part);
      if constexpr (NX > 0) {
        pb.setup_extra(sp.first, ca.ldx, part);
        pb.setup_extra(sp.first, cb.ldx, part);
      }
      auto advance = [&](Cursor& c, int slots) {
        c.slot = (c.slot + 1 == slots) ? 0 : c.slot + 1;
        ++c.n;
        if (++c.kt == nk) {
          c.kt = 0;
          if (++c.ord < n_mine) {
            const int item = sp.first + c.ord * sp.stride;
            pb.setup(item, c.ld, part);
            if constexpr (NX > 0) pb.setup_extra(item, c.ldx, part);
          }
        }
      };
      auto issue_a = [&]() {
        if (ca.n >= total) return;
        bf16_t* dst = ring + ca.slot * Cfg::A_ELEMS;
        if (NX > 0 && ca.kt >= nk_main)
          dma_issue_a<Cfg>(ca.ldx, ca.kt - nk_main, dst, part);
        else
          dma_issue_a<Cfg>(ca.ld, ca.kt, dst, part);
        advance(ca, S);
      };
      auto issue_b = [&]() {
        if (cb.n >= total) return;
        bf16_t* dst = ring + S * Cfg::A_ELEMS + cb.slot * Cfg::B_ELEMS;
        if (NX > 0 && cb.kt >= nk_main)
          dma_issue_b<Cfg>(cb.ldx, cb.kt - nk_main, dst, part);
        else
          dma_issue_b<Cfg>(cb.ld, cb.kt, dst, part);
        advance(cb, Cfg::SB);
      };
      for (int p = 0; p < Cfg::B_LEAD; ++p) issue_b();
      for (int p = 0; p < S - 1; ++p) {
        issue_a();
        issue_b();
      }
      // barrier "-1": stage 0 landed
      split_wait_stage<Cfg>(total);
      ring_barrier();
      issue_a();
      issue_b();
      for (int g = 0; g < total; ++g) {
        if (g + 1 < total) split_wait_stage<Cfg>(total - 1 - g);
        ring_barrier();
        issue_a();  // stage g + S into A slot g % S
        issue_b();  // stage g + SB into B slot g % SB
      }
      return;
    }
  } else if (wave >= Cfg::CW) {
    const int part = wave - Cfg::CW;
    DmaLoader<Cfg> ld, ldx;
    int l_ord = 0, l_kt = 0, l_slot = 0;  // load cursor
    pb.setup(sp.first, ld, part);
    if constexpr (NX > 0) pb.setup_extra(sp.first, ldx, part);
    auto issue_next = [&]() {
      if (NX > 0 && l_kt >= nk_main)
        dma_issue<Cfg>(ldx, l_kt - nk_main, ring + l_slot * Cfg::STAGE_ELEMS, part);
      else
        dma_issue<Cfg>(ld, l_kt, ring + l_slot * Cfg::STAGE_ELEMS, part);
      l_slot = (l_slot + 1 == S) ? 0 : l_slot + 1;
      if (++l_kt == nk) {
        l_kt = 0;
        if (++l_ord < n_mine) {
          const int item = sp.first + l_ord * sp.stride;
          pb.setup(item, ld, part);
          if constexpr (NX > 0) pb.setup_extra(item, ldx, part);
        }
      }
    };
    for (int p = 0; p < S - 1 && p < total; ++p) issue_next();
    // barrier "-1": stage 0 landed
    dma_wait_stage<Cfg>(total - 1);
    ring_barrier();
    if (S - 1 < total) issue_next();
    for (int g = 0; g < total; ++g) {
      // barrier g: stage g + 1 landed (the compute waves read it during step g)
      if (g + 1 < total) dma_wait_stage<Cfg>(total - 2 - g);
      ring_barrier();
      if (g + S < total) issue_next();
    }
    return;
  }

  const int lane = threadIdx.x & 63;
  const int wm = wave / Cfg::WN, wn = wave % Cfg::WN;
  Acc<Cfg> acc;
  Frags<Cfg> f0, f1;
  ring_barrier();  // barrier "-1"
  RingCursor<Cfg> rc{ring};  // next stage to read: 1
  read_frags_ab<Cfg>(f0, ring, ring + (Cfg::SPLIT ? S * Cfg::A_ELEMS : Cfg::A_ELEMS), wm, wn, lane);
  wait_lgkm0();
  // K steps ping-pong between the two register sets; every item starts with
  // its first stage in f0 (with an odd step count the last step reads the
  // next item's first stage into f1, which is moved to f0 after the epilogue)
  for (int c_ord = 0; c_ord < n_mine; ++c_ord) {
    const int item = sp.first + c_ord * sp.stride;
    const int nf = dma_active_frags<Cfg>(wm, pb.rows(item));
    const int g0 = c_ord * nk;
    acc.zero();
    int kt = 0;
    for (; kt + 1 < nk; kt += 2) {
      mma_pp_step<Cfg>(g0 + kt, total, nf, rc, f0, f1, acc, wm, wn, lane);
      wait_lgkm0();
      mma_pp_step<Cfg>(g0 + kt + 1, total, nf, rc, f1, f0, acc, wm, wn, lane);
      wait_lgkm0();
    }
    const bool odd = kt < nk;  // wave-uniform
    if (odd) mma_pp_step<Cfg>(g0 + kt, total, nf, rc, f0, f1, acc, wm, wn, lane);
    pb.epilogue(item, acc);
    wait_lgkm0();
    if (odd) f0 = f1;
  }
}

// Persistent symmetric driver (DmaCfg with PW = 0): every wave issues its
// share of each stage's DMAs and computes. Meant for a dense GEMM whose
// workgroups process few items (the router), where the cost the wave roles
// of persistent_gemm_dma avoid - a wave waiting for loads issued after its
// own epilogue stores - occurs once per item: the first wait after an
// epilogue drains the wave's counter.
//
// Half-step software pipeline: a wave's A fragments split into a low half
// (rows i < FM/2) and a high half. Step g runs in two phases:
//   1. LDS reads of stage g's high half; MFMAs of the low half (stage g's B
//      and low A, read during phase 2 of step g - 1).
//   2. wait for the wave's reads and for its own DMAs of stage g + 1;
//      barrier (stage g + 1 landed everywhere; stage g fully read, so its
//      slot g % STAGES is free); issue stage g + STAGES into that slot; LDS
//      reads of stage g + 1's B and low half; MFMAs of the high half.
// So every group of LDS reads is in flight behind FM/2 x FN MFMAs of the same
// wave, and the two waves of a SIMD need not interleave to hide it. B and the
// low half alternate between two register sets (two steps per loop turn, so
// nk must be even); all rows are computed (rows past the valid ones on
// clamped data) and the epilogue stores the valid ones.
template <class Cfg>
struct SymFrags {
  bf16x8 b[Cfg::FN];
  bf16x8 a[Cfg::FM / 2];
};

template <class Cfg>
__device__ __forceinline__ void sym_read_lo(SymFrags<Cfg>& f, const bf16_t* st, int wm, int wn, int lane) {
  const bf16_t* As = st;
  const bf16_t* Bs = st + Cfg::A_ELEMS;
  const int r = lane & 15;
  const int slot = (lane >> 4) ^ lds_key<Cfg>(r);
#pragma unroll
  for (int j = 0; j < Cfg::FN; ++j)
    f.b[j] = *reinterpret_cast<const bf16x8*>(&Bs[(wn * (Cfg::BN / Cfg::WN) + j * 16 + r) * Cfg::BK + slot * 8]);
#pragma unroll
  for (int i = 0; i < Cfg::FM / 2; ++i)
    f.a[i] = *reinterpret_cast<const bf16x8*>(&As[(frag_row0<Cfg>(wm, i) + r) * Cfg::BK + slot * 8]);
}

template <class Cfg>
__device__ __forceinline__ void sym_read_hi(bf16x8 (&ahi)[Cfg::FM / 2], const bf16_t* st, int wm, int lane) {
  const int r = lane & 15;
  const int slot = (lane >> 4) ^ lds_key<Cfg>(r);
#pragma unroll
  for (int i = 0; i < Cfg::FM / 2; ++i)
    ahi[i] = *reinterpret_cast<const bf16x8*>(&st[(frag_row0<Cfg>(wm, i + Cfg::FM / 2) + r) * Cfg::BK + slot * 8]);
}

template <class Cfg>
__device__ __forceinline__ void sym_mma(Acc<Cfg>& acc, const bf16x8 (&b)[Cfg::FN], const bf16x8 (&a)[Cfg::FM / 2],
                                        int i0) {
#pragma unroll
  for (int i = 0; i < Cfg::FM / 2; ++i)
#pragma unroll
    for (int j = 0; j < Cfg::FN; ++j)
      acc.v[i0 + i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(b[j], a[i], acc.v[i0 + i][j], 0, 0, 0);
}

// Symmetric driver for 64-K stages (KSUB = 2): the two phases of a step are
// the stage's two MFMA K steps instead of two halves of the A fragments.
//   1. LDS reads of stage g's second K half (all fragments) into one set;
//      MFMAs of its first half from the other set (read in phase 2 of step
//      g - 1).
//   2. wait for the reads and the wave's own DMAs of stage g + 1; barrier;
//      issue stage g + STAGES into slot g % STAGES; reads of stage g + 1's
//      first half; MFMAs of stage g's second half.
template <class Cfg, class Prob>
__device__ __forceinline__ void persistent_gemm_sym_k64(Prob& pb, int items, int nk) {
  static_assert(Cfg::PW == 0 && Cfg::KSUB == 2, "symmetric configuration, 64-K stages");
  constexpr int S = Cfg::STAGES;
  static_assert(!Cfg::SPLIT, "joint ring");
  __shared__ __align__(16) bf16_t ring[S * Cfg::STAGE_ELEMS];
  const XcdSplit sp = xcd_split(items);
  if (sp.first >= sp.end || nk <= 0) return;
  const int n_mine = (sp.end - sp.first + sp.stride - 1) / sp.stride;
  const int total = n_mine * nk;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int wm = wave / Cfg::WN, wn = wave % Cfg::WN;
  DmaLoader<Cfg> ld;
  int l_ord = 0, l_kt = 0, l_slot = 0;  // load cursor
  pb.setup(sp.first, ld, wave);
  auto issue_next = [&]() {
    dma_issue<Cfg>(ld, l_kt, ring + l_slot * Cfg::STAGE_ELEMS, wave);
    l_slot = (l_slot + 1 == S) ? 0 : l_slot + 1;
    if (++l_kt == nk) {
      l_kt = 0;
      if (++l_ord < n_mine) pb.setup(sp.first + l_ord * sp.stride, ld, wave);
    }
  };
  for (int p = 0; p < S - 1 && p < total; ++p) issue_next();
  dma_wait_stage<Cfg>(total - 1);
  ring_barrier();
  if (S - 1 < total) issue_next();
  Acc<Cfg> acc;
  Frags<Cfg> f0, f1;  // first / second K half of a stage
  read_frags<Cfg>(f0, ring, wm, wn, lane, 0);
  int c_slot = 0;
  bool drain = false;  // epilogue stores are still counted on vmcnt
  auto mma = [&](const Frags<Cfg>& f) {
#pragma unroll
    for (int i = 0; i < Cfg::FM; ++i)
#pragma unroll
      for (int j = 0; j < Cfg::FN; ++j)
        acc.v[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(f.b[j], f.a[i], acc.v[i][j], 0, 0, 0);
  };
  for (int c_ord = 0; c_ord < n_mine; ++c_ord) {
    const int g0 = c_ord * nk;
    acc.zero();
    for (int kt = 0; kt < nk; ++kt) {
      const int g = g0 + kt;
      read_frags<Cfg>(f1, ring + c_slot * Cfg::STAGE_ELEMS, wm, wn, lane, 1);
      __builtin_amdgcn_sched_barrier(0);
      mma(f0);
      __builtin_amdgcn_sched_barrier(0);
      wait_lgkm0();
      if (g + 1 < total) {
        if (drain) {
          wait_vmcnt_imm<0>();
          drain = false;
        } else {
          dma_wait_stage<Cfg>(total - 2 - g);
        }
      }
      ring_barrier();
      if (g + S < total) issue_next();
      c_slot = (c_slot + 1 == S) ? 0 : c_slot + 1;
      if (g + 1 < total) read_frags<Cfg>(f0, ring + c_slot * Cfg::STAGE_ELEMS, wm, wn, lane, 0);
      __builtin_amdgcn_sched_barrier(0);
      mma(f1);
      __builtin_amdgcn_sched_barrier(0);
    }
    pb.epilogue(sp.first + c_ord * sp.stride, acc);
    drain = true;
  }
}

template <class Cfg, class Prob>
__device__ __forceinline__ void persistent_gemm_sym(Prob& pb, int items, int nk) {
  static_assert(Cfg::PW == 0, "symmetric configuration");
  if constexpr (Cfg::KSUB == 2) {
    persistent_gemm_sym_k64<Cfg>(pb, items, nk);
    return;
  } else {
  static_assert(Cfg::FM % 2 == 0, "two halves of A fragments");
  constexpr int S = Cfg::STAGES;
  constexpr int H = Cfg::FM / 2;
  static_assert(!Cfg::SPLIT, "joint ring");
  __shared__ __align__(16) bf16_t ring[S * Cfg::STAGE_ELEMS];
  const XcdSplit sp = xcd_split(items);
  if (sp.first >= sp.end || nk <= 0) return;
  const int n_mine = (sp.end - sp.first + sp.stride - 1) / sp.stride;
  const int total = n_mine * nk;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int wm = wave / Cfg::WN, wn = wave % Cfg::WN;
  DmaLoader<Cfg> ld;
  int l_ord = 0, l_kt = 0, l_slot = 0;  // load cursor
  pb.setup(sp.first, ld, wave);
  auto issue_next = [&]() {
    dma_issue<Cfg>(ld, l_kt, ring + l_slot * Cfg::STAGE_ELEMS, wave);
    l_slot = (l_slot + 1 == S) ? 0 : l_slot + 1;
    if (++l_kt == nk) {
      l_kt = 0;
      if (++l_ord < n_mine) pb.setup(sp.first + l_ord * sp.stride, ld, wave);
    }
  };
  // stages 0 .. S-1: S-1 before barrier "-1", stage S-1 into the never-used
  // last slot right after it
  for (int p = 0; p < S - 1 && p < total; ++p) issue_next();
  dma_wait_stage<Cfg>(total - 1);
  ring_barrier();
  if (S - 1 < total) issue_next();
  Acc<Cfg> acc;
  SymFrags<Cfg> f0, f1;
  bf16x8 ahi[H];
  sym_read_lo<Cfg>(f0, ring, wm, wn, lane);
  int c_slot = 0;      // ring slot of stage g
  bool drain = false;  // epilogue stores are still counted on vmcnt
  // phase 2 of step g: publish stage g + 1, refill slot g % S, read stage
  // g + 1's low set into `nxt`, MFMAs of the high half from `cur`.b
  auto phase2 = [&](int g, const SymFrags<Cfg>& cur, SymFrags<Cfg>& nxt) {
    wait_lgkm0();
    if (g + 1 < total) {
      if (drain) {
        wait_vmcnt_imm<0>();
        drain = false;
      } else {
        dma_wait_stage<Cfg>(total - 2 - g);
      }
    }
    ring_barrier();
    if (g + S < total) issue_next();
    const int n_slot = (c_slot + 1 == S) ? 0 : c_slot + 1;
    if (g + 1 < total) sym_read_lo<Cfg>(nxt, ring + n_slot * Cfg::STAGE_ELEMS, wm, wn, lane);
    __builtin_amdgcn_sched_barrier(0);
    sym_mma<Cfg>(acc, cur.b, ahi, H);
    __builtin_amdgcn_sched_barrier(0);
    c_slot = n_slot;
  };
  // phase 1 of step g: read stage g's high half, MFMAs of the low half
  auto phase1 = [&](const SymFrags<Cfg>& cur) {
    sym_read_hi<Cfg>(ahi, ring + c_slot * Cfg::STAGE_ELEMS, wm, lane);
    __builtin_amdgcn_sched_barrier(0);
    sym_mma<Cfg>(acc, cur.b, cur.a, 0);
    __builtin_amdgcn_sched_barrier(0);
  };
  for (int c_ord = 0; c_ord < n_mine; ++c_ord) {
    const int g0 = c_ord * nk;
    acc.zero();
    for (int kt = 0; kt < nk; kt += 2) {
      phase1(f0);
      phase2(g0 + kt, f0, f1);
      phase1(f1);
      phase2(g0 + kt + 1, f1, f0);
    }
    pb.epilogue(sp.first + c_ord * sp.stride, acc);
    drain = true;
  }
  }
}

}  // namespace moe
