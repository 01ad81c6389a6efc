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
// Wave roles. A workgroup has 4 compute waves and 2 producer waves. The
// producers issue every DMA of the ring and never store; the compute waves
// read LDS, run the MFMAs and write the results. On this GPU stores share
// the vector-memory counter with loads and the counter retires in issue
// order, so in a wave that both loads and stores, every load issued after an
// epilogue's stores could only be waited for once those stores were
// acknowledged - a bubble of a full write latency after every output tile.
// With the roles split, a producer's waits count its own DMAs only (a
// constant in the steady state) and the compute waves never wait on memory
// counters. Two producers share each stage's DMAs: one wave alone issues
// them too slowly to keep the memory system busy.
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

constexpr int kComputeWaves = 4;  // waves 0..3
constexpr int kProducers = 2;     // waves 4..5; producer p issues the DMAs i with i % kProducers == p
constexpr int kDmaThreads = 64 * (kComputeWaves + kProducers);  // workgroup size of the DMA GEMMs

template <int BM_, int BN_, int STAGES_ = 4, int WM_ = 2>
struct DmaCfg {
  static constexpr int BM = BM_;
  static constexpr int BN = BN_;
  static constexpr int BK = 32;
  static constexpr int STAGES = STAGES_;  // ring slots; STAGES - 1 stages in flight
  static constexpr int WM = WM_;          // the compute waves form a WM x WN grid over the tile
  static constexpr int WN = kComputeWaves / WM_;
  static constexpr int FM = BM / (16 * WM);  // 16 x 16 fragments per wave along M
  static constexpr int FN = BN / (16 * WN);
  static constexpr int A_DMA = BM / 16;  // producer DMA instructions per stage (16 rows each)
  static constexpr int B_DMA = BN / 16;
  static constexpr int DMA_PER_STAGE = A_DMA + B_DMA;
  static constexpr int A_ELEMS = BM * BK;
  static constexpr int B_ELEMS = BN * BK;
  static constexpr int STAGE_ELEMS = A_ELEMS + B_ELEMS;
  static_assert(WM == 1 || WM == 2 || WM == 4, "wave grid");
  static_assert(FM >= 1 && FN >= 1 && FM * 16 * WM == BM && FN * 16 * WN == BN, "fragments");
  static_assert(BM % 16 == 0 && BN % 16 == 0, "DMA tiles are multiples of 16 rows");
  static constexpr int DMA_PER_PRODUCER = DMA_PER_STAGE / kProducers;  // per stage
  static_assert(A_DMA % kProducers == 0 && B_DMA % kProducers == 0, "DMA split");
  static_assert(STAGES >= 3 && (STAGES - 2) * DMA_PER_PRODUCER <= 63, "ring depth vs vmcnt");
};

// Lane pointers of one producer for one item: a[q] / b[q] belong to the
// producer's q-th DMA instruction of each operand, i = q * kProducers + part,
// and point at the logical chunk this lane fetches ((lane & 3) ^
// chunk_key(lane / 4)) of tile row 16 i + lane / 4; set by
// Prob::setup(item, ld, part).
// a_kstep / b_kstep: elements between consecutive K steps of one operand
// (32 for a row-major operand; one whole packed tile for a packed one).
template <class Cfg>
struct DmaLoader {
  const bf16_t* a[Cfg::A_DMA / kProducers];
  const bf16_t* b[Cfg::B_DMA / kProducers];
  int a_kstep = Cfg::BK;
  int b_kstep = Cfg::BK;
};

// Swizzle key of tile row r (only r mod 16 matters): bit 0 = bit 2 of r,
// bit 1 = bit 1 ^ bit 3 of r. XOR with it maps chunk -> slot and back.
__host__ __device__ __forceinline__ int chunk_key(int r) {
  return ((r >> 2) & 1) | ((((r >> 1) ^ (r >> 3)) & 1) << 1);
}

// Tile row whose chunk this (producer) lane fetches in DMA instruction i, and
// the element offset of that chunk inside the row: lane l writes slot l % 4
// of row l / 4 of the instruction's 16-row group, so it fetches chunk
// (l % 4) ^ key.
__device__ __forceinline__ int dma_row(int i) { return 16 * i + ((threadIdx.x & 63) >> 2); }
__device__ __forceinline__ int dma_chunk_elem() {
  const int lane = threadIdx.x & 63;
  return ((lane & 3) ^ chunk_key(lane >> 2)) * 8;
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

// Producer `part`'s share of the DMA instructions of K step kt into stage
// `stage`: A and B instructions i with i % kProducers == part.
template <class Cfg>
__device__ __forceinline__ void dma_issue(const DmaLoader<Cfg>& ld, int kt, bf16_t* stage, int part) {
  const int64_t ka = (int64_t)kt * ld.a_kstep, kb = (int64_t)kt * ld.b_kstep;
#pragma unroll
  for (int q = 0; q < Cfg::A_DMA / kProducers; ++q)
    dma16(ld.a[q] + ka, stage + 16 * (q * kProducers + part) * Cfg::BK);
#pragma unroll
  for (int q = 0; q < Cfg::B_DMA / kProducers; ++q)
    dma16(ld.b[q] + kb, stage + Cfg::A_ELEMS + 16 * (q * kProducers + part) * Cfg::BK);
}

// Packed B operand: the weight tile of one (n block, K step) stored as the
// exact image of its LDS stage (BN rows x 32, chunks swizzled as above), so
// a DMA instruction copies 1 KB of contiguous memory. Pointer for this lane's
// chunk of DMA instruction i, K step 0, given the tile's base.
template <class Cfg>
__device__ __forceinline__ const bf16_t* packed_b_ptr(const bf16_t* tile0, int i) {
  return tile0 + (int64_t)i * 16 * Cfg::BK + (threadIdx.x & 63) * 8;
}
constexpr int kPackTileElems = 128 * 32;  // one packed weight tile: 128 rows x 32 (8 KB)

// One K step of 32 from a swizzled stage (compute wave) over the wave's first
// NF row fragments. Straight-line code: the fragment reads are issued up
// front (B, then A by row fragment) and each MFMA group waits only for its
// own operands, so LDS latency overlaps the matrix work. The MFMA is fed
// (B, A) so that it produces C^T fragments: lane l then holds output row
// (l % 16) and the four consecutive output columns 4 * (l / 16) .. +3 of a
// 16 x 16 fragment, which the epilogues write as one 8- or 16-byte store
// instead of four scattered 2-byte ones (see dma_out_row / dma_out_col).
template <class Cfg, int NF>
__device__ __forceinline__ void mma_step_n(const bf16_t* st, Acc<Cfg>& acc, int wm, int wn, int lane) {
  const bf16_t* As = st;
  const bf16_t* Bs = st + Cfg::A_ELEMS;
  const int r = lane & 15;
  const int slot = (lane >> 4) ^ chunk_key(r);
  bf16x8 a[NF], b[Cfg::FN];
#pragma unroll
  for (int j = 0; j < Cfg::FN; ++j)
    b[j] = *reinterpret_cast<const bf16x8*>(&Bs[(wn * (Cfg::BN / Cfg::WN) + j * 16 + r) * Cfg::BK + slot * 8]);
#pragma unroll
  for (int i = 0; i < NF; ++i)
    a[i] = *reinterpret_cast<const bf16x8*>(&As[(wm * (Cfg::BM / Cfg::WM) + i * 16 + r) * Cfg::BK + slot * 8]);
#pragma unroll
  for (int i = 0; i < NF; ++i)
#pragma unroll
    for (int j = 0; j < Cfg::FN; ++j)
      acc.v[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(b[j], a[i], acc.v[i][j], 0, 0, 0);
  // keep every LDS read ahead of the MFMAs (the scheduler would otherwise
  // recycle operand registers in pairs and wait a full LDS round trip per pair)
  __builtin_amdgcn_sched_group_barrier(0x100, NF + Cfg::FN, 0);  // DS reads
  __builtin_amdgcn_sched_group_barrier(0x008, NF * Cfg::FN, 0);  // MFMAs
}

// The K loop of one item on the compute side, over the wave's first NF row
// fragments: one barrier per K step (matching the producer's), then the
// MFMAs of the stage in the ring slot `slot`.
template <class Cfg, int NF>
__device__ __forceinline__ void mma_item_n(int nk, const bf16_t* ring, int& slot, Acc<Cfg>& acc,
                                           int wm, int wn, int lane) {
  for (int kt = 0; kt < nk; ++kt) {
    __builtin_amdgcn_s_barrier();
    if constexpr (NF > 0) mma_step_n<Cfg, NF>(ring + slot * Cfg::STAGE_ELEMS, acc, wm, wn, lane);
    slot = (slot + 1 == Cfg::STAGES) ? 0 : slot + 1;
  }
}

// One item's K loop for a wave whose first nf row fragments hold valid rows.
// The rest (padding of a partly filled row tile) is skipped in coarse steps -
// the wave's whole tile, or its first 3/4, 1/2 or 1/4 - each its own loop,
// so the choice is made once per item and every K step stays straight-line.
template <class Cfg>
__device__ __forceinline__ void mma_item(int nf, int nk, const bf16_t* ring, int& slot,
                                         Acc<Cfg>& acc, int wm, int wn, int lane) {
  constexpr int F = Cfg::FM;
  if constexpr (F % 4 == 0) {
    if (nf > 3 * F / 4)
      mma_item_n<Cfg, F>(nk, ring, slot, acc, wm, wn, lane);
    else if (nf > F / 2)
      mma_item_n<Cfg, 3 * F / 4>(nk, ring, slot, acc, wm, wn, lane);
    else if (nf > F / 4)
      mma_item_n<Cfg, F / 2>(nk, ring, slot, acc, wm, wn, lane);
    else if (nf > 0)
      mma_item_n<Cfg, F / 4>(nk, ring, slot, acc, wm, wn, lane);
    else
      mma_item_n<Cfg, 0>(nk, ring, slot, acc, wm, wn, lane);
  } else {
    if (nf > 0)
      mma_item_n<Cfg, F>(nk, ring, slot, acc, wm, wn, lane);
    else
      mma_item_n<Cfg, 0>(nk, ring, slot, acc, wm, wn, lane);
  }
}

// Row fragments of wave row wm that hold some of the tile's first `valid` rows.
template <class Cfg>
__device__ __forceinline__ int dma_active_frags(int wm, int valid) {
  const int rows = valid - wm * (Cfg::BM / Cfg::WM);
  return rows <= 0 ? 0 : min(Cfg::FM, (rows + 15) >> 4);
}

// Output coordinates (within the tile) of acc.v[i][j][r] for the DMA driver:
// row dma_out_row(i), column dma_out_col(j) + r, r = 0..3. Compute wave w is
// at (wm, wn) = (w / WN, w % WN) of the wave grid.
template <class Cfg>
__device__ __forceinline__ int dma_out_row(int wm, int i, int lane) {
  return wm * (Cfg::BM / Cfg::WM) + i * 16 + (lane & 15);
}
template <class Cfg>
__device__ __forceinline__ int dma_out_col(int wn, int j, int lane) {
  return wn * (Cfg::BN / Cfg::WN) + j * 16 + (lane >> 4) * 4;
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

// Persistent warp-specialised driver on the DMA ring. Items are processed in
// order; Prob::rows(item) gives an item's valid tile rows (row fragments past
// them skip their MFMAs), Prob::setup(item, ld, part) fills producer part's
// DmaLoader, Prob::epilogue(item, acc) writes an item's result (compute
// waves). Step g (one K step of some item):
//   producers: wait until their DMAs of stage g landed; barrier; issue stage
//             g + STAGES - 1 into slot (g - 1) % STAGES.
//   compute:  barrier; MFMAs of stage g; epilogue if g closes an item
//             (the K loop of each item is specialised on how many of the
//             wave's row fragments hold valid rows).
// The barrier of step g publishes stage g to the compute waves and tells the
// producer that slot (g - 1) % STAGES has been read. It is a bare s_barrier:
// the producer's explicit vmcnt wait already orders its DMA writes, and a
// fenced barrier would wait for every stage in flight.
template <class Cfg, class Prob>
__device__ __forceinline__ void persistent_gemm_dma(Prob& pb, int items, int nk) {
  constexpr int S = Cfg::STAGES;
  __shared__ __align__(16) bf16_t ring[S * Cfg::STAGE_ELEMS];
  const XcdSplit sp = xcd_split(items);
  if (sp.first >= sp.end || nk <= 0) return;
  const int n_mine = (sp.end - sp.first + sp.stride - 1) / sp.stride;
  const int total = n_mine * nk;
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));

  if (wave >= kComputeWaves) {
    const int part = wave - kComputeWaves;
    DmaLoader<Cfg> ld;
    int l_ord = 0, l_kt = 0, l_slot = 0;  // load cursor
    pb.setup(sp.first, ld, part);
    auto issue_next = [&]() {
      dma_issue<Cfg>(ld, l_kt, ring + l_slot * Cfg::STAGE_ELEMS, part);
      l_slot = (l_slot + 1 == S) ? 0 : l_slot + 1;
      if (++l_kt == nk) {
        l_kt = 0;
        if (++l_ord < n_mine) pb.setup(sp.first + l_ord * sp.stride, ld, part);
      }
    };
    for (int p = 0; p < S - 1 && p < total; ++p) issue_next();
    for (int g = 0; g < total; ++g) {
      dma_wait_stage<Cfg>(total - 1 - g);
      __builtin_amdgcn_s_barrier();
      if (g + S - 1 < total) issue_next();
    }
    return;
  }

  const int lane = threadIdx.x & 63;
  const int wm = wave / Cfg::WN, wn = wave % Cfg::WN;
  Acc<Cfg> acc;
  int c_slot = 0;
  for (int c_ord = 0; c_ord < n_mine; ++c_ord) {
    const int item = sp.first + c_ord * sp.stride;
    acc.zero();
    mma_item<Cfg>(dma_active_frags<Cfg>(wm, pb.rows(item)), nk, ring, c_slot, acc, wm, wn, lane);
    pb.epilogue(item, acc);
  }
}

}  // namespace moe
