// Grouped SwiGLU expert FFN over the ragged per-expert row blocks.
//
// "Trillion-Parameter MoE Model Training Adaptation: Full-Stack Optimization
// Practices", §3: after the permute, the experts compute in grouped matrix
// multiplications; "Adapting Ultra-Large MoE Models: Engineering Practices and
// Optimization Pathways", §3.3: each expert's tokens form a regular GEMM batch.
// LoRA ("Adapting Trillion-Parameter MoE Models for LoRA Fine-Tuning: A
// Full-Stack Engineering Guide", §3): U += s (X A_u^T) B_u^T and
// O += s (H A_d^T) B_d^T, with the rank-r products kept in fp32.
//
// bf16 path:
//   K-tiles   one block turns offsets into the list of (expert, first row)
//             row tiles of 128 rows; the GEMMs walk that list on the device,
//             so no row count ever travels to the host.
//   K8 gate_up  per (row tile, 128 FFN columns), reading token rows through
//             row_src (the dispatch gather fused into the A loader, so the
//             permuted copy of x never has to exist); the B tile interleaves 16 rows
//             of W_g and the same 16 rows of W_u, so each lane ends up holding
//             G and U of the same (row, column) and applies silu(G) * U in
//             registers; H is rounded to bf16.
//   K9 down   per (row tile, 256 output columns): O = H W_d^T (+ LoRA).
// Both run on the persistent pipelined driver of mfma_tile.h: one workgroup
// per CU walks the items, each XCD taking a contiguous range so row tiles
// that share A or B stay in one L2.
// fp32 path (small parity shapes): one thread per output element.
#include <type_traits>

#include "common.h"
#include "mfma_tile.h"

namespace moe {

// Ring depth of the grouped GEMMs (slots of 24 KB; one workgroup per CU).
#ifndef MOE_GEMM_STAGES
#define MOE_GEMM_STAGES 6
#endif
// 128 x 256 tiles. Two wave layouts:
//   GemmCfg      2 x 2 compute waves (one per SIMD), each with 4 interleaved
//                row fragments x 8 column fragments (64 x 128 of the tile),
//                + 4 producers: for weight-streaming shapes (few rows per
//                expert), where the MFMAs are far from the bound;
//   GemmCfgWide  2 x 4 compute waves (two per SIMD: one wave alone issues
//                MFMAs at about half the unit's rate), 64 x 64 each, + 4
//                producers: for shapes with many rows per expert, where the
//                MFMA issue rate decides.
using GemmCfg = DmaCfg<kGemmBM, 256, MOE_GEMM_STAGES, 2>;
using GemmCfgWide = DmaCfg<kGemmBM, 256, MOE_GEMM_STAGES, 2, 8, 4>;
// 320 x 128 tiles for experts with a few hundred rows: an item takes up to
// 320 rows, i.e. all rows of an expert with at most 320, so each weight tile
// is streamed once per expert instead of once per 128-row tile, and the
// items (experts x column blocks) fit the CUs in one round. 4 x 2 compute
// waves (two per SIMD), each 5 interleaved row fragments x 4 column
// fragments (80 x 64), + 4 producers. Split ring: the token rows (20 KB a
// stage, shared through the L2 by the expert's column blocks) in
// MOE_GEMM_TALL_STAGES slots, the streamed weight tiles (8 KB a stage, from
// HBM) in MOE_GEMM_TALL_BSTAGES slots, so more of the weight stream is in
// flight.
#ifndef MOE_GEMM_TALL_STAGES
#define MOE_GEMM_TALL_STAGES 3
#endif
#ifndef MOE_GEMM_TALL_BSTAGES
#define MOE_GEMM_TALL_BSTAGES 12
#endif
constexpr int kTallBM = 320;
using GemmCfgTall = DmaCfg<kTallBM, 128, MOE_GEMM_TALL_STAGES, 4, 8, 4, 32, MOE_GEMM_TALL_BSTAGES>;

// Rows per local expert expected under uniform routing (capped by the
// capacity) at which the tall layout is used.
constexpr int kWideRowsPerExpert = 192;

int gemm_tile_rows(const moe_shape_t& s) {
  int64_t per_expert = (int64_t)s.T * s.k / s.E;
  if (s.capacity > 0 && per_expert > s.capacity) per_expert = s.capacity;
  return per_expert >= kWideRowsPerExpert ? GemmCfgTall::BM : GemmCfg::BM;
}

int64_t packed_h_elems(const moe_shape_t& s) {
  const int64_t bm = gemm_tile_rows(s);
  if (bm != kTallBM) return 0;  // the 128-row tiles keep H row-major
  return ((max_rows(s) + bm - 1) / bm + (s.e_hi - s.e_lo)) * bm * s.f;
}

__global__ __launch_bounds__(1024) void build_row_tiles(const int32_t* __restrict__ offsets, int L,
                                                        int bm, int max_tiles,
                                                        int32_t* __restrict__ tiles) {
  __shared__ int wsum[16];
  const int le = threadIdx.x;
  const int n = le < L ? offsets[le + 1] - offsets[le] : 0;
  const int mt = (n + bm - 1) / bm;
  // exclusive scan of mt over the block
  const int lane = le & 63, wave = le >> 6;
  int incl = mt;
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) {
    const int o = __shfl_up(incl, m, kWave);
    if (lane >= m) incl += o;
  }
  if (lane == 63) wsum[wave] = incl;
  __syncthreads();
  int before = 0, total = 0;
  for (int w = 0; w < 16; ++w) {
    if (w < wave) before += wsum[w];
    total += wsum[w];
  }
  const int base = before + incl - mt;
  for (int i = 0; i < mt; ++i) {
    tiles[2 * (base + i)] = le;
    tiles[2 * (base + i) + 1] = i * bm;
  }
  if (le == 0) tiles[2 * max_tiles] = total;
}

// 64 bytes of zeros: the B rows of gate columns in the extra adapter K step.
__device__ __align__(64) bf16_t kLoraZeroRow[32] = {};

// Row-tile item of a grouped GEMM: expert, first row of the tile, rows valid.
struct RowTile {
  int le, r0, valid;
  int64_t row0;  // first dispatched row of the tile
};
template <int BM>
__device__ __forceinline__ RowTile row_tile(const int32_t* tiles, const int32_t* offsets, int ti) {
  RowTile t;
  t.le = ld_uniform(tiles, 2 * ti);
  t.r0 = ld_uniform(tiles, 2 * ti + 1);
  const int seg = ld_uniform(offsets, t.le);
  t.valid = min(BM, ld_uniform(offsets, t.le + 1) - seg - t.r0);
  t.row0 = (int64_t)seg + t.r0;
  return t;
}

// Source row of this lane's chunk in DMA instruction i of an A tile gathered
// through row_src (first = 16 i). Lane l needs entry row0 + min(first + l / 4, valid - 1)
// of row_src; the 16 entries of one instruction's rows are fetched with one
// 16-dword scalar load from a window [base, base + 16) inside the R written
// entries, and each lane picks its entry with a 4-level select on the bits of
// its offset in the window. Scalar loads count on the LGKM counter, so a new
// item's gather does not drain the DMA stages still in flight the way a
// vector load's vmcnt(0) wait would. With fewer than 16 rows in all, a plain
// vector load is used.
template <class Cfg>
__device__ __forceinline__ int64_t gathered_row(const int32_t* row_src, const RowTile& t, int i, int R) {
  const int first = 16 * i;
  const int64_t gr = t.row0 + min(first + (int)((threadIdx.x & 63) >> 2), t.valid - 1);
  if (R < 16) return row_src[gr];
  const int64_t base = min(t.row0 + min(first, t.valid - 1), (int64_t)R - 16);  // wave-uniform
  const i32x16_t v = *(const_i32x16_ptr_t)(row_src + base);
  const int e = (int)(gr - base);  // 0 .. 15
  // bitwise selects (not an indexed array, which would live in scratch)
  const int m0 = -(e & 1), m1 = -((e >> 1) & 1), m2 = -((e >> 2) & 1), m3 = -((e >> 3) & 1);
  int l1[8], l2[4], l3[2];
#pragma unroll
  for (int k = 0; k < 8; ++k) l1[k] = (v[2 * k + 1] & m0) | (v[2 * k] & ~m0);
#pragma unroll
  for (int k = 0; k < 4; ++k) l2[k] = (l1[2 * k + 1] & m1) | (l1[2 * k] & ~m1);
#pragma unroll
  for (int k = 0; k < 2; ++k) l3[k] = (l2[2 * k + 1] & m2) | (l2[2 * k] & ~m2);
  return (l3[1] & m3) | (l3[0] & ~m3);
}

// K8: H = silu(X W_g^T) * (X W_u^T [+ s Z_u B_u^T]) for one (row tile, 128
// FFN columns) item. Rows of X are x[row_src[p]] (gather fused into the A
// loader) or, with row_src == NULL, x[p] of an already gathered matrix.
// LORA (a separate instantiation each, so the plain kernels carry no adapter
// code): 0 none; 1 the epilogue adds the rank-r adapter term in fp32;
// 2 (r = 16) one extra K step carries it through the matrix cores: A = the
// row's s Z as bf16 high and low parts (zx, 32 per row), B = the adapter row
// twice (high and low parts meet the same values), zeros for gate columns.
template <class Cfg, int LORA = 0>
struct GateUpProb {
  static_assert(Cfg::FN % 4 == 0, "the epilogue stores two (G, U) fragment pairs at a time");
  static constexpr int kExtra = LORA == 2 ? 1 : 0;
  // H tile-packed on the tall tiles (see DownProb)
  static constexpr bool kPackedH = LORA == 0 && Cfg::BM == kTallBM;
  const bf16_t* x;
  const int32_t* row_src;
  const int32_t* offsets;
  const int32_t* tiles;
  const bf16_t* w_gate;
  const bf16_t* w_up;
  const bf16_t* w_packed;  // packed gate/up tiles, or NULL for row-major w_gate / w_up
  int d, f, nt, L;
  const float* zu;
  const bf16_t* b_up;
  int r;
  float scale;
  bf16_t* hbuf;
  bf16_t* act_save;
  const bf16_t* zx = nullptr;  // LORA == 2: [Rmax, 32] s Z_u high | low
  // the weight tiles are expected to be read by one row tile each (an
  // expert's rows fit one tile): fetch them with the streaming hint
  bool stream_b = false;
  static constexpr int HALF = Cfg::BN / 2;  // FFN columns per item (the last item may be partial)

  __device__ __forceinline__ int rows(int item) const {
    return row_tile<Cfg::BM>(tiles, offsets, item / nt).valid;
  }

  __device__ __forceinline__ void setup(int item, DmaLoader<Cfg>& ld, int part) const {
    const RowTile t = row_tile<Cfg::BM>(tiles, offsets, item / nt);
    const int ni = item % nt;
    const int ce = dma_chunk_elem<Cfg>();
    ld.b_stream = stream_b;
#pragma unroll
    for (int q = 0; q < Cfg::A_DMA / Cfg::DW; ++q) {
      const int i = q * Cfg::DW + part;
      const int64_t src = row_src ? gathered_row<Cfg>(row_src, t, i, ld_uniform(offsets, L))
                                  : t.row0 + min(dma_row<Cfg>(i), t.valid - 1);
      ld.a[q] = x + src * d + ce;
    }
    if (w_packed) {
      // packed tiles hold 64 FFN columns (128 interleaved rows) each; blocks
      // past f (a partial last item) re-read the last block, never stored
      const int nb = f / 64, nk = d / Cfg::BK;
      const int64_t bstride = (int64_t)nk * kPackTileElems;
#pragma unroll
      for (int q = 0; q < Cfg::B_DMA / Cfg::DW; ++q) {
        const int i = q * Cfg::DW + part;
        const int b = min(ni * (HALF / 64) + i / (kPackTileRows / 16), nb - 1);
        const bf16_t* tile0 = w_packed + ((int64_t)t.le * nb + b) * bstride;
        ld.b[q] = packed_b_ptr(tile0, i % (kPackTileRows / 16), 0);
      }
      ld.b_kstep = kPackTileElems;
      return;
    }
#pragma unroll
    for (int q = 0; q < Cfg::B_DMA / Cfg::DW; ++q) {
      const int jb = dma_row<Cfg>(q * Cfg::DW + part);
      const int frag = jb >> 4;
      const int fcol = min(ni * HALF + (frag >> 1) * 16 + (jb & 15), f - 1);
      ld.b[q] = ((frag & 1) ? w_up : w_gate) + ((int64_t)t.le * f + fcol) * d + ce;
    }
  }

  // LORA == 2: pointers of the extra K step (see above)
  __device__ __forceinline__ void setup_extra(int item, DmaLoader<Cfg>& ld, int part) const {
    const RowTile t = row_tile<Cfg::BM>(tiles, offsets, item / nt);
    const int ni = item % nt;
    const int ce = dma_chunk_elem<Cfg>();
#pragma unroll
    for (int q = 0; q < Cfg::A_DMA / Cfg::DW; ++q)
      ld.a[q] = zx + (t.row0 + min(dma_row<Cfg>(q * Cfg::DW + part), t.valid - 1)) * 32 + ce;
#pragma unroll
    for (int q = 0; q < Cfg::B_DMA / Cfg::DW; ++q) {
      const int jb = dma_row<Cfg>(q * Cfg::DW + part);
      const int frag = jb >> 4;
      const int fcol = min(ni * HALF + (frag >> 1) * 16 + (jb & 15), f - 1);
      ld.b[q] = (frag & 1) ? b_up + ((int64_t)t.le * f + fcol) * 16 + (ce & 8) : kLoraZeroRow;
    }
  }

  __device__ __forceinline__ void epilogue(int item, Acc<Cfg>& acc) const {
    const RowTile t = row_tile<Cfg::BM>(tiles, offsets, item / nt);
    const int ni = item % nt;
    // wave-uniform, so the column tests below branch on scalars and the
    // lane swaps of the paired stores run with every lane active
    const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    const int wm = wave / Cfg::WN, wn = wave % Cfg::WN;
#pragma unroll
    for (int i = 0; i < Cfg::FM; ++i) {
      const int base = frag_row0<Cfg>(wm, i);  // wave-uniform
      if (base >= t.valid) continue;
      const int rin = base + (lane & 15);
      const bool ok = rin < t.valid;
      const int64_t row = t.row0 + rin;
#pragma unroll
      for (int jj = 0; jj < Cfg::FN; jj += 4) {
        // fragments jg + 2 h (h = 0, 1) hold G and jg + 2 h + 1 hold U, of the
        // 16 FFN columns c0 + 16 h .. +15; f % 64 == 0, so the 32 columns are
        // all inside f or all past it
        const int jg = wn * Cfg::FN + jj;
        const int c0 = ni * HALF + (jg >> 1) * 16;
        if (c0 >= f) continue;
        float h[2][4], g[2][4], uu[2][4];
#pragma unroll
        for (int p = 0; p < 2; ++p) {
          float lt[4] = {0.f, 0.f, 0.f, 0.f};
          if constexpr (LORA == 1) {
            const int fcol = c0 + 16 * p + (lane >> 4) * 4;
            if (ok) lora_term_rows(zu + row * r, b_up + ((int64_t)t.le * f + fcol) * r, r, lt);
          }
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            g[p][q] = acc.v[i][jj + 2 * p][q];
            float u = acc.v[i][jj + 2 * p + 1][q];
            if constexpr (LORA == 1) u = fmaf(scale, lt[q], u);
            uu[p][q] = u;
            h[p][q] = silu_f(g[p][q]) * u;
          }
        }
        const int col = c0 + pair_col(lane);
        const uint4 hv = pair_cols_bf16(h[0], h[1]);
        // H (read by the down GEMM) and the saved rows (read by the
        // backward) with the non-temporal hint: the token rows this launch
        // still gathers keep the L2 (896 experts of ~73 rows, d = 2048: gate/up
        // 363 -> 348 us)
        if constexpr (kPackedH) {
          // one 16-row x 64-byte block: the store writes 1 KB contiguously
          bf16_t* hp = hbuf + (int64_t)(item / nt) * Cfg::BM * f + ((c0 >> 5) * Cfg::BM + rin) * 32 + pair_col(lane);
          if (ok) store16_nt(hp, hv);
        } else {
          if (ok) store16_nt(hbuf + row * f + col, hv);
        }
        if (act_save) {  // kernel-uniform
          const uint4 gv = pair_cols_bf16(g[0], g[1]);
          const uint4 uv = pair_cols_bf16(uu[0], uu[1]);
          if (ok) {
            bf16_t* as = act_save + row * 3 * f + col;
            store16_nt(as, gv);
            store16_nt(as + f, hv);
            store16_nt(as + 2 * f, uv);
          }
        }
      }
    }
  }
};

template <class Cfg, int LORA>
__global__ __launch_bounds__(Cfg::THREADS, Cfg::WAVES_PER_SIMD) void gate_up_bf16(GateUpProb<Cfg, LORA> pb, int max_tiles) {
  const int items = ld_uniform(pb.tiles, 2 * max_tiles) * pb.nt;
  persistent_gemm_dma<Cfg>(pb, items, pb.d / Cfg::BK);
}

// K9: O = H W_d^T [+ s Z_d B_d^T] for one (row tile, 256 output columns) item.
// LORA (a separate instantiation each, so the plain kernels carry no adapter
// code): 0 none; 1 the epilogue adds the rank-r adapter term in fp32;
// 2 (r = 16) one extra K step carries it through the matrix cores: A = the
// row's s Z as bf16 high and low parts (zx, 32 per row), B = the adapter row
// twice (high and low parts meet the same values), zeros for gate columns.
template <class Cfg, int LORA = 0>
struct DownProb {
  static_assert(Cfg::FN % 2 == 0, "the epilogue stores fragment pairs");
  static constexpr int kExtra = LORA == 2 ? 1 : 0;
  // On the tall tiles, without adapters, H is tile-packed: row tile t owns
  // BM x f elements at t * BM * f, stored [K step of 32][tile row][32
  // values], so the 16 rows of one DMA instruction are 1 KB of contiguous
  // memory (64-byte pieces 2 f bytes apart in the row-major form), and the
  // gate/up epilogue writes each such block with one store instruction.
  // Measured on 14 experts of ~296 rows (d = 4096, f = 1024): down 59 -> 52
  // us, gate/up unchanged; on the 128-row tiles (896 experts of ~73 rows) a
  // wash (down -1, gate/up +3..+5 us), so
  // those keep the row-major form, as do the adapter paths, which read H
  // row by row.
  static constexpr bool kPackedH = LORA == 0 && Cfg::BM == kTallBM;
  const bf16_t* hbuf;
  const int32_t* offsets;
  const int32_t* tiles;
  const bf16_t* w_down;
  const bf16_t* w_packed;  // packed down tiles, or NULL for row-major w_down
  int d, f, nt;
  const float* zd;
  const bf16_t* b_down;
  int r;
  float scale;
  bf16_t* y_perm;
  const bf16_t* zx = nullptr;  // LORA == 2: [Rmax, 32] s Z_d high | low
  bool stream_b = false;        // as GateUpProb

  __device__ __forceinline__ int rows(int item) const {
    return row_tile<Cfg::BM>(tiles, offsets, item / nt).valid;
  }

  __device__ __forceinline__ void setup(int item, DmaLoader<Cfg>& ld, int part) const {
    const RowTile t = row_tile<Cfg::BM>(tiles, offsets, item / nt);
    const int n0 = (item % nt) * Cfg::BN;
    const int ce = dma_chunk_elem<Cfg>();
    ld.b_stream = stream_b;
    if constexpr (kPackedH) {
      // instructions wholly past the valid rows re-read the last valid block
      const bf16_t* hp = hbuf + (int64_t)(item / nt) * Cfg::BM * f;
      const int last = (t.valid - 1) / Cfg::RPD;
#pragma unroll
      for (int q = 0; q < Cfg::A_DMA / Cfg::DW; ++q) {
        const int blk = min(q * Cfg::DW + part, last);
        ld.a[q] = hp + (Cfg::RPD * blk + (threadIdx.x & 63) / Cfg::CPR) * Cfg::BK + ce;
      }
      ld.a_kstep = Cfg::BM * Cfg::BK;
    } else {
#pragma unroll
      for (int q = 0; q < Cfg::A_DMA / Cfg::DW; ++q)
        ld.a[q] = hbuf + (t.row0 + min(dma_row<Cfg>(q * Cfg::DW + part), t.valid - 1)) * f + ce;
    }
    if (w_packed) {
      // packed tiles hold 128 output columns each; blocks past d (a partial
      // last item) re-read the last block, never stored
      const int nb = d / kPackTileRows, nk = f / Cfg::BK;
      const int64_t bstride = (int64_t)nk * kPackTileElems;
#pragma unroll
      for (int q = 0; q < Cfg::B_DMA / Cfg::DW; ++q) {
        const int i = q * Cfg::DW + part;
        const int b = min((item % nt) * (Cfg::BN / kPackTileRows) + i / (kPackTileRows / 16), nb - 1);
        const bf16_t* tile0 = w_packed + ((int64_t)t.le * nb + b) * bstride;
        ld.b[q] = packed_b_ptr(tile0, i % (kPackTileRows / 16), 0);
      }
      ld.b_kstep = kPackTileElems;
      return;
    }
#pragma unroll
    for (int q = 0; q < Cfg::B_DMA / Cfg::DW; ++q)
      ld.b[q] = w_down + ((int64_t)t.le * d + min(n0 + dma_row<Cfg>(q * Cfg::DW + part), d - 1)) * f + ce;
  }

  // LORA == 2: pointers of the extra K step (see GateUpProb)
  __device__ __forceinline__ void setup_extra(int item, DmaLoader<Cfg>& ld, int part) const {
    const RowTile t = row_tile<Cfg::BM>(tiles, offsets, item / nt);
    const int n0 = (item % nt) * Cfg::BN;
    const int ce = dma_chunk_elem<Cfg>();
#pragma unroll
    for (int q = 0; q < Cfg::A_DMA / Cfg::DW; ++q)
      ld.a[q] = zx + (t.row0 + min(dma_row<Cfg>(q * Cfg::DW + part), t.valid - 1)) * 32 + ce;
#pragma unroll
    for (int q = 0; q < Cfg::B_DMA / Cfg::DW; ++q) {
      const int n = min(n0 + dma_row<Cfg>(q * Cfg::DW + part), d - 1);
      ld.b[q] = b_down + ((int64_t)t.le * d + n) * 16 + (ce & 8);
    }
  }

  __device__ __forceinline__ void epilogue(int item, Acc<Cfg>& acc) const {
    const RowTile t = row_tile<Cfg::BM>(tiles, offsets, item / nt);
    const int n0 = (item % nt) * Cfg::BN;
    // wave-uniform, so the column tests below branch on scalars and the
    // lane swaps of the paired stores run with every lane active
    const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    const int wm = wave / Cfg::WN, wn = wave % Cfg::WN;
#pragma unroll
    for (int i = 0; i < Cfg::FM; ++i) {
      const int base = frag_row0<Cfg>(wm, i);  // wave-uniform
      if (base >= t.valid) continue;
      const int rin = base + (lane & 15);
      const bool ok = rin < t.valid;
      const int64_t row = t.row0 + rin;
#pragma unroll
      for (int j = 0; j < Cfg::FN; j += 2) {
        // fragments j, j + 1: 32 output columns from c0; d % 64 == 0, so
        // they are all valid or all not
        const int c0 = n0 + wn * (Cfg::BN / Cfg::WN) + j * 16;
        if (c0 >= d) continue;
        float o[2][4];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          float lt[4] = {0.f, 0.f, 0.f, 0.f};
          if constexpr (LORA == 1) {
            const int n = n0 + dma_out_col<Cfg>(wn, j + h, lane);
            if (ok) lora_term_rows(zd + row * r, b_down + ((int64_t)t.le * d + n) * r, r, lt);
          }
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            o[h][q] = acc.v[i][j + h][q];
            if constexpr (LORA == 1) o[h][q] = fmaf(scale, lt[q], o[h][q]);
          }
        }
        const uint4 v = pair_cols_bf16(o[0], o[1]);
        if (ok) *reinterpret_cast<uint4*>(y_perm + row * d + c0 + pair_col(lane)) = v;
      }
    }
  }
};

template <class Cfg, int LORA>
__global__ __launch_bounds__(Cfg::THREADS, Cfg::WAVES_PER_SIMD) void down_bf16(DownProb<Cfg, LORA> pb, int max_tiles) {
  const int items = ld_uniform(pb.tiles, 2 * max_tiles) * pb.nt;
  persistent_gemm_dma<Cfg>(pb, items, pb.f / Cfg::BK);
}

// ------------------------------------------------- backward on the DMA engine
// The full backward's two grouped GEMMs contract over the other index of the
// frozen weights than the forward does (dH = dO W_d contracts over d, dX =
// [dG dU] [W_g; W_u] over f), so their B operands are the transposed weights,
// packed once (pack_trans below) into the same tile format as the forward's
// down weights: W_d^T [L, f, d] for dH, [W_g; W_u]^T [L, d, 2f] for dX.

// dH[row, n] = g_row dY[src_row] . W_d^T[n] (+ s wproj[row] . A_d[:, n]), then
// dG = dH U silu'(G), dU = dH silu(G) (G, U from act_save) -> dgu bf16.
// LORA: the epilogue adds the rank-r adapter term (a separate instantiation,
// so the plain kernels carry no adapter code).
// DU32: only dU = dH silu(G), in fp32, to du32 [Rmax, f] (the LoRA adapter
// gradients need no dG).
// KX (with LORA): the adapter term rides as one extra K step instead: A =
// zx (s dY B_d as bf16 high | low, 32 per row), B = adt rows (A_d^T, the
// 16 adapter values of each output column, read twice); the row gate then
// scales the whole sum.
template <class Cfg, bool LORA = false, bool DU32 = false, bool KX = false>
struct DguPackedProb {
  static_assert(Cfg::FN % 2 == 0, "the epilogue takes fragment pairs");
  static constexpr int kExtra = KX ? 1 : 0;
  const bf16_t* dy;
  const int32_t* row_src;
  const float* row_gate;
  const int32_t* offsets;
  const int32_t* tiles;
  const bf16_t* packed;  // W_d^T tiles
  int d, f, nt, L;
  const float* wproj;
  const bf16_t* a_down;
  int r;
  float scale;
  const bf16_t* act_save;
  bf16_t* dgu;
  float* du32 = nullptr;
  const bf16_t* zx = nullptr;   // KX: [Rmax, 32]
  const bf16_t* adt = nullptr;  // KX: [L, f, 16]

  __device__ __forceinline__ void setup_extra(int item, DmaLoader<Cfg>& ld, int part) const {
    const RowTile t = row_tile<Cfg::BM>(tiles, offsets, item / nt);
    const int n0 = (item % nt) * Cfg::BN;
    const int ce = dma_chunk_elem<Cfg>();
#pragma unroll
    for (int q = 0; q < Cfg::A_DMA / Cfg::DW; ++q)
      ld.a[q] = zx + (t.row0 + min(dma_row<Cfg>(q * Cfg::DW + part), t.valid - 1)) * 32 + ce;
#pragma unroll
    for (int q = 0; q < Cfg::B_DMA / Cfg::DW; ++q) {
      const int n = min(n0 + dma_row<Cfg>(q * Cfg::DW + part), f - 1);
      ld.b[q] = adt + ((int64_t)t.le * f + n) * 16 + (ce & 8);
    }
  }

  __device__ __forceinline__ int rows(int item) const {
    return row_tile<Cfg::BM>(tiles, offsets, item / nt).valid;
  }

  __device__ __forceinline__ void setup(int item, DmaLoader<Cfg>& ld, int part) const {
    const RowTile t = row_tile<Cfg::BM>(tiles, offsets, item / nt);
    const int ni = item % nt;
    const int ce = dma_chunk_elem<Cfg>();
#pragma unroll
    for (int q = 0; q < Cfg::A_DMA / Cfg::DW; ++q) {
      const int i = q * Cfg::DW + part;
      ld.a[q] = dy + gathered_row<Cfg>(row_src, t, i, ld_uniform(offsets, L)) * d + ce;
    }
    const int nb = f / kPackTileRows, nk = d / Cfg::BK;
    const int64_t bstride = (int64_t)nk * kPackTileElems;
#pragma unroll
    for (int q = 0; q < Cfg::B_DMA / Cfg::DW; ++q) {
      const int i = q * Cfg::DW + part;
      const int b = min(ni * (Cfg::BN / kPackTileRows) + i / (kPackTileRows / 16), nb - 1);
      ld.b[q] = packed_b_ptr(packed + ((int64_t)t.le * nb + b) * bstride, i % (kPackTileRows / 16), 0);
    }
    ld.b_kstep = kPackTileElems;
  }

  __device__ __forceinline__ void epilogue(int item, Acc<Cfg>& acc) const {
    const RowTile t = row_tile<Cfg::BM>(tiles, offsets, item / nt);
    const int n0 = (item % nt) * Cfg::BN;
    // wave-uniform, so the column tests below branch on scalars and the
    // lane swaps of the paired stores run with every lane active
    const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    const int wm = wave / Cfg::WN, wn = wave % Cfg::WN;
#pragma unroll
    for (int i = 0; i < Cfg::FM; ++i) {
      const int base = frag_row0<Cfg>(wm, i);
      if (base >= t.valid) continue;
      const int rin = base + (lane & 15);
      const bool ok = rin < t.valid;
      const int64_t row = t.row0 + rin;
      const float g_row = ok ? row_gate[row] : 0.f;
      if constexpr (DU32) {
        // fp32 dU only: a lane's four columns are one 16-byte store already
#pragma unroll
        for (int j = 0; j < Cfg::FN; ++j) {
          if (n0 + wn * (Cfg::BN / Cfg::WN) + j * 16 >= f) continue;
          const int n = n0 + dma_out_col<Cfg>(wn, j, lane);
          if (!ok) continue;
          const uint2 gv = *reinterpret_cast<const uint2*>(act_save + row * 3 * f + n);
          float duv[4], lt[4] = {0.f, 0.f, 0.f, 0.f};
          if constexpr (LORA && !KX) lora_term_cols(wproj + row * r, a_down + (int64_t)t.le * r * f + n, f, r, lt);
          const uint32_t gw[2] = {gv.x, gv.y};
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const float dh = fmaf(g_row, acc.v[i][j][q], scale * lt[q]);
            const float g = bf16_to_f32(static_cast<bf16_t>(gw[q >> 1] >> ((q & 1) * 16)));
            duv[q] = dh * (g / (1.0f + expf(-g)));
          }
          *reinterpret_cast<float4*>(du32 + row * f + n) = make_float4(duv[0], duv[1], duv[2], duv[3]);
        }
        continue;
      }
#pragma unroll
      for (int j = 0; j < Cfg::FN; j += 2) {
        // fragments j, j + 1: 32 FFN columns from c0, all inside f or all
        // past it (f % 64 == 0); lane l takes columns n .. n + 7
        const int c0 = n0 + wn * (Cfg::BN / Cfg::WN) + j * 16;
        if (c0 >= f) continue;
        float a[8];
        pair_cols_f32(acc.v[i][j], acc.v[i][j + 1], a);  // every lane, before the row test
        const int n = c0 + pair_col(lane);
        if (!ok) continue;
        const bf16_t* as = act_save + row * 3 * f + n;
        const uint4 gv = *reinterpret_cast<const uint4*>(as);
        const uint4 uv = *reinterpret_cast<const uint4*>(as + 2 * f);
        float lt[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
        if constexpr (LORA && !KX) {
          float l0[4], l1[4];
          lora_term_cols(wproj + row * r, a_down + (int64_t)t.le * r * f + n, f, r, l0);
          lora_term_cols(wproj + row * r, a_down + (int64_t)t.le * r * f + n + 4, f, r, l1);
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            lt[q] = l0[q];
            lt[4 + q] = l1[q];
          }
        }
        const uint32_t gw[4] = {gv.x, gv.y, gv.z, gv.w}, uw[4] = {uv.x, uv.y, uv.z, uv.w};
        float dgv[8], duv[8];
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          const float dh = fmaf(g_row, a[q], scale * lt[q]);
          const float g = bf16_to_f32(static_cast<bf16_t>(gw[q >> 1] >> ((q & 1) * 16)));
          const float u = bf16_to_f32(static_cast<bf16_t>(uw[q >> 1] >> ((q & 1) * 16)));
          const float sg = 1.0f / (1.0f + expf(-g));
          dgv[q] = dh * u * (sg * (1.0f + g * (1.0f - sg)));
          duv[q] = dh * g * sg;
        }
        *reinterpret_cast<uint4*>(dgu + row * 2 * f + n) =
            make_uint4(f32x2_to_bf16x2(dgv[0], dgv[1]), f32x2_to_bf16x2(dgv[2], dgv[3]),
                       f32x2_to_bf16x2(dgv[4], dgv[5]), f32x2_to_bf16x2(dgv[6], dgv[7]));
        *reinterpret_cast<uint4*>(dgu + row * 2 * f + f + n) =
            make_uint4(f32x2_to_bf16x2(duv[0], duv[1]), f32x2_to_bf16x2(duv[2], duv[3]),
                       f32x2_to_bf16x2(duv[4], duv[5]), f32x2_to_bf16x2(duv[6], duv[7]));
      }
    }
  }
};

template <class Cfg, bool LORA, bool DU32 = false, bool KX = false>
__global__ __launch_bounds__(Cfg::THREADS, Cfg::WAVES_PER_SIMD) void expert_dgu_dma(DguPackedProb<Cfg, LORA, DU32, KX> pb,
                                                                                   int max_tiles) {
  const int items = ld_uniform(pb.tiles, 2 * max_tiles) * pb.nt;
  persistent_gemm_dma<Cfg>(pb, items, pb.d / Cfg::BK);
}

// dX[row, n] = dgu[row] . [W_g; W_u]^T[n] (+ s vproj[row] . A_u[:, n]), fp32.
// LORA: the epilogue adds the rank-r adapter term (a separate instantiation,
// so the plain kernels carry no adapter code).
template <class Cfg, bool LORA = false>
struct DxPackedProb {
  const bf16_t* dgu;
  const int32_t* offsets;
  const int32_t* tiles;
  const bf16_t* packed;  // [W_g; W_u]^T tiles
  int d, f, nt;
  const float* vproj;
  const bf16_t* a_up;
  int r;
  float scale;
  float* dx_rows;

  __device__ __forceinline__ int rows(int item) const {
    return row_tile<Cfg::BM>(tiles, offsets, item / nt).valid;
  }

  __device__ __forceinline__ void setup(int item, DmaLoader<Cfg>& ld, int part) const {
    const RowTile t = row_tile<Cfg::BM>(tiles, offsets, item / nt);
    const int ni = item % nt;
    const int ce = dma_chunk_elem<Cfg>();
#pragma unroll
    for (int q = 0; q < Cfg::A_DMA / Cfg::DW; ++q)
      ld.a[q] = dgu + (t.row0 + min(dma_row<Cfg>(q * Cfg::DW + part), t.valid - 1)) * 2 * f + ce;
    const int nb = d / kPackTileRows, nk = 2 * f / Cfg::BK;
    const int64_t bstride = (int64_t)nk * kPackTileElems;
#pragma unroll
    for (int q = 0; q < Cfg::B_DMA / Cfg::DW; ++q) {
      const int i = q * Cfg::DW + part;
      const int b = min(ni * (Cfg::BN / kPackTileRows) + i / (kPackTileRows / 16), nb - 1);
      ld.b[q] = packed_b_ptr(packed + ((int64_t)t.le * nb + b) * bstride, i % (kPackTileRows / 16), 0);
    }
    ld.b_kstep = kPackTileElems;
  }

  __device__ __forceinline__ void epilogue(int item, Acc<Cfg>& acc) const {
    const RowTile t = row_tile<Cfg::BM>(tiles, offsets, item / nt);
    const int n0 = (item % nt) * Cfg::BN;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int wm = wave / Cfg::WN, wn = wave % Cfg::WN;
#pragma unroll
    for (int i = 0; i < Cfg::FM; ++i) {
      const int base = frag_row0<Cfg>(wm, i);
      if (base >= t.valid) continue;
      const int rin = base + (lane & 15);
      if (rin >= t.valid) continue;
      const int64_t row = t.row0 + rin;
#pragma unroll
      for (int j = 0; j < Cfg::FN; ++j) {
        if (n0 + wn * (Cfg::BN / Cfg::WN) + j * 16 >= d) continue;
        const int n = n0 + dma_out_col<Cfg>(wn, j, lane);
        float o[4], lt[4] = {0.f, 0.f, 0.f, 0.f};
        if constexpr (LORA) lora_term_cols(vproj + row * r, a_up + (int64_t)t.le * r * d + n, d, r, lt);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          o[q] = acc.v[i][j][q];
          if constexpr (LORA) o[q] = fmaf(scale, lt[q], o[q]);
        }
        *reinterpret_cast<float4*>(dx_rows + row * d + n) = make_float4(o[0], o[1], o[2], o[3]);
      }
    }
  }
};

template <class Cfg, bool LORA>
__global__ __launch_bounds__(Cfg::THREADS, Cfg::WAVES_PER_SIMD) void expert_dx_dma(DxPackedProb<Cfg, LORA> pb,
                                                                                  int max_tiles) {
  const int items = ld_uniform(pb.tiles, 2 * max_tiles) * pb.nt;
  persistent_gemm_dma<Cfg>(pb, items, 2 * pb.f / Cfg::BK);
}

// dG/dU on CfgH tiles, then dX on Cfg tiles; with rebuild_for_dx the row
// tiles are rebuilt for Cfg's height in between (the list the caller built
// is for CfgH).
template <class CfgH, class Cfg>
static hipError_t launch_bwd_gemms_cfg(const Ctx& c, const moe_shape_t& s, const Workspace& ws,
                                       const LoraArgs* lo, const bf16_t* dy, const int32_t* row_src,
                                       const float* row_gate, const int32_t* offsets, const bf16_t* act_save,
                                       const bf16_t* dgu_packed, const bf16_t* dx_packed, bf16_t* dgu,
                                       float* dx_rows, int max_tiles, bool rebuild_for_dx = false) {
  const int L = s.e_hi - s.e_lo;
  const int64_t rmax = max_rows(s);
  hipError_t err;
  if (lo) {
    err = launch_lora_rowproj<bf16_t>(c, L, offsets, rmax, dy, s.d, row_src, row_gate, s.d, lo->b_down, false,
                                      lo->r, ws.wproj, ws.lora_mt);
    if (err != hipSuccess) return err;
  }
  auto dgu_launch = [&](auto with_lora) {
    constexpr bool LO = decltype(with_lora)::value;
    DguPackedProb<CfgH, LO> pb{dy, row_src, row_gate, offsets, ws.gemm_tiles, dgu_packed, s.d, s.f,
                               (s.f + CfgH::BN - 1) / CfgH::BN, L, lo ? ws.wproj : nullptr,
                               lo ? lo->a_down : nullptr, lo ? lo->r : 0, lo ? lo->scale : 0.f, act_save, dgu};
    TimedLaunch tl(MOE_K_EXPERT_DGU, c.stream);
    hipLaunchKernelGGL((expert_dgu_dma<CfgH, LO>), dim3(c.num_cus), dim3(CfgH::THREADS), 0, c.stream, pb,
                       max_tiles);
    return hipGetLastError();
  };
  if ((err = lo ? dgu_launch(std::true_type{}) : dgu_launch(std::false_type{})) != hipSuccess) return err;
  if (lo) {
    err = launch_lora_rowproj<bf16_t>(c, L, offsets, rmax, dgu + s.f, 2 * s.f, nullptr, nullptr, s.f, lo->b_up,
                                      false, lo->r, ws.vproj, ws.lora_mt);
    if (err != hipSuccess) return err;
  }
  if (rebuild_for_dx && (err = launch_row_tiles(c, offsets, L, max_tiles, ws.gemm_tiles, Cfg::BM)) != hipSuccess)
    return err;
  auto dx_launch = [&](auto with_lora) {
    constexpr bool LO = decltype(with_lora)::value;
    DxPackedProb<Cfg, LO> pb{dgu, offsets, ws.gemm_tiles, dx_packed, s.d, s.f, (s.d + Cfg::BN - 1) / Cfg::BN,
                             lo ? ws.vproj : nullptr, lo ? lo->a_up : nullptr, lo ? lo->r : 0,
                             lo ? lo->scale : 0.f, dx_rows};
    TimedLaunch tl(MOE_K_EXPERT_DX, c.stream);
    hipLaunchKernelGGL((expert_dx_dma<Cfg, LO>), dim3(c.num_cus), dim3(Cfg::THREADS), 0, c.stream, pb, max_tiles);
    return hipGetLastError();
  };
  return lo ? dx_launch(std::true_type{}) : dx_launch(std::false_type{});
}

// The LoRA backward's dU = (g dY W_d + s (dO B_d) A_d) silu(G), fp32 into
// ws.du, on the packed W_d^T (moe_pack_backward_weights); ws.wproj holds
// dO B_d and ws.gemm_tiles the row tiles.
template <class Cfg, bool KX>
static hipError_t launch_lora_dh_cfg(const Ctx& c, const moe_shape_t& s, const Workspace& ws, const LoraArgs& lo,
                                     const bf16_t* dy, const int32_t* row_src, const float* row_gate,
                                     const int32_t* offsets, const bf16_t* act_save, const bf16_t* dgu_packed,
                                     const bf16_t* adt, int max_tiles) {
  DguPackedProb<Cfg, true, true, KX> pb{dy, row_src, row_gate, offsets, ws.gemm_tiles, dgu_packed, s.d, s.f,
                                        (s.f + Cfg::BN - 1) / Cfg::BN, s.e_hi - s.e_lo, ws.wproj, lo.a_down, lo.r,
                                        lo.scale, act_save, nullptr, ws.du};
  pb.zx = ws.zx;
  pb.adt = adt;
  TimedLaunch tl(MOE_K_LORA_DH, c.stream);
  hipLaunchKernelGGL((expert_dgu_dma<Cfg, true, true, KX>), dim3(c.num_cus), dim3(Cfg::THREADS), 0, c.stream, pb,
                     max_tiles);
  return hipGetLastError();
}

hipError_t launch_lora_dh_packed(const Ctx& c, const moe_shape_t& s, const Workspace& ws, const LoraArgs& lo,
                                 const bf16_t* dy, const int32_t* row_src, const float* row_gate,
                                 const int32_t* offsets, const bf16_t* act_save, const bf16_t* dgu_packed,
                                 const bf16_t* adt) {
  const int max_tiles = gemm_max_tiles(s);
  int64_t per_expert = (int64_t)s.T * s.k / s.E;
  if (s.capacity > 0 && per_expert > s.capacity) per_expert = s.capacity;
  const bool wide = per_expert >= kWideRowsPerExpert;
#define MOE_DH(C, K) \
  launch_lora_dh_cfg<C, K>(c, s, ws, lo, dy, row_src, row_gate, offsets, act_save, dgu_packed, adt, max_tiles)
  if (adt) return wide ? MOE_DH(GemmCfgWide, true) : MOE_DH(GemmCfg, true);
  return wide ? MOE_DH(GemmCfgWide, false) : MOE_DH(GemmCfg, false);
#undef MOE_DH
}

hipError_t launch_bwd_gemms_packed(const Ctx& c, const moe_shape_t& s, const Workspace& ws, const LoraArgs* lo,
                                   const bf16_t* dy, const int32_t* row_src, const float* row_gate,
                                   const int32_t* offsets, const bf16_t* act_save, const bf16_t* dgu_packed,
                                   const bf16_t* dx_packed, bf16_t* dgu, float* dx_rows) {
  const int L = s.e_hi - s.e_lo;
  const int max_tiles = gemm_max_tiles(s);
  hipError_t err = launch_row_tiles(c, offsets, L, max_tiles, ws.gemm_tiles);
  if (err != hipSuccess) return err;
  int64_t per_expert = (int64_t)s.T * s.k / s.E;
  if (s.capacity > 0 && per_expert > s.capacity) per_expert = s.capacity;
  // dG/dU runs the two-waves-per-SIMD layout at every row count (its
  // epilogue reads G and U and writes two outputs per element; smaller wave
  // tiles measured faster even at 73 rows per expert: 293 -> 265 us; on
  // 320 x 64 tall tiles it measured 101 us against 86 on 14 experts of ~296
  // rows). dX (N = d) takes the tall tiles where the forward does: each
  // packed weight tile streams once per expert instead of once per 128-row
  // tile (14 experts of ~296 rows, d = 4096: 140 -> 119 us).
  if (per_expert >= kWideRowsPerExpert)
    return launch_bwd_gemms_cfg<GemmCfgWide, GemmCfgTall>(c, s, ws, lo, dy, row_src, row_gate, offsets, act_save,
                                                          dgu_packed, dx_packed, dgu, dx_rows, max_tiles, true);
  return launch_bwd_gemms_cfg<GemmCfgWide, GemmCfg>(c, s, ws, lo, dy, row_src, row_gate, offsets, act_save,
                                                    dgu_packed, dx_packed, dgu, dx_rows, max_tiles);
}

// Transposing pack: tile (le, n block of 128 rows, K step) of the matrix
// B[le][n][k] = (k < k_split ? src0 : src1)[le][k mod k_split][n] (row stride
// ld_k between consecutive k), laid out like pack_down's tiles.
__global__ __launch_bounds__(256) void pack_trans(const bf16_t* __restrict__ src0, const bf16_t* __restrict__ src1,
                                                  int k_split, int L, int rows, int K, int64_t ld_k,
                                                  int64_t le_stride, u32x4* __restrict__ out) {
  const int nk = K / 32, nt = rows / 128;
  const int64_t total = (int64_t)L * nt * nk * 512;
  for (int64_t id = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; id < total;
       id += (int64_t)gridDim.x * blockDim.x) {
    const int slot = (int)(id & 3), jb = (int)((id >> 2) & 127);
    const int64_t tile = id >> 9;
    const int kt = (int)(tile % nk);
    const int64_t rest = tile / nk;
    const int ni = (int)(rest % nt), le = (int)(rest / nt);
    const int c = slot ^ chunk_key(jb);
    const int n = ni * 128 + jb;
    uint32_t w[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      uint32_t pair = 0;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int k = kt * 32 + c * 8 + 2 * u + h;
        const bf16_t* src = k < k_split ? src0 : src1;
        const int kk = k < k_split ? k : k - k_split;
        const uint32_t v = static_cast<uint32_t>(src[(int64_t)le * le_stride + (int64_t)kk * ld_k + n]);
        pair |= v << (16 * h);
      }
      w[u] = pair;
    }
    out[id] = u32x4{w[0], w[1], w[2], w[3]};
  }
}

// Router part of dx on the DMA engine: dx[t, n] += dl_bf16[t] . W_r^T[n]
// (W_r^T packed like the expert tiles, rows n < d, K = E), dense items of
// 128 tokens x BN columns; the epilogue adds into the fp32 dx.
// STORE: dx = the product, written without reading dx (the expert part is
// added afterwards, only where a token has local rows).
template <class Cfg, bool STORE = false>
struct RouterBwdPackedProb {
  const bf16_t* dl;      // [T, E] bf16
  const bf16_t* packed;  // W_r^T tiles
  int T, E, d, nt;
  float* dx;

  __device__ __forceinline__ int rows(int item) const { return min(Cfg::BM, T - (item / nt) * Cfg::BM); }

  __device__ __forceinline__ void setup(int item, DmaLoader<Cfg>& ld, int part) const {
    const int m0 = (item / nt) * Cfg::BM, ni = item % nt;
    const int ce = dma_chunk_elem<Cfg>();
#pragma unroll
    for (int q = 0; q < Cfg::A_DMA / Cfg::DW; ++q)
      ld.a[q] = dl + (int64_t)min(m0 + dma_row<Cfg>(q * Cfg::DW + part), T - 1) * E + ce;
    const int nb = d / kPackTileRows, nk = E / Cfg::BK;
    const int64_t bstride = (int64_t)nk * kPackTileElems;
#pragma unroll
    for (int q = 0; q < Cfg::B_DMA / Cfg::DW; ++q) {
      const int i = q * Cfg::DW + part;
      const int b = min(ni * (Cfg::BN / kPackTileRows) + i / (kPackTileRows / 16), nb - 1);
      ld.b[q] = packed_b_ptr(packed + (int64_t)b * bstride, i % (kPackTileRows / 16), 0);
    }
    ld.b_kstep = kPackTileElems;
  }

  __device__ __forceinline__ void epilogue(int item, Acc<Cfg>& acc) const {
    const int m0 = (item / nt) * Cfg::BM, n0 = (item % nt) * Cfg::BN;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int wm = wave / Cfg::WN, wn = wave % Cfg::WN;
#pragma unroll
    for (int i = 0; i < Cfg::FM; ++i) {
      const int m = m0 + dma_out_row<Cfg>(wm, i, lane);
      if (m0 + frag_row0<Cfg>(wm, i) >= T || m >= T) continue;
#pragma unroll
      for (int j = 0; j < Cfg::FN; ++j) {
        if (n0 + wn * (Cfg::BN / Cfg::WN) + j * 16 >= d) continue;
        const int n = n0 + dma_out_col<Cfg>(wn, j, lane);
        float4* p = reinterpret_cast<float4*>(dx + (int64_t)m * d + n);
        float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
        if constexpr (!STORE) v = *p;
        v.x += acc.v[i][j][0];
        v.y += acc.v[i][j][1];
        v.z += acc.v[i][j][2];
        v.w += acc.v[i][j][3];
        *p = v;
      }
    }
  }
};
template <class Cfg, bool STORE>
__global__ __launch_bounds__(Cfg::THREADS, Cfg::WAVES_PER_SIMD) void router_bwd_dma(RouterBwdPackedProb<Cfg, STORE> pb,
                                                                                   int items) {
  persistent_gemm_dma<Cfg>(pb, items, pb.E / Cfg::BK);
}

hipError_t launch_router_bwd_packed(const Ctx& c, const moe_shape_t& s, const bf16_t* dl, const bf16_t* wr_packed,
                                    float* dx, bool store) {
  using Cfg = GemmCfgWide;
  const int nt = (s.d + Cfg::BN - 1) / Cfg::BN;
  const int items = ((s.T + Cfg::BM - 1) / Cfg::BM) * nt;
  const int grid = std::min(((items + 7) / 8) * 8, c.num_cus);
  if (store) {
    RouterBwdPackedProb<Cfg, true> pb{dl, wr_packed, s.T, s.E, s.d, nt, dx};
    hipLaunchKernelGGL((router_bwd_dma<Cfg, true>), dim3(grid), dim3(Cfg::THREADS), 0, c.stream, pb, items);
  } else {
    RouterBwdPackedProb<Cfg, false> pb{dl, wr_packed, s.T, s.E, s.d, nt, dx};
    hipLaunchKernelGGL((router_bwd_dma<Cfg, false>), dim3(grid), dim3(Cfg::THREADS), 0, c.stream, pb, items);
  }
  return hipGetLastError();
}

hipError_t launch_pack_router_bwd(const Ctx& c, const moe_shape_t& s, const void* w_router, void* wr_packed) {
  // W_r^T: rows n < d, K = E, element (n, e) = w_router[e][n]
  hipLaunchKernelGGL(pack_trans, dim3(c.num_cus * 8), dim3(256), 0, c.stream, (const bf16_t*)w_router,
                     (const bf16_t*)w_router, s.E, 1, s.d, s.E, (int64_t)s.d, (int64_t)0, (u32x4*)wr_packed);
  return hipGetLastError();
}

hipError_t launch_pack_bwd(const Ctx& c, const moe_shape_t& s, const void* w_gate, const void* w_up,
                           const void* w_down, void* dgu_packed, void* dx_packed) {
  const int L = s.e_hi - s.e_lo;
  const int grid = c.num_cus * 8;
  if (dgu_packed) {
    // W_d^T: rows n < f, K = d, element (n, k) = w_down[le][k][n]
    hipLaunchKernelGGL(pack_trans, dim3(grid), dim3(256), 0, c.stream, (const bf16_t*)w_down,
                       (const bf16_t*)w_down, s.d, L, s.f, s.d, (int64_t)s.f, (int64_t)s.d * s.f,
                       (u32x4*)dgu_packed);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  if (dx_packed)
    // [W_g; W_u]^T: rows n < d, K = 2f, element (n, k) = w_gate / w_up[le][k][n]
    hipLaunchKernelGGL(pack_trans, dim3(grid), dim3(256), 0, c.stream, (const bf16_t*)w_gate,
                       (const bf16_t*)w_up, s.f, L, s.d, 2 * s.f, (int64_t)s.d, (int64_t)s.f * s.d,
                       (u32x4*)dx_packed);
  return hipGetLastError();
}

// ------------------------------------------------------------ packing ---
//
// Frozen weights rearranged once so that every weight tile the grouped GEMMs
// stream is one contiguous 8 KB block holding the exact LDS image of a B
// stage (128 rows x 32 K values, 16-byte chunk c of row r at slot
// c ^ chunk_key(r)). gate/up: tile (le, n block of 64 FFN columns, K step)
// with rows interleaving 16 W_g rows and the same 16 W_u rows; down: tile
// (le, n block of 128 output columns, K step).
__global__ __launch_bounds__(256) void pack_gate_up(const bf16_t* __restrict__ w_gate,
                                                    const bf16_t* __restrict__ w_up, int L, int d,
                                                    int f, u32x4* __restrict__ out) {
  const int nk = d / 32, nt = f / 64;
  const int64_t total = (int64_t)L * nt * nk * 512;
  for (int64_t id = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; id < total;
       id += (int64_t)gridDim.x * blockDim.x) {
    const int slot = (int)(id & 3), jb = (int)((id >> 2) & 127);
    const int64_t tile = id >> 9;
    const int kt = (int)(tile % nk);
    const int64_t rest = tile / nk;
    const int ni = (int)(rest % nt), le = (int)(rest / nt);
    const int frag = jb >> 4;
    const int fcol = ni * 64 + (frag >> 1) * 16 + (jb & 15);
    const int c = slot ^ chunk_key(jb);
    const bf16_t* src = ((frag & 1) ? w_up : w_gate) + ((int64_t)le * f + fcol) * d + kt * 32 + c * 8;
    out[id] = *reinterpret_cast<const u32x4*>(src);
  }
}

__global__ __launch_bounds__(256) void pack_down(const bf16_t* __restrict__ w_down, int L, int d,
                                                 int f, u32x4* __restrict__ out) {
  const int nk = f / 32, nt = d / 128;
  const int64_t total = (int64_t)L * nt * nk * 512;
  for (int64_t id = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; id < total;
       id += (int64_t)gridDim.x * blockDim.x) {
    const int slot = (int)(id & 3), jb = (int)((id >> 2) & 127);
    const int64_t tile = id >> 9;
    const int kt = (int)(tile % nk);
    const int64_t rest = tile / nk;
    const int ni = (int)(rest % nt), le = (int)(rest / nt);
    const int c = slot ^ chunk_key(jb);
    out[id] = *reinterpret_cast<const u32x4*>(w_down + ((int64_t)le * d + ni * 128 + jb) * f + kt * 32 + c * 8);
  }
}

hipError_t launch_pack(const Ctx& c, const moe_shape_t& s, const void* w_gate, const void* w_up,
                       const void* w_down, void* gu_packed, void* d_packed) {
  const int L = s.e_hi - s.e_lo;
  const int grid = c.num_cus * 8;
  if (gu_packed) {
    hipLaunchKernelGGL(pack_gate_up, dim3(grid), dim3(256), 0, c.stream, (const bf16_t*)w_gate,
                       (const bf16_t*)w_up, L, s.d, s.f, (u32x4*)gu_packed);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  if (d_packed)
    hipLaunchKernelGGL(pack_down, dim3(grid), dim3(256), 0, c.stream, (const bf16_t*)w_down, L, s.d,
                       s.f, (u32x4*)d_packed);
  return hipGetLastError();
}

// ------------------------------------------------------------- fp32 path ---

__global__ __launch_bounds__(256) void gate_up_f32(const float* __restrict__ x_rows,
                                                   const int32_t* __restrict__ row_src,
                                                   const int32_t* __restrict__ offsets, int L,
                                                   int64_t rmax, const float* __restrict__ w_gate,
                                                   const float* __restrict__ w_up, int d, int f,
                                                   float* __restrict__ hbuf,
                                                   float* __restrict__ act_save) {
  const int R = offsets[L];
  for (int64_t id = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; id < (int64_t)R * f;
       id += (int64_t)gridDim.x * blockDim.x) {
    const int p = (int)(id / f), c = (int)(id % f);
    const int le = segment_of(offsets, L, p);
    const float* xr = x_rows + (int64_t)(row_src ? row_src[p] : p) * d;
    const float* wg = w_gate + ((int64_t)le * f + c) * d;
    const float* wu = w_up + ((int64_t)le * f + c) * d;
    float g = 0.f, u = 0.f;
    for (int i = 0; i < d; ++i) {
      g = fmaf(xr[i], wg[i], g);
      u = fmaf(xr[i], wu[i], u);
    }
    const float h = silu_f(g) * u;
    hbuf[(int64_t)p * f + c] = h;
    if (act_save) {
      act_save[(int64_t)p * 3 * f + c] = g;
      act_save[(int64_t)p * 3 * f + f + c] = h;
      act_save[(int64_t)p * 3 * f + 2 * f + c] = u;
    }
  }
}

__global__ __launch_bounds__(256) void down_f32(const float* __restrict__ hbuf,
                                                const int32_t* __restrict__ offsets, int L,
                                                const float* __restrict__ w_down, int d, int f,
                                                float* __restrict__ y_perm) {
  const int R = offsets[L];
  for (int64_t id = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; id < (int64_t)R * d;
       id += (int64_t)gridDim.x * blockDim.x) {
    const int p = (int)(id / d), n = (int)(id % d);
    const int le = segment_of(offsets, L, p);
    const float* hr = hbuf + (int64_t)p * f;
    const float* wd = w_down + ((int64_t)le * d + n) * f;
    float o = 0.f;
    for (int c = 0; c < f; ++c) o = fmaf(hr[c], wd[c], o);
    y_perm[id] = o;
  }
}

// ------------------------------------------------------------- launchers ---

hipError_t launch_row_tiles(const Ctx& c, const int32_t* offsets, int L, int max_tiles,
                            int32_t* tiles, int bm) {
  TimedLaunch tl(MOE_K_TILES, c.stream);
  hipLaunchKernelGGL(build_row_tiles, dim3(1), dim3(1024), 0, c.stream, offsets, L, bm,
                     max_tiles, tiles);
  return hipGetLastError();
}

template <class Cfg>
hipError_t launch_grouped_bf16(const Ctx& c, const moe_shape_t& s, const Workspace& ws, const bf16_t* xr,
                               const int32_t* row_src, const int32_t* offsets, const void* gu_packed,
                               const void* d_packed, const void* w_gate, const void* w_up,
                               const void* w_down, const LoraArgs* lora, void* act_save, void* y_perm,
                               int max_tiles, int lora_mode);

hipError_t launch_expert_gemm(const Ctx& c, const moe_shape_t& s, const Workspace& ws,
                              const void* x_rows, const int32_t* row_src, const int32_t* offsets,
                              const void* gu_packed, const void* d_packed, const void* w_gate,
                              const void* w_up, const void* w_down, const LoraArgs* lora,
                              void* act_save, void* y_perm) {
  const int L = s.e_hi - s.e_lo;
  const int64_t rmax = max_rows(s);
  hipError_t err;
  if (s.dtype != MOE_BF16) {
    const int grid = c.num_cus * 4;
    {
      TimedLaunch tl(MOE_K_GATE_UP, c.stream);
      hipLaunchKernelGGL(gate_up_f32, dim3(grid), dim3(256), 0, c.stream, (const float*)x_rows,
                         row_src, offsets, L, rmax, (const float*)w_gate, (const float*)w_up, s.d, s.f,
                         (float*)ws.hbuf, (float*)act_save);
    }
    if ((err = hipGetLastError()) != hipSuccess) return err;
    TimedLaunch tl(MOE_K_DOWN, c.stream);
    hipLaunchKernelGGL(down_f32, dim3(grid), dim3(256), 0, c.stream, (const float*)ws.hbuf, offsets,
                       L, (const float*)w_down, s.d, s.f, (float*)y_perm);
    return hipGetLastError();
  }
  const int max_tiles = gemm_max_tiles(s);
  const bf16_t* xr = (const bf16_t*)x_rows;
  // adapter terms: through the matrix cores as one extra K step at r = 16
  // (the projection's matrix-core path applies: d, f % 32 == 0), else in
  // the epilogues
  const int lora_mode = !lora ? 0 : (lora->r == 16 && s.d % 32 == 0 && s.f % 32 == 0 && ws.zx) ? 2 : 1;
  // fp32 Z_u: kept for the backward in the caller's z_save, else in ws
  // (needed there only by the epilogue form)
  float* zu = lora && lora->z_save ? lora->z_save : ws.zu;
  if (lora) {
    err = lora_mode == 2
              ? launch_lora_rowproj<bf16_t>(c, L, offsets, rmax, xr, s.d, row_src, nullptr, s.d, lora->a_up, true,
                                            lora->r, lora->z_save ? zu : nullptr, nullptr, ws.zx, lora->scale)
              : launch_lora_rowproj<bf16_t>(c, L, offsets, rmax, xr, s.d, row_src, nullptr, s.d, lora->a_up, true,
                                            lora->r, zu);
    if (err != hipSuccess) return err;
  }
  if (gemm_tile_rows(s) == GemmCfgTall::BM)
    return launch_grouped_bf16<GemmCfgTall>(c, s, ws, xr, row_src, offsets, gu_packed, d_packed, w_gate,
                                            w_up, w_down, lora, act_save, y_perm, max_tiles, lora_mode);
  return launch_grouped_bf16<GemmCfg>(c, s, ws, xr, row_src, offsets, gu_packed, d_packed, w_gate, w_up,
                                      w_down, lora, act_save, y_perm, max_tiles, lora_mode);
}

template <class Cfg>
hipError_t launch_grouped_bf16(const Ctx& c, const moe_shape_t& s, const Workspace& ws, const bf16_t* xr,
                               const int32_t* row_src, const int32_t* offsets, const void* gu_packed,
                               const void* d_packed, const void* w_gate, const void* w_up,
                               const void* w_down, const LoraArgs* lora, void* act_save, void* y_perm,
                               int max_tiles, int lora_mode) {
  hipError_t err;
  const int L = s.e_hi - s.e_lo;
  const int64_t rmax = max_rows(s);
  const int grid = c.num_cus;  // one workgroup per CU (see mfma_tile.h)
  float* zu = lora && lora->z_save ? lora->z_save : ws.zu;
  float* zd = lora && lora->z_save ? lora->z_save + rmax * lora->r : ws.zd;
  if ((err = launch_row_tiles(c, offsets, L, max_tiles, ws.gemm_tiles, Cfg::BM)) != hipSuccess) return err;
  // Weight tiles are fetched with the streaming hint when an expert's rows are
  // expected to fit one row tile (the capacity, or the even share T k / E
  // with 5% to spare); where experts span several row tiles that share each
  // weight tile, the hint measured slower (capacity 183 on 128-row tiles).
  const int64_t even = (int64_t)s.T * s.k / s.E;
  const bool stream_b = s.capacity > 0 ? s.capacity <= Cfg::BM : even * 20 <= (int64_t)Cfg::BM * 19;
  auto gu_launch = [&](auto mode) {
    constexpr int LO = decltype(mode)::value;
    using P = GateUpProb<Cfg, LO>;
    P pb{xr, row_src, offsets, ws.gemm_tiles, (const bf16_t*)w_gate,
         (const bf16_t*)w_up, (const bf16_t*)gu_packed, s.d, s.f,
         (s.f + P::HALF - 1) / P::HALF, s.e_hi - s.e_lo,
         lora ? zu : nullptr, lora ? lora->b_up : nullptr, lora ? lora->r : 0,
         lora ? lora->scale : 0.f, (bf16_t*)ws.hbuf, (bf16_t*)act_save};
    pb.zx = ws.zx;
    pb.stream_b = stream_b;
    TimedLaunch tl(MOE_K_GATE_UP, c.stream);
    hipLaunchKernelGGL((gate_up_bf16<Cfg, LO>), dim3(grid), dim3(Cfg::THREADS), 0, c.stream, pb, max_tiles);
    return hipGetLastError();
  };
  err = lora_mode == 2   ? gu_launch(std::integral_constant<int, 2>{})
        : lora_mode == 1 ? gu_launch(std::integral_constant<int, 1>{})
                         : gu_launch(std::integral_constant<int, 0>{});
  if (err != hipSuccess) return err;
  if (lora) {
    err = lora_mode == 2 ? launch_lora_rowproj<bf16_t>(c, L, offsets, rmax, (const bf16_t*)ws.hbuf, s.f, nullptr,
                                                       nullptr, s.f, lora->a_down, true, lora->r,
                                                       lora->z_save ? zd : nullptr, nullptr, ws.zx, lora->scale)
                         : launch_lora_rowproj<bf16_t>(c, L, offsets, rmax, (const bf16_t*)ws.hbuf, s.f, nullptr,
                                                       nullptr, s.f, lora->a_down, true, lora->r, zd);
    if (err != hipSuccess) return err;
  }
  auto dn_launch = [&](auto mode) {
    constexpr int LO = decltype(mode)::value;
    DownProb<Cfg, LO> pb{(const bf16_t*)ws.hbuf, offsets, ws.gemm_tiles, (const bf16_t*)w_down,
                         (const bf16_t*)d_packed, s.d, s.f,
                         (s.d + Cfg::BN - 1) / Cfg::BN, lora ? zd : nullptr,
                         lora ? lora->b_down : nullptr, lora ? lora->r : 0, lora ? lora->scale : 0.f,
                         (bf16_t*)y_perm};
    pb.zx = ws.zx;
    pb.stream_b = stream_b;
    TimedLaunch tl(MOE_K_DOWN, c.stream);
    hipLaunchKernelGGL((down_bf16<Cfg, LO>), dim3(grid), dim3(Cfg::THREADS), 0, c.stream, pb, max_tiles);
    return hipGetLastError();
  };
  return lora_mode == 2   ? dn_launch(std::integral_constant<int, 2>{})
         : lora_mode == 1 ? dn_launch(std::integral_constant<int, 1>{})
                          : dn_launch(std::integral_constant<int, 0>{});
}

}  // namespace moe
