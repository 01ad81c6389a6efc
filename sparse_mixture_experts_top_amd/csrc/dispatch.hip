// Dispatch: group the T*k (token, slot) assignments by local expert.
//
// "Trillion-Parameter MoE Model Training Adaptation: Full-Stack Optimization
// Practices", §3 and §4.3: tokens are permuted by the routing result before
// the grouped GEMM; "Adapting Ultra-Large MoE Models: Engineering Practices and
// Optimization Pathways", §3.3: per-expert capacity with overflow dropping.
//
// Rows are ordered by (local expert, token). No step depends on the order in
// which threads run: per-tile histograms use integer atomics (order-free), the
// rank of a token inside its tile comes from a per-expert token bitmask and a
// popcount, and the capacity threshold comes from an exact radix select.
//
//   K3 hist      per 256-token tile: LDS histogram over E -> tile_counts
//   K4 scan      one block: per-expert running sum over tiles -> tile_base,
//                counts; kept = min(count, C) -> offsets (exclusive scan)
//   K6 scatter   per tile: position of (t, j) inside its expert =
//                tile_base + number of earlier tokens of the tile with that
//                expert; writes slot / row_src / row_gate, or, for an expert
//                over capacity, a candidate (gate bits, assignment)
//   K5 capacity  per over-capacity expert: C-th largest (gate, -token) key by
//                radix select, then kept candidates in token order -> rows
//   K7 gather    x_perm[p] = x[row_src[p]] with 16-byte loads and stores
//                (optional: the grouped GEMM can read x through row_src)
#include "common.h"

namespace moe {

__global__ __launch_bounds__(256) void dispatch_hist(const int32_t* __restrict__ idx, int T, int k,
                                                     int E, int32_t* __restrict__ tile_counts) {
  __shared__ int32_t cnt[1024];
  for (int e = threadIdx.x; e < E; e += 256) cnt[e] = 0;
  __syncthreads();
  const int t0 = blockIdx.x * kTokTile;
  const int n = min(kTokTile, T - t0) * k;
  const int32_t* base = idx + (int64_t)t0 * k;
  for (int a = threadIdx.x; a < n; a += 256) atomicAdd(&cnt[base[a]], 1);
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += 256) tile_counts[(int64_t)blockIdx.x * E + e] = cnt[e];
}

// Exclusive scan of v over the block (blockDim.x == 1024); returns the
// exclusive prefix for this thread and writes the total to *total.
__device__ int block_exclusive_scan_1024(int v, int* total) {
  __shared__ int wsum[16];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int incl = v;
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) {
    const int o = __shfl_up(incl, m, kWave);
    if (lane >= m) incl += o;
  }
  if (lane == 63) wsum[wave] = incl;
  __syncthreads();
  int before = 0, all = 0;
  for (int w = 0; w < 16; ++w) {
    const int sw = wsum[w];
    if (w < wave) before += sw;
    all += sw;
  }
  __syncthreads();
  *total = all;
  return before + incl - v;
}

__global__ __launch_bounds__(1024) void dispatch_scan(const int32_t* __restrict__ tile_counts,
                                                      int ntiles, int E, int e_lo, int L,
                                                      int capacity,
                                                      int32_t* __restrict__ tile_base,
                                                      int32_t* __restrict__ counts,
                                                      int32_t* __restrict__ offsets,
                                                      int32_t* __restrict__ cseg,
                                                      int32_t* __restrict__ dropped) {
  const int e = threadIdx.x;
  int run = 0;
  if (e < E) {
    for (int tl = 0; tl < ntiles; ++tl) {
      tile_base[(int64_t)tl * E + e] = run;
      run += tile_counts[(int64_t)tl * E + e];
    }
    counts[e] = run;
  }
  const int le = e - e_lo;
  const bool local = e < E && le >= 0 && le < L;
  const int cnt = local ? run : 0;
  const int kept = (capacity > 0 && cnt > capacity) ? capacity : cnt;
  const int over = (capacity > 0 && cnt > capacity) ? cnt : 0;
  int tot_kept, tot_over;
  const int off = block_exclusive_scan_1024(kept, &tot_kept);
  const int coff = block_exclusive_scan_1024(over, &tot_over);
  if (local) {
    offsets[le] = off;
    cseg[le] = coff;
  }
  if (e == 0) {
    offsets[L] = tot_kept;
    cseg[L] = tot_over;
  }
  // dropped = sum over local experts of (cnt - kept)
  int tot_drop;
  block_exclusive_scan_1024(cnt - kept, &tot_drop);
  if (e == 0 && dropped) *dropped = tot_drop;
}

__global__ __launch_bounds__(256) void dispatch_scatter(
    const int32_t* __restrict__ idx, const float* __restrict__ gate, int T, int k, int E, int e_lo,
    int L, int capacity, const int32_t* __restrict__ tile_base, const int32_t* __restrict__ counts,
    const int32_t* __restrict__ offsets, const int32_t* __restrict__ cseg,
    int32_t* __restrict__ slot, int32_t* __restrict__ row_src, float* __restrict__ row_gate,
    uint32_t* __restrict__ cand_key, int32_t* __restrict__ cand_idx) {
  constexpr int W = kTokTile / 32;  // bitmask words per expert
  __shared__ uint32_t mask[1024 * W];
  for (int i = threadIdx.x; i < E * W; i += 256) mask[i] = 0u;
  __syncthreads();
  const int tl = blockIdx.x;
  const int lt = threadIdx.x;  // token within the tile
  const int t = tl * kTokTile + lt;
  const bool valid = t < T;
  if (valid)
    for (int j = 0; j < k; ++j) atomicOr(&mask[idx[(int64_t)t * k + j] * W + (lt >> 5)], 1u << (lt & 31));
  __syncthreads();
  if (!valid) return;
  for (int j = 0; j < k; ++j) {
    const int64_t a = (int64_t)t * k + j;
    const int e = idx[a];
    const int le = e - e_lo;
    if (le < 0 || le >= L) {
      slot[a] = -1;
      continue;
    }
    int rank = 0;
    const uint32_t* mw = &mask[e * W];
    for (int w = 0; w < (lt >> 5); ++w) rank += __popc(mw[w]);
    rank += __popc(mw[lt >> 5] & ((1u << (lt & 31)) - 1u));
    const int pos = tile_base[(int64_t)tl * E + e] + rank;
    const float g = gate[a];
    if (capacity > 0 && counts[e] > capacity) {
      const int ci = cseg[le] + pos;
      cand_key[ci] = __float_as_uint(g);
      cand_idx[ci] = (int32_t)a;
    } else {
      const int row = offsets[le] + pos;
      slot[a] = row;
      row_src[row] = t;
      row_gate[row] = g;
    }
  }
}

// One block per local expert; experts within capacity return at once.
// Key of a candidate: gate bits (positive floats order like their bits) in
// the high word, ~token in the low word, so the largest key is the largest
// gate and, among equal gates, the lowest token. Keys are unique.
__global__ __launch_bounds__(256) void dispatch_capacity(
    int k, int e_lo, int L, int capacity, const int32_t* __restrict__ counts,
    const int32_t* __restrict__ offsets, const int32_t* __restrict__ cseg,
    const uint32_t* __restrict__ cand_key, const int32_t* __restrict__ cand_idx,
    int32_t* __restrict__ slot, int32_t* __restrict__ row_src, float* __restrict__ row_gate) {
  __shared__ int hist[256];
  __shared__ uint64_t s_prefix;
  __shared__ int s_need;
  __shared__ int wsum[4];
  const int le = blockIdx.x;
  const int n = counts[e_lo + le];
  if (n <= capacity) return;
  const uint32_t* ck = cand_key + cseg[le];
  const int32_t* ci = cand_idx + cseg[le];
  auto key_of = [&](int i) -> uint64_t {
    const uint32_t tok = (uint32_t)(ci[i] / k);
    return ((uint64_t)ck[i] << 32) | (uint64_t)(0xffffffffu - tok);
  };
  if (threadIdx.x == 0) {
    s_prefix = 0;
    s_need = capacity;
  }
  uint64_t pmask = 0;
  for (int shift = 56; shift >= 0; shift -= 8) {
    hist[threadIdx.x] = 0;
    __syncthreads();
    const uint64_t prefix = s_prefix;
    for (int i = threadIdx.x; i < n; i += 256) {
      const uint64_t key = key_of(i);
      if ((key & pmask) == prefix) atomicAdd(&hist[(key >> shift) & 255], 1);
    }
    __syncthreads();
    if (threadIdx.x == 0) {
      int need = s_need, above = 0, b = 255;
      for (; b > 0; --b) {
        if (above + hist[b] >= need) break;
        above += hist[b];
      }
      s_prefix = prefix | ((uint64_t)b << shift);
      s_need = need - above;
    }
    pmask |= (uint64_t)255 << shift;
    __syncthreads();
  }
  const uint64_t thr = s_prefix;  // the capacity-th largest key
  // Kept candidates in token order get consecutive rows.
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int carry = 0;
  for (int base = 0; base < n; base += 256) {
    const int i = base + threadIdx.x;
    const bool in = i < n;
    const bool keep = in && key_of(i) >= thr;
    const unsigned long long bal = __ballot(keep);
    const int before_in_wave = __popcll(bal & ((1ull << lane) - 1ull));
    if (lane == 0) wsum[wave] = __popcll(bal);
    __syncthreads();
    int before = carry;
    for (int w = 0; w < wave; ++w) before += wsum[w];
    const int chunk_total = wsum[0] + wsum[1] + wsum[2] + wsum[3];
    if (in) {
      const int a = ci[i];
      if (keep) {
        const int row = offsets[le] + before + before_in_wave;
        slot[a] = row;
        row_src[row] = a / k;
        row_gate[row] = __uint_as_float(ck[i]);
      } else {
        slot[a] = -1;
      }
    }
    carry += chunk_total;
    __syncthreads();
  }
}

// x_perm[p, :] = x[row_src[p], :] for p < R = offsets[L]; one row per
// block iteration, 16-byte vectors.
__global__ __launch_bounds__(256) void dispatch_gather(const uint4* __restrict__ x,
                                                       const int32_t* __restrict__ row_src,
                                                       const int32_t* __restrict__ offsets, int L,
                                                       int vec_per_row, uint4* __restrict__ x_perm) {
  const int R = offsets[L];
  for (int p = blockIdx.x; p < R; p += gridDim.x) {
    const uint4* src = x + (int64_t)row_src[p] * vec_per_row;
    uint4* dst = x_perm + (int64_t)p * vec_per_row;
    for (int v = threadIdx.x; v < vec_per_row; v += 256) dst[v] = src[v];
  }
}

// Same for rows whose byte size is not a multiple of 16 (fp32, d % 4 != 0).
__global__ __launch_bounds__(256) void dispatch_gather_f32(const float* __restrict__ x,
                                                           const int32_t* __restrict__ row_src,
                                                           const int32_t* __restrict__ offsets,
                                                           int L, int d, float* __restrict__ x_perm) {
  const int R = offsets[L];
  for (int p = blockIdx.x; p < R; p += gridDim.x) {
    const float* src = x + (int64_t)row_src[p] * d;
    float* dst = x_perm + (int64_t)p * d;
    for (int v = threadIdx.x; v < d; v += 256) dst[v] = src[v];
  }
}

hipError_t launch_dispatch(const Ctx& c, const moe_shape_t& s, const Workspace& ws,
                           const int32_t* idx, const float* gate, const void* x, int32_t* counts,
                           int32_t* offsets, int32_t* slot, int32_t* row_src, float* row_gate,
                           void* x_perm, int32_t* dropped) {
  const int ntiles = (s.T + kTokTile - 1) / kTokTile;
  const int L = s.e_hi - s.e_lo;
  hipError_t err;
  if (ntiles > 0) {
    TimedLaunch tl(MOE_K_HIST, c.stream);
    hipLaunchKernelGGL(dispatch_hist, dim3(ntiles), dim3(256), 0, c.stream, idx, s.T, s.k, s.E,
                       ws.tile_counts);
  }
  if ((err = hipGetLastError()) != hipSuccess) return err;
  {
    TimedLaunch tl(MOE_K_SCAN, c.stream);
    hipLaunchKernelGGL(dispatch_scan, dim3(1), dim3(1024), 0, c.stream, ws.tile_counts, ntiles,
                       s.E, s.e_lo, L, s.capacity, ws.tile_base, counts, offsets, ws.cseg, dropped);
  }
  if ((err = hipGetLastError()) != hipSuccess) return err;
  if (ntiles > 0) {
    TimedLaunch tl(MOE_K_SCATTER, c.stream);
    hipLaunchKernelGGL(dispatch_scatter, dim3(ntiles), dim3(kTokTile), 0, c.stream, idx, gate, s.T,
                       s.k, s.E, s.e_lo, L, s.capacity, ws.tile_base, counts, offsets, ws.cseg,
                       slot, row_src, row_gate, ws.cand_key, ws.cand_idx);
  }
  if ((err = hipGetLastError()) != hipSuccess) return err;
  if (s.capacity > 0) {
    TimedLaunch tl(MOE_K_CAPACITY, c.stream);
    hipLaunchKernelGGL(dispatch_capacity, dim3(L), dim3(256), 0, c.stream, s.k, s.e_lo, L,
                       s.capacity, counts, offsets, ws.cseg, ws.cand_key, ws.cand_idx, slot,
                       row_src, row_gate);
    if ((err = hipGetLastError()) != hipSuccess) return err;
  }
  if (!x_perm) return hipSuccess;  // the grouped GEMM gathers through row_src itself
  const int64_t rmax = max_rows(s);
  const int grid = (int)std::min<int64_t>(rmax > 0 ? rmax : 1, (int64_t)c.num_cus * 8);
  const size_t row_bytes = (size_t)s.d * (s.dtype == MOE_BF16 ? 2 : 4);
  TimedLaunch tl(MOE_K_GATHER, c.stream);
  if (row_bytes % 16 == 0) {
    hipLaunchKernelGGL(dispatch_gather, dim3(grid), dim3(256), 0, c.stream, (const uint4*)x,
                       row_src, offsets, L, (int)(row_bytes / 16), (uint4*)x_perm);
  } else {
    hipLaunchKernelGGL(dispatch_gather_f32, dim3(grid), dim3(256), 0, c.stream, (const float*)x,
                       row_src, offsets, L, s.d, (float*)x_perm);
  }
  return hipGetLastError();
}

}  // namespace moe
