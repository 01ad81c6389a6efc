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
// Token tiles are 32 tokens wide, so a tile's tokens routed to one expert
// form a single 32-bit mask; T = 4096 gives 128 tiles, enough workgroups to
// spread over the GPU.
//
//   K3 hist       per tile: LDS histogram over E -> tile_counts (or the
//                 top-k kernel adds its selections into them, when routing
//                 and dispatch run as one call)
//   K4 tile scan  per expert (16 per workgroup, 16 threads splitting the
//                 tiles): running sum over tiles -> tile_base, counts
//   K6 scatter    per tile: each workgroup first scans the per-expert kept
//                 counts, kept = min(count, C), over the experts (workgroup
//                 0 also writes offsets / dropped); then the position of
//                 (t, j) inside its expert = tile_base + number of earlier
//                 tokens of the tile with that expert; writes slot / row_src
//                 / row_gate, or, for an expert over capacity, a candidate
//                 (gate bits, assignment)
//   K5 capacity   per over-capacity expert: C-th largest gate (bitwise
//                 search over keys held in registers, or radix select for
//                 more than 8192 candidates), ties to the lower token, then
//                 kept candidates in token order -> rows
//   K7 gather     x_perm[p] = x[row_src[p]] with 16-byte loads and stores
//                 (optional: the grouped GEMM can read x through row_src)
#include "common.h"

namespace moe {

static_assert(kTokTile == 32, "one 32-bit token mask per (tile, expert)");

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

// tile_base[tl, e] = sum of tile_counts[tl' < tl, e]; counts[e] = the total.
// Workgroup b takes experts 16b .. 16b+15; thread (part, ex) sums one
// sixteenth of the tiles, the parts are combined in LDS, then each thread
// writes the running sums of its part.
constexpr int kScanParts = 16;
__global__ __launch_bounds__(256) void dispatch_tile_scan(const int32_t* __restrict__ tile_counts,
                                                          int ntiles, int E,
                                                          int32_t* __restrict__ tile_base,
                                                          int32_t* __restrict__ counts) {
  constexpr int EX = 256 / kScanParts;
  __shared__ int psum[kScanParts][EX];
  const int ex = threadIdx.x % EX, part = threadIdx.x / EX;
  const int e = blockIdx.x * EX + ex;
  const int per = (ntiles + kScanParts - 1) / kScanParts;
  const int lo = min(part * per, ntiles), hi = min(lo + per, ntiles);
  int sum = 0;
  if (e < E) {
#pragma unroll 8
    for (int tl = lo; tl < hi; ++tl) sum += tile_counts[(int64_t)tl * E + e];
  }
  psum[part][ex] = sum;
  __syncthreads();
  int run = 0;
  for (int p = 0; p < part; ++p) run += psum[p][ex];
  if (e < E) {
#pragma unroll 8
    for (int tl = lo; tl < hi; ++tl) {
      const int v = tile_counts[(int64_t)tl * E + e];
      tile_base[(int64_t)tl * E + e] = run;
      run += v;
    }
    if (part == kScanParts - 1) counts[e] = run;
  }
}

// Exclusive scans over the experts (E <= 1024, 4 per thread of a 256-thread
// workgroup) of kept = min(local count, C) and over = local count if above C
// (else 0): s_off[e], s_cs[e] (non-local experts contribute 0, so the scans
// over all experts equal the scans over local experts in order). Returns
// (total kept, total over, total dropped) through the last three arguments.
__device__ void expert_scans(const int32_t* __restrict__ counts, int E, int e_lo, int L,
                             int capacity, int* s_off, int* s_cs, int* tot_kept, int* tot_over,
                             int* tot_drop) {
  __shared__ int wk[4], wo[4], wd[4];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int kv[4], ov[4], ks = 0, os = 0, ds = 0;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int e = 4 * threadIdx.x + q;
    const int le = e - e_lo;
    const int c = (e < E && le >= 0 && le < L) ? counts[e] : 0;
    const bool over = capacity > 0 && c > capacity;
    kv[q] = over ? capacity : c;
    ov[q] = over ? c : 0;
    ks += kv[q];
    os += ov[q];
    ds += c - kv[q];
  }
  int ki = ks, oi = os;
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) {
    const int a = __shfl_up(ki, m, kWave), b = __shfl_up(oi, m, kWave);
    if (lane >= m) {
      ki += a;
      oi += b;
    }
  }
  int dsum = ds;
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) dsum += __shfl_xor(dsum, m, kWave);
  if (lane == 63) {
    wk[wave] = ki;
    wo[wave] = oi;
  }
  if (lane == 0) wd[wave] = dsum;
  __syncthreads();
  int kb = 0, ob = 0;
  for (int w = 0; w < wave; ++w) {
    kb += wk[w];
    ob += wo[w];
  }
  kb += ki - ks;
  ob += oi - os;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int e = 4 * threadIdx.x + q;
    if (e < E) {
      s_off[e] = kb;
      s_cs[e] = ob;
    }
    kb += kv[q];
    ob += ov[q];
  }
  *tot_kept = wk[0] + wk[1] + wk[2] + wk[3];
  *tot_over = wo[0] + wo[1] + wo[2] + wo[3];
  *tot_drop = wd[0] + wd[1] + wd[2] + wd[3];
  __syncthreads();
}

// 256 threads: thread (token lt = tid / 8, jg = tid % 8) handles the
// assignments j = jg, jg + 8, ... of token tile * 32 + lt.
__global__ __launch_bounds__(256) void dispatch_scatter(
    const int32_t* __restrict__ idx, const float* __restrict__ gate, int T, int k, int E, int e_lo,
    int L, int capacity, const int32_t* __restrict__ tile_base, const int32_t* __restrict__ counts,
    int32_t* __restrict__ offsets, int32_t* __restrict__ cseg, int32_t* __restrict__ dropped,
    int32_t* __restrict__ slot, int32_t* __restrict__ row_src, float* __restrict__ row_gate,
    uint32_t* __restrict__ cand_key, int32_t* __restrict__ cand_idx) {
  __shared__ uint32_t mask[1024];
  __shared__ int s_off[1024], s_cs[1024];
  for (int i = threadIdx.x; i < E; i += 256) mask[i] = 0u;
  int tot_kept, tot_over, tot_drop;
  expert_scans(counts, E, e_lo, L, capacity, s_off, s_cs, &tot_kept, &tot_over, &tot_drop);
  if (blockIdx.x == 0) {
    for (int le = threadIdx.x; le < L; le += 256) {
      offsets[le] = s_off[e_lo + le];
      cseg[le] = s_cs[e_lo + le];
    }
    if (threadIdx.x == 0) {
      offsets[L] = tot_kept;
      cseg[L] = tot_over;
      if (dropped) *dropped = tot_drop;
    }
  }
  const int tl = blockIdx.x;
  const int lt = threadIdx.x >> 3, jg = threadIdx.x & 7;
  const int t = tl * kTokTile + lt;
  const bool valid = t < T;
  if (valid)
    for (int j = jg; j < k; j += 8) atomicOr(&mask[idx[(int64_t)t * k + j]], 1u << lt);
  __syncthreads();
  if (!valid) return;
  const uint32_t below = (1u << lt) - 1u;
  for (int j = jg; j < k; j += 8) {
    const int64_t a = (int64_t)t * k + j;
    const int e = idx[a];
    const int le = e - e_lo;
    if (le < 0 || le >= L) {
      slot[a] = -1;
      continue;
    }
    const int pos = tile_base[(int64_t)tl * E + e] + __popc(mask[e] & below);
    const float g = gate[a];
    if (capacity > 0 && counts[e] > capacity) {
      const int ci = s_cs[e] + pos;
      cand_key[ci] = __float_as_uint(g);
      cand_idx[ci] = (int32_t)a;
    } else {
      const int row = s_off[e] + pos;
      slot[a] = row;
      row_src[row] = t;
      row_gate[row] = g;
    }
  }
}

// Exclusive scan of v over a workgroup of NW waves; *total gets the sum.
template <int NW>
__device__ int block_exclusive_scan(int v, int* total) {
  __shared__ int wsum[NW];
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
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    before += w < wave ? wsum[w] : 0;
    all += wsum[w];
  }
  *total = all;
  __syncthreads();
  return before + incl - v;
}

// One workgroup per local expert; experts within capacity return at once.
// The candidates of an over-capacity expert sit in token order (cseg[le]
// onwards, written by the scatter). The kept set is the C assignments with
// the largest gate, equal gates going to the lower token:
//   1. g* = the C-th largest gate: radix select over the gate's 32 bits (gates
//      are positive, so their bit patterns order like the values), four
//      passes of 8 bits, each an LDS histogram and a suffix scan of its bins;
//      `need` ends as the number of candidates equal to g* that are kept.
//   2. keep = gate > g*, or gate == g* and fewer than `need` earlier
//      candidates (lower tokens) equal g*.
//   3. kept candidates get consecutive rows in token order: per (round of
//      1024 consecutive candidates, wave) ballot counts of the equal and then
//      of the kept candidates, each turned into candidate-order offsets by one
//      workgroup scan, a chunk of kCapRounds rounds at a time.
// Up to kCapLds candidates are held in registers (capacity_core_regs, which
// finds g* by a bitwise search instead of the histograms); larger experts
// read them from global memory in every pass.
constexpr int kCapThreads = 1024;
constexpr int kCapWaves = kCapThreads / 64;
constexpr int kCapLds = 8192;
constexpr int kCapRounds = 16;  // rounds of 1024 per chunk, (round, wave) counts in LDS
static_assert(kCapLds % kCapThreads == 0, "LDS staging in whole rounds");

struct CapShared {
  int hist[256];
  int cnt[kCapWaves * kCapRounds], pre[kCapWaves * kCapRounds], kpre[kCapWaves * kCapRounds];
  uint32_t prefix;
  int need;
  int eq_total, kept_total;  // running totals over the chunks done
};

// The selection and compaction for one expert; key_at(i) / idx_at(i) read
// candidate i (from LDS or global memory: one instantiation each, so every
// access has its own address space).
template <class Key, class Idx>
__device__ __forceinline__ void capacity_core(CapShared& sh, Key key_at, Idx idx_at, int n, int k,
                                              int capacity, int base, int32_t* __restrict__ slot,
                                              int32_t* __restrict__ row_src,
                                              float* __restrict__ row_gate) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (tid == 0) {
    sh.prefix = 0u;
    sh.need = capacity;
    sh.eq_total = 0;
    sh.kept_total = 0;
  }
  uint32_t pmask = 0u;
  for (int shift = 24; shift >= 0; shift -= 8) {
    if (tid < 256) sh.hist[tid] = 0;
    __syncthreads();
    const uint32_t prefix = sh.prefix;
    for (int i = tid; i < n; i += kCapThreads) {
      const uint32_t key = key_at(i);
      bool act = (key & pmask) == prefix;
      const int bin = (int)((key >> shift) & 255u);
      // gates crowd into few bins (the high bytes of values in (0, 1]): the
      // lanes sharing the first active lane's bin add their count with one
      // atomic, a few rounds, before the rest add one by one
      for (int r = 0; r < 4; ++r) {
        const uint64_t am = __ballot(act);
        if (am == 0) break;
        const int leader = __ffsll((long long)am) - 1;
        const int lbin = __builtin_amdgcn_readlane(bin, leader);
        const uint64_t same = __ballot(act && bin == lbin);
        if (lane == leader) atomicAdd(&sh.hist[lbin], __popcll(same));
        if (bin == lbin) act = false;
      }
      if (act) atomicAdd(&sh.hist[bin], 1);
    }
    __syncthreads();
    // suffix sums: thread t holds bin 255 - t, so an exclusive scan over t
    // gives the number of candidates in the bins above
    const int need = sh.need;
    const int bin = 255 - tid;
    const int cnt = tid < 256 ? sh.hist[bin] : 0;
    int tot;
    const int above = block_exclusive_scan<kCapWaves>(cnt, &tot);
    if (tid < 256 && above < need && above + cnt >= need) {  // exactly one bin
      sh.prefix = prefix | ((uint32_t)bin << shift);
      sh.need = need - above;
    }
    pmask |= 255u << shift;
    __syncthreads();
  }
  const uint32_t gstar = sh.prefix;
  const int need_eq = sh.need;  // candidates equal to g* that are kept (lowest tokens)
  const uint64_t below = (1ull << lane) - 1ull;
  const int rounds = (n + kCapThreads - 1) / kCapThreads;
  for (int c0 = 0; c0 < rounds; c0 += kCapRounds) {
    const int nr = min(kCapRounds, rounds - c0);
    const int eq_carry = sh.eq_total, kept_carry = sh.kept_total;
    for (int r = 0; r < nr; ++r) {
      const int i = (c0 + r) * kCapThreads + tid;
      const uint64_t bal = __ballot(i < n && key_at(i) == gstar);
      if (lane == 0) sh.cnt[r * kCapWaves + wave] = __popcll(bal);
    }
    __syncthreads();
    int etot;
    int pre = block_exclusive_scan<kCapWaves>(tid < nr * kCapWaves ? sh.cnt[tid] : 0, &etot);
    if (tid < nr * kCapWaves) sh.pre[tid] = eq_carry + pre;
    __syncthreads();
    for (int r = 0; r < nr; ++r) {
      const int i = (c0 + r) * kCapThreads + tid;
      const bool in = i < n;
      const uint32_t key = in ? key_at(i) : 0u;
      const bool eq = in && key == gstar;
      const int eq_rank = sh.pre[r * kCapWaves + wave] + __popcll(__ballot(eq) & below);
      const uint64_t kbal = __ballot(in && (key > gstar || (eq && eq_rank < need_eq)));
      if (lane == 0) sh.cnt[r * kCapWaves + wave] = __popcll(kbal);
    }
    __syncthreads();
    int ktot;
    pre = block_exclusive_scan<kCapWaves>(tid < nr * kCapWaves ? sh.cnt[tid] : 0, &ktot);
    if (tid < nr * kCapWaves) sh.kpre[tid] = kept_carry + pre;
    __syncthreads();
    for (int r = 0; r < nr; ++r) {
      const int i = (c0 + r) * kCapThreads + tid;
      const bool in = i < n;
      const uint32_t key = in ? key_at(i) : 0u;
      const bool eq = in && key == gstar;
      const int eq_rank = sh.pre[r * kCapWaves + wave] + __popcll(__ballot(eq) & below);
      const bool keep = in && (key > gstar || (eq && eq_rank < need_eq));
      const uint64_t kbal = __ballot(keep);
      if (in) {
        const int a = idx_at(i);
        if (keep) {
          const int row = base + sh.kpre[r * kCapWaves + wave] + __popcll(kbal & below);
          slot[a] = row;
          row_src[row] = a / k;
          row_gate[row] = __uint_as_float(key);
        } else {
          slot[a] = -1;
        }
      }
    }
    __syncthreads();
    if (tid == 0) {
      sh.eq_total = eq_carry + etot;
      sh.kept_total = kept_carry + ktot;
    }
    __syncthreads();
  }
}

// The same selection for n <= kCapLds with the candidates in registers:
// candidate i = u * kCapThreads + tid is kv[u] / iv[u] (round u of the
// compaction). g* is found bit by bit, from the top: v | 2^b is kept as the
// prefix when at least C candidates are >= it, one workgroup count per bit
// (each reads only registers; the per-wave counts alternate between two LDS
// rows so one barrier per bit suffices), stopping early once exactly C
// candidates are >= the prefix. The counts are exact, so g* and `need`
// equal the radix select's.
template <int U>
__device__ __forceinline__ void capacity_core_regs(CapShared& sh, const uint32_t (&kv)[U],
                                                   const int32_t (&iv)[U], int n, int k, int capacity,
                                                   int base, int32_t* __restrict__ slot,
                                                   int32_t* __restrict__ row_src,
                                                   float* __restrict__ row_gate) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  // padding keys (i >= n) are 0 and every threshold tried is >= 1, so the
  // compare alone decides
  auto count_ge = [&](uint32_t t, int buf) {
    int c = 0;
#pragma unroll
    for (int u = 0; u < U; ++u) c += __popcll(__ballot(kv[u] >= t));
    if (lane == 0) sh.cnt[buf * kCapWaves + wave] = c;
    __syncthreads();
    int tot = 0;
#pragma unroll
    for (int w = 0; w < kCapWaves; ++w) tot += sh.cnt[buf * kCapWaves + w];
    return tot;
  };
  // v: the bits of g* fixed so far, cv = #keys >= v (>= C). Once cv == C the
  // keys >= v are exactly the C largest and g* is the smallest of them.
  uint32_t v = 0u;
  int cv = n, buf = 0;
  for (int b = 31; b >= 0 && cv != capacity; --b) {
    const uint32_t t = v | (1u << b);
    const int c = count_ge(t, buf);
    buf ^= 1;
    if (c >= capacity) {
      v = t;
      cv = c;
    }
  }
  __syncthreads();  // the last count's reads end before its rows are reused
  uint32_t gstar = v;
  if (cv == capacity) {
    uint32_t m = 0xffffffffu;
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (u * kCapThreads + tid < n && kv[u] >= v) m = min(m, kv[u]);
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) m = min(m, (uint32_t)__shfl_xor((int)m, o, kWave));
    if (lane == 0) sh.hist[wave] = (int)m;
    __syncthreads();
    uint32_t mm = 0xffffffffu;
    for (int w = 0; w < kCapWaves; ++w) mm = min(mm, (uint32_t)sh.hist[w]);
    gstar = mm;
  }
  // keys > g* are those >= g* + 1 (g* + 1 >= 1, so padding stays out)
  const int above = gstar == 0xffffffffu ? 0 : count_ge(gstar + 1u, 0);
  const int need_eq = capacity - above;
  __syncthreads();
  const uint64_t below = (1ull << lane) - 1ull;
  // equal-gate ranks, then kept ranks, in candidate order
  bool eqs[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    eqs[u] = u * kCapThreads + tid < n && kv[u] == gstar;
    const uint64_t bal = __ballot(eqs[u]);
    if (lane == 0) sh.cnt[u * kCapWaves + wave] = __popcll(bal);
  }
  __syncthreads();
  int etot;
  int pre = block_exclusive_scan<kCapWaves>(tid < U * kCapWaves ? sh.cnt[tid] : 0, &etot);
  if (tid < U * kCapWaves) sh.pre[tid] = pre;
  __syncthreads();
  bool keep[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const bool in = u * kCapThreads + tid < n;
    const int eq_rank = sh.pre[u * kCapWaves + wave] + __popcll(__ballot(eqs[u]) & below);
    keep[u] = in && (kv[u] > gstar || (eqs[u] && eq_rank < need_eq));
    const uint64_t kbal = __ballot(keep[u]);
    if (lane == 0) sh.cnt[u * kCapWaves + wave] = __popcll(kbal);
  }
  __syncthreads();
  int ktot;
  pre = block_exclusive_scan<kCapWaves>(tid < U * kCapWaves ? sh.cnt[tid] : 0, &ktot);
  if (tid < U * kCapWaves) sh.kpre[tid] = pre;
  __syncthreads();
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const uint64_t kbal = __ballot(keep[u]);
    if (u * kCapThreads + tid >= n) continue;
    const int a = iv[u];
    if (keep[u]) {
      const int row = base + sh.kpre[u * kCapWaves + wave] + __popcll(kbal & below);
      slot[a] = row;
      row_src[row] = a / k;
      row_gate[row] = __uint_as_float(kv[u]);
    } else {
      slot[a] = -1;
    }
  }
}

__global__ __launch_bounds__(kCapThreads) void dispatch_capacity(
    int k, int e_lo, int L, int capacity, const int32_t* __restrict__ counts,
    const int32_t* __restrict__ offsets, const int32_t* __restrict__ cseg,
    const uint32_t* __restrict__ cand_key, const int32_t* __restrict__ cand_idx,
    int32_t* __restrict__ slot, int32_t* __restrict__ row_src, float* __restrict__ row_gate) {
  __shared__ CapShared sh;
  const int le = blockIdx.x;
  // the three loads issued together (le < L: all in bounds)
  const int n = counts[e_lo + le];
  const int cs = cseg[le];
  const int base = offsets[le];
  if (n <= capacity) return;
  const uint32_t* ck = cand_key + cs;
  const int32_t* ci = cand_idx + cs;
  if (n <= kCapLds) {
    // all of a thread's loads in flight at once; the candidates stay in
    // registers
    constexpr int U = kCapLds / kCapThreads;
    uint32_t kv[U];
    int32_t iv[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int i = u * kCapThreads + (int)threadIdx.x;
      kv[u] = i < n ? ck[i] : 0u;
      iv[u] = i < n ? ci[i] : 0;
    }
    capacity_core_regs<U>(sh, kv, iv, n, k, capacity, base, slot, row_src, row_gate);
  } else {
    capacity_core(sh, [&](int i) { return ck[i]; }, [&](int i) { return ci[i]; }, n, k, capacity,
                  base, slot, row_src, row_gate);
  }
}

// ------------------------------------------------------ token remapping ---
// Overflowing assignments go to the token's next-ranked experts instead of
// being dropped ("Adapting Ultra-Large MoE Models: Engineering Practices and
// Optimization Pathways", §3.3: excess tokens are remapped or dropped). Four
// steps on the stream:
//   1. the capacity dispatch over all E experts (which slots overflow);
//   2. remap_prep: per token, the m-th overflowing slot (j order) proposes to
//      alt[t, m], the expert ranked k + m, keyed by its gate; a kept slot
//      stays with its expert and a key above every gate (+inf);
//   3. the capacity dispatch of those (expert, key) pairs over the local
//      experts: an expert keeps all its kept slots (at most C, all +inf) and
//      fills the room left with the best proposals (key desc, token asc),
//      rows in token order;
//   4. remap_fixup: the rows' gates (step 3 stored the keys) and the number
//      of accepted proposals.
// A token's served experts stay distinct: alternates lie outside its
// selection and are distinct among themselves.

// One wave per token (4 per workgroup), lanes j < k. Workgroup 0 also zeroes
// `moved`, which remap_fixup counts into afterwards on the same stream.
__global__ __launch_bounds__(256) void remap_prep(const int32_t* __restrict__ idx,
                                                  const int32_t* __restrict__ alt,
                                                  const float* __restrict__ gate,
                                                  const int32_t* __restrict__ slot1, int T, int k,
                                                  int32_t* __restrict__ idx2, float* __restrict__ key2,
                                                  int32_t* __restrict__ moved) {
  if (blockIdx.x == 0 && threadIdx.x == 0 && moved) *moved = 0;
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (int)(threadIdx.x >> 6);
  if (t >= T) return;
  const bool in = lane < k;
  const int64_t a = (int64_t)t * k + lane;
  const bool kept = in && slot1[a] >= 0;
  const uint64_t over = __ballot(in && !kept);
  const int m = __popcll(over & ((1ull << lane) - 1ull));  // earlier overflowing slots
  if (in) {
    idx2[a] = kept ? idx[a] : alt[(int64_t)t * k + m];
    key2[a] = kept ? __uint_as_float(0x7f800000u) : gate[a];
  }
}

// row_gate[slot[a]] = gate[a] for every served assignment; *moved += the
// served assignments that were proposals (key below +inf). Integer adds, so
// the count does not depend on the order.
__global__ __launch_bounds__(256) void remap_fixup(const float* __restrict__ gate,
                                                   const float* __restrict__ key2,
                                                   const int32_t* __restrict__ slot, int64_t n,
                                                   float* __restrict__ row_gate, int32_t* __restrict__ moved) {
  int cnt = 0;
  for (int64_t a = (int64_t)blockIdx.x * 256 + threadIdx.x; a < n; a += (int64_t)gridDim.x * 256) {
    const int r = slot[a];
    if (r >= 0) {
      row_gate[r] = gate[a];
      cnt += __float_as_uint(key2[a]) != 0x7f800000u ? 1 : 0;
    }
  }
  if (!moved) return;
  for (int o = 32; o >= 1; o >>= 1) cnt += __shfl_xor(cnt, o, kWave);
  if ((threadIdx.x & 63) == 0 && cnt) atomicAdd(moved, cnt);
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
                           void* x_perm, int32_t* dropped, bool hist_done) {
  const int ntiles = (s.T + kTokTile - 1) / kTokTile;
  const int L = s.e_hi - s.e_lo;
  hipError_t err;
  if (ntiles > 0 && !hist_done) {  // else the top-k kernel filled tile_counts
    TimedLaunch tl(MOE_K_HIST, c.stream);
    hipLaunchKernelGGL(dispatch_hist, dim3(ntiles), dim3(256), 0, c.stream, idx, s.T, s.k, s.E,
                       ws.tile_counts);
  }
  if ((err = hipGetLastError()) != hipSuccess) return err;
  {
    TimedLaunch tl(MOE_K_SCAN, c.stream);
    hipLaunchKernelGGL(dispatch_tile_scan, dim3((s.E + 256 / kScanParts - 1) / (256 / kScanParts)),
                       dim3(256), 0, c.stream,
                       ws.tile_counts, ntiles, s.E, ws.tile_base, counts);
  }
  if ((err = hipGetLastError()) != hipSuccess) return err;
  {
    // at least one workgroup: workgroup 0 writes offsets / dropped even for T = 0
    TimedLaunch tl(MOE_K_SCATTER, c.stream);
    hipLaunchKernelGGL(dispatch_scatter, dim3(ntiles > 0 ? ntiles : 1), dim3(256), 0, c.stream, idx,
                       gate, s.T, s.k, s.E, s.e_lo, L, s.capacity, ws.tile_base, counts, offsets,
                       ws.cseg, dropped, slot, row_src, row_gate, ws.cand_key, ws.cand_idx);
  }
  if ((err = hipGetLastError()) != hipSuccess) return err;
  if (s.capacity > 0) {
    TimedLaunch tl(MOE_K_CAPACITY, c.stream);
    hipLaunchKernelGGL(dispatch_capacity, dim3(L), dim3(kCapThreads), 0, c.stream, s.k, s.e_lo, L,
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

hipError_t launch_dispatch_remap(const Ctx& c, const moe_shape_t& s, const Workspace& ws, const int32_t* idx,
                                 const float* gate, const int32_t* alt, const void* x, int32_t* counts,
                                 int32_t* offsets, int32_t* slot, int32_t* row_src, float* row_gate, void* x_perm,
                                 int32_t* moved, int32_t* dropped) {
  hipError_t err;
  // 1. which slots overflow: the capacity rule over every expert
  moe_shape_t all = s;
  all.e_lo = 0;
  all.e_hi = s.E;
  if ((err = launch_dispatch(c, all, ws, idx, gate, nullptr, counts, ws.rm_offsets1, ws.rm_slot1, ws.rm_src1,
                             ws.rm_gate1, nullptr, nullptr)) != hipSuccess)
    return err;
  // 2. proposals
  const int blocks = s.T > 0 ? (s.T + 3) / 4 : 1;
  hipLaunchKernelGGL(remap_prep, dim3(blocks), dim3(256), 0, c.stream, idx, alt, gate, ws.rm_slot1, s.T, s.k,
                     ws.rm_idx2, ws.rm_key2, moved);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  // 3. kept slots plus the best proposals, on the local experts
  if ((err = launch_dispatch(c, s, ws, ws.rm_idx2, ws.rm_key2, x, ws.rm_counts2, offsets, slot, row_src, row_gate,
                             x_perm, dropped)) != hipSuccess)
    return err;
  // 4. gates of the rows, accepted proposals
  const int64_t n = (int64_t)s.T * s.k;
  if (n == 0) return hipSuccess;
  const int grid = (int)std::min<int64_t>((n + 255) / 256, (int64_t)c.num_cus * 8);
  hipLaunchKernelGGL(remap_fixup, dim3(grid), dim3(256), 0, c.stream, gate, ws.rm_key2, slot, n, row_gate, moved);
  return hipGetLastError();
}

}  // namespace moe
