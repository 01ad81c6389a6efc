// Routing: router GEMM, softmax + top-k + renormalised gates, load-balance loss.
//
// The router scores every expert for every token (logits = x W_r^T + b), each
// token keeps its k best experts, and the gate is the softmax restricted to
// them ("Adapting Trillion-Parameter MoE Models for LoRA Fine-Tuning: A
// Full-Stack Engineering Guide", §2.1: g_i is the routing gate score; "Day-
// Level Adaptation and LoRA Fine-Tuning of Ultra-Large-Scale Sparse MoE
// Models", §2.1: Top-16 selection and the auxiliary load-balancing loss).
#include "common.h"
#include "mfma_tile.h"

namespace moe {

// ------------------------------------------------------------ router GEMM ---

// bf16: logits[T, E] (f32) = x[T, d] * w[E, d]^T + bias, one 128 x 128 (or
// 64 x 128) tile per item on the persistent pipelined driver.
// The same engine computes the latent router's projection z = x W_c^T
// (T, d, E read as rows, K, output columns): out_b set stores the product
// rounded to bf16, without a bias.
template <class Cfg>
struct RouterProb {
  const bf16_t* x;
  const bf16_t* w;
  const float* bias;
  float* logits;
  int T, d, E, nt;
  bf16_t* out_b = nullptr;
  int32_t* zero = nullptr;  // cleared by the kernel on the side (zero_n entries)
  int64_t zero_n = 0;

  __device__ __forceinline__ int rows(int item) const { return min(Cfg::BM, T - (item / nt) * Cfg::BM); }

  __device__ __forceinline__ void setup(int item, DmaLoader<Cfg>& ld, int part) const {
    const int m0 = (item / nt) * Cfg::BM, n0 = (item % nt) * Cfg::BN;
    const int ce = dma_chunk_elem<Cfg>();
#pragma unroll
    for (int q = 0; q < Cfg::A_DMA / Cfg::DW; ++q)
      ld.a[q] = x + (int64_t)min(m0 + dma_row<Cfg>(q * Cfg::DW + part), T - 1) * d + ce;
#pragma unroll
    for (int q = 0; q < Cfg::B_Q; ++q)
      ld.b[q] = w + (int64_t)min(n0 + dma_row<Cfg>(b_inst<Cfg>(q, part)), E - 1) * d + ce;
  }

  __device__ __forceinline__ void epilogue(int item, Acc<Cfg>& acc) const {
    const int m0 = (item / nt) * Cfg::BM, n0 = (item % nt) * Cfg::BN;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int wm = wave / Cfg::WN, wn = wave % Cfg::WN;
    if (out_b) {  // E % 4 == 0 here: a lane's four columns are all valid or all not
#pragma unroll
      for (int j = 0; j < Cfg::FN; ++j) {
        const int n = n0 + dma_out_col<Cfg>(wn, j, lane);
        if (n >= E) continue;
#pragma unroll
        for (int i = 0; i < Cfg::FM; ++i) {
          const int m = m0 + dma_out_row<Cfg>(wm, i, lane);
          if (m < T)
            *reinterpret_cast<uint2*>(out_b + (int64_t)m * E + n) =
                pack4_bf16(acc.v[i][j][0], acc.v[i][j][1], acc.v[i][j][2], acc.v[i][j][3]);
        }
      }
      return;
    }
#pragma unroll
    for (int j = 0; j < Cfg::FN; ++j) {
      const int n = n0 + dma_out_col<Cfg>(wn, j, lane);
      if (n >= E) continue;
      float b[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) b[q] = (bias && n + q < E) ? bias[n + q] : 0.f;
#pragma unroll
      for (int i = 0; i < Cfg::FM; ++i) {
        const int m = m0 + dma_out_row<Cfg>(wm, i, lane);
        if (m >= T) continue;
        float* dst = logits + (int64_t)m * E + n;
        if (n + 4 <= E && (E & 3) == 0) {
          *reinterpret_cast<float4*>(dst) = make_float4(acc.v[i][j][0] + b[0], acc.v[i][j][1] + b[1],
                                                        acc.v[i][j][2] + b[2], acc.v[i][j][3] + b[3]);
        } else {
#pragma unroll
          for (int q = 0; q < 4; ++q)
            if (n + q < E) dst[q] = acc.v[i][j][q] + b[q];
        }
      }
    }
  }
};

// Grid-stride clear of n int32 (16-byte stores; the buffer is 16-byte aligned).
__device__ __forceinline__ void clear_i32(int32_t* p, int64_t n) {
  const int64_t tid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t nthr = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = tid; i < n / 4; i += nthr) reinterpret_cast<int4*>(p)[i] = make_int4(0, 0, 0, 0);
  for (int64_t i = (n / 4) * 4 + tid; i < n; i += nthr) p[i] = 0;
}

template <class Cfg>
__global__ __launch_bounds__(Cfg::THREADS, Cfg::WAVES_PER_SIMD) void router_gemm_bf16(RouterProb<Cfg> pb, int items) {
  if constexpr (Cfg::PW == 0)
    persistent_gemm_sym<Cfg>(pb, items, pb.d / Cfg::BK);
  else
    persistent_gemm_dma<Cfg>(pb, items, pb.d / Cfg::BK);
  if (pb.zero) clear_i32(pb.zero, pb.zero_n);
}

// fp32: one thread per logit, plain dot product (small parity workloads).
__global__ __launch_bounds__(256) void router_gemm_f32(const float* __restrict__ x,
                                                       const float* __restrict__ w,
                                                       const float* __restrict__ bias,
                                                       float* __restrict__ logits, int T, int d,
                                                       int E, int32_t* __restrict__ zero, int64_t zero_n) {
  const int64_t id = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (id < zero_n) zero[id] = 0;  // zero_n <= T * E
  if (id >= (int64_t)T * E) return;
  const int t = (int)(id / E), e = (int)(id % E);
  const float* xr = x + (int64_t)t * d;
  const float* wr = w + (int64_t)e * d;
  float acc = 0.f;
  for (int i = 0; i < d; ++i) acc = fmaf(xr[i], wr[i], acc);
  logits[id] = acc + (bias ? bias[e] : 0.f);
}

template <class Cfg>
static hipError_t launch_router_bf16(const Ctx& c, int M, int N, int K, const bf16_t* x, const bf16_t* w,
                                     const float* bias, float* logits, bf16_t* out_b, int32_t* zero,
                                     int64_t zero_n) {
  const int mt = (M + Cfg::BM - 1) / Cfg::BM, nt = (N + Cfg::BN - 1) / Cfg::BN;
  const int items = mt * nt;
  // one workgroup per CU (the workgroups are sized to fill one), a multiple of 8 (XCDs)
  const int grid = std::min(((items + 7) / 8) * 8, c.num_cus);
  RouterProb<Cfg> pb{x, w, bias, logits, M, K, N, nt};
  pb.out_b = out_b;
  pb.zero = zero;
  pb.zero_n = zero_n;
  TimedLaunch tl(MOE_K_ROUTER_GEMM, c.stream);
  hipLaunchKernelGGL(router_gemm_bf16<Cfg>, dim3(grid), dim3(Cfg::THREADS), 0, c.stream, pb, items);
  return hipGetLastError();
}

// Router tile configurations (the router is a dense, compute-bound GEMM, so
// the large ones run 8 compute waves - two per SIMD, which the MFMA issue
// rate needs):
//   wide    256 x 224, 8 symmetric waves (each computes 64 x 112 and issues
//           DMAs), when there are at least as many such tiles as CUs and
//           224-wide column tiles waste fewer columns than 256-wide ones
//           (e.g. T = 16384, E = 896: 4 x 224 columns exactly, where 256-wide
//           tiles would compute 1024);
//   huge    256 x 256, 8 symmetric waves (each computes 128 x 64 and issues
//           DMAs), when there are at least as many such tiles as CUs;
//   large   128 x 256, 8 compute waves of 64 x 64 + 4 producers, when there are at least
//           as many such tiles as CUs (e.g. T = 16384, E = 896);
//   medium  128 x 128, 8 compute waves of 64 x 32, when the 128 x 128 tiles
//           cover at least half of the CUs (e.g. T = 4096, E = 896);
//   small   64 x 128, 4 compute waves, otherwise.
#ifndef MOE_ROUTER_STAGES
#define MOE_ROUTER_STAGES 6
#endif
using RouterWide = DmaCfg<256, 224, 2, 4, 8, 0, 64>;
using RouterHuge = DmaCfg<256, 256, 2, 2, 8, 0, 64>;
using RouterLarge = DmaCfg<128, 256, MOE_ROUTER_STAGES, 2, 8, 4>;
using RouterMedium = DmaCfg<128, 128, MOE_ROUTER_STAGES, 2, 8, 4>;
using RouterSmall = DmaCfg<64, 128, 4, 2, 4, 4>;

// bf16 [M, K] x [N, K]^T on the router engine: fp32 out (+ bias) or, with
// out_b, bf16 out. K % 64 == 0.
hipError_t launch_router_mnk(const Ctx& c, int M, int N, int K, const bf16_t* xb, const bf16_t* wb,
                             const float* bias, float* logits, bf16_t* out_b, int32_t* zero, int64_t zero_n) {
  const int mt128 = (M + 127) / 128;
  const int nt224 = (N + 223) / 224, nt256 = (N + 255) / 256;
  if (((M + 255) / 256) * nt224 >= c.num_cus && nt224 * 224 < nt256 * 256)
    return launch_router_bf16<RouterWide>(c, M, N, K, xb, wb, bias, logits, out_b, zero, zero_n);
  if (((M + 255) / 256) * nt256 >= c.num_cus)
    return launch_router_bf16<RouterHuge>(c, M, N, K, xb, wb, bias, logits, out_b, zero, zero_n);
  if (mt128 * ((N + 255) / 256) >= c.num_cus)
    return launch_router_bf16<RouterLarge>(c, M, N, K, xb, wb, bias, logits, out_b, zero, zero_n);
  if (2 * mt128 * ((N + 127) / 128) >= c.num_cus)
    return launch_router_bf16<RouterMedium>(c, M, N, K, xb, wb, bias, logits, out_b, zero, zero_n);
  return launch_router_bf16<RouterSmall>(c, M, N, K, xb, wb, bias, logits, out_b, zero, zero_n);
}

hipError_t launch_router(const Ctx& c, const moe_shape_t& s, const void* x, const void* w,
                         const float* bias, float* logits, int32_t* zero, int64_t zero_n) {
  if (s.dtype == MOE_BF16)
    return launch_router_mnk(c, s.T, s.E, s.d, (const bf16_t*)x, (const bf16_t*)w, bias, logits, nullptr, zero,
                             zero_n);
  const int64_t n = (int64_t)s.T * s.E;
  TimedLaunch tl(MOE_K_ROUTER_GEMM, c.stream);
  hipLaunchKernelGGL(router_gemm_f32, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, c.stream,
                     (const float*)x, (const float*)w, bias, logits, s.T, s.d, s.E, zero, zero_n);
  return hipGetLastError();
}

// --------------------------------------------------------- top-k + gates ---

// Order-preserving map of an fp32 value to uint32 (larger value -> larger
// code); -0.0 is mapped like +0.0 so the two compare equal.
__device__ __forceinline__ uint32_t ordered_bits(float v) {
  uint32_t u = __float_as_uint(v);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float from_ordered(uint32_t o) {
  return __uint_as_float((o & 0x80000000u) ? (o & 0x7fffffffu) : ~o);
}

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) {
    const uint32_t lo = __shfl_xor((uint32_t)v, m, kWave);
    const uint32_t hi = __shfl_xor((uint32_t)(v >> 32), m, kWave);
    const uint64_t o = ((uint64_t)hi << 32) | lo;
    v = o > v ? o : v;
  }
  return v;
}

// One wave per token. Lane l holds the logits of experts l, l+64, ... as
// 64-bit keys (ordered logit bits << 32 | ~expert): the largest key is the
// largest logit and, among equal logits, the lowest expert id; keys are
// unique. The k largest keys are found exactly in three steps:
//   1. tau = the high word of the k-th largest of the 64 lane maxima
//      (bitwise search over the 32 logit bits with ballot counts, no
//      cross-lane shuffles). At least k keys (those maxima) have a high word
//      >= tau, so every one of the k largest keys does.
//   2. keys >= tau are compacted through LDS (ballot + popcount positions).
//   3. if at most 64 survive (typically k plus a few), each survivor counts
//      the larger survivors (LDS broadcast reads) and the one of rank r < k
//      lands in position r, so lanes 0..k-1 hold the answer in order;
//      otherwise (many equal logits) k rounds of "wave maximum, remove it"
//      over all keys.
// Gates: exp(l_j - l_0) / sum over the first kg picks. With alt_out, k = kg +
// the number of alternates: picks kg .. k-1 (the experts ranked next) go to
// alt_out [T, k - kg] and take no gate. With prob_part, the wave also sums the
// full softmax of its tokens per expert; the block's waves are added in a
// fixed order into prob_part[block, E]. With hist, each of the first kg
// picks adds one to hist[t / 32, expert] (integer atomics: the counts do not
// depend on the order the waves run in), the per-tile expert histogram the
// dispatch's tile scan starts from.
template <int EPL, int TPW>
__global__ __launch_bounds__(256) void topk_softmax(const float* __restrict__ logits, int T, int E,
                                                    int k, int kg, int32_t* __restrict__ idx_out,
                                                    float* __restrict__ gate_out,
                                                    int32_t* __restrict__ alt_out,
                                                    float* __restrict__ prob_part,
                                                    int32_t* __restrict__ hist) {
  __shared__ uint64_t cand[4][64];
  __shared__ uint64_t sel[4][32];
  __shared__ float red[4][EPL * 64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));  // lanes < this one
  float psum[EPL];
#pragma unroll
  for (int i = 0; i < EPL; ++i) psum[i] = 0.f;
  for (int q = 0; q < TPW; ++q) {
    const int t = (blockIdx.x * 4 + wave) * TPW + q;
    if (t >= T) break;
    const float* row = logits + (int64_t)t * E;
    uint64_t key[EPL];
    float val[EPL];
    uint64_t lmax = 0;
    // all loads first (clamped, so unconditional): issued back to back, one wait
#pragma unroll
    for (int i = 0; i < EPL; ++i) val[i] = row[min(lane + 64 * i, E - 1)];
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
      const int e = lane + 64 * i;
      const bool ok = e < E;
      val[i] = ok ? val[i] : 0.f;
      key[i] = ok ? ((uint64_t)ordered_bits(val[i]) << 32) | (uint32_t)(0xffffffffu - (uint32_t)e) : 0ull;
      lmax = key[i] > lmax ? key[i] : lmax;
    }
    // 1. tau: the largest logit-bits value t (the key's high word) such that
    //    at least k lane maxima have high word >= t; then at least k keys are
    //    >= t << 32, so the k-th largest key is too, and every top-k key is a
    //    candidate below. The low word (expert id) only orders ties, which
    //    the sort of the candidates settles.
    uint64_t tau = 0;
    for (int b = 63; b >= 32; --b) {
      const uint64_t c = tau | (1ull << b);
      if (__popcll(__ballot(lmax >= c)) >= k) tau = c;
    }
    // 2. candidates
    int n = 0;
#pragma unroll
    for (int i = 0; i < EPL; ++i) n += __popcll(__ballot(key[i] >= tau));
    uint64_t mine = 0;  // this lane's key after selection (lanes 0..k-1)
    if (n <= 64) {
      int base = 0;
#pragma unroll
      for (int i = 0; i < EPL; ++i) {
        const bool in = key[i] >= tau;
        const uint64_t bal = __ballot(in);
        if (in) cand[wave][base + __popcll(bal & below)] = key[i];
        base += __popcll(bal);
      }
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
      // rank of each candidate = number of larger candidates (keys are
      // unique); the candidate of rank r < k goes to position r
      const uint64_t v = lane < n ? cand[wave][lane] : 0ull;
      int rank = 0;
      for (int j = 0; j < n; ++j) rank += cand[wave][j] > v ? 1 : 0;
      __builtin_amdgcn_wave_barrier();
      if (lane < n && rank < k) sel[wave][rank] = v;
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
      mine = lane < k ? sel[wave][lane] : 0ull;
      __builtin_amdgcn_wave_barrier();
    } else {
      uint64_t kk[EPL];
#pragma unroll
      for (int i = 0; i < EPL; ++i) kk[i] = key[i];
      for (int j = 0; j < k; ++j) {
        uint64_t best = 0;
#pragma unroll
        for (int i = 0; i < EPL; ++i) best = kk[i] > best ? kk[i] : best;
        const uint64_t win = wave_max_u64(best);
#pragma unroll
        for (int i = 0; i < EPL; ++i)
          if (kk[i] == win) kk[i] = 0;
        if (lane == j) mine = win;
      }
    }
    const float top = from_ordered((uint32_t)(__shfl(mine, 0, kWave) >> 32));
    const float my_logit = from_ordered((uint32_t)(mine >> 32));
    const int my_idx = (int)(0xffffffffu - (uint32_t)mine);
    const float ex = lane < kg ? expf(my_logit - top) : 0.f;
    const float den = wave_sum(ex);
    if (lane < kg) {
      idx_out[(int64_t)t * kg + lane] = my_idx;
      gate_out[(int64_t)t * kg + lane] = ex / den;
      if (hist) atomicAdd(hist + (int64_t)(t / kTokTile) * E + my_idx, 1);
    } else if (lane < k) {
      alt_out[(int64_t)t * (k - kg) + (lane - kg)] = my_idx;
    }
    if (prob_part) {
      float z[EPL], zs = 0.f;
#pragma unroll
      for (int i = 0; i < EPL; ++i) {
        z[i] = (lane + 64 * i < E) ? expf(val[i] - top) : 0.f;
        zs += z[i];
      }
      const float Z = wave_sum(zs);
      const float inv = 1.0f / Z;
#pragma unroll
      for (int i = 0; i < EPL; ++i) psum[i] += z[i] * inv;
    }
  }
  if (!prob_part) return;
#pragma unroll
  for (int i = 0; i < EPL; ++i) red[wave][lane + 64 * i] = psum[i];
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += 256)
    prob_part[(int64_t)blockIdx.x * E + e] = ((red[0][e] + red[1][e]) + red[2][e]) + red[3][e];
}

// prob_sum[e] = sum over blocks of prob_part[b, e]. Workgroup of 1024
// threads for kReduceE experts: thread (j, u) (u = expert within the group,
// j = 0 .. 1023 / kReduceE) sums blocks j, j + J, j + 2 J, ... of its expert
// in order (kReduceNB loads in flight per batch; a block's kReduceE experts
// are one 128-byte line), then the J partials of an expert are added
// pairwise in a fixed tree through LDS, so the result does not depend on
// scheduling. At the LoRA step's shape (2048 blocks x 896 experts) this
// takes 8 us against 11 for 64 experts per workgroup summed by 16 waves
// (8 and 16 experts per workgroup: 9.1 and 8.2 us).
constexpr int kReduceE = 32;
constexpr int kReduceNB = 16;
__global__ __launch_bounds__(1024) void prob_reduce(const float* __restrict__ part, int nblk, int E,
                                                    float* __restrict__ out) {
  constexpr int J = 1024 / kReduceE;
  __shared__ float red[J][kReduceE];
  const int u = threadIdx.x % kReduceE, j = threadIdx.x / kReduceE;
  const int e = blockIdx.x * kReduceE + u;
  float acc = 0.f;
  if (e < E) {
    for (int b0 = j; b0 < nblk; b0 += J * kReduceNB) {
      float v[kReduceNB];
#pragma unroll
      for (int q = 0; q < kReduceNB; ++q) {
        const int b = b0 + J * q;
        v[q] = b < nblk ? part[(int64_t)b * E + e] : 0.f;
      }
#pragma unroll
      for (int q = 0; q < kReduceNB; ++q) acc += v[q];
    }
  }
  red[j][u] = acc;
  __syncthreads();
  for (int h = J / 2; h >= 1; h >>= 1) {
    if (j < h) red[j][u] += red[j + h][u];
    __syncthreads();
  }
  if (j == 0 && e < E) out[e] = red[0][u];
}

hipError_t launch_topk(const Ctx& c, const moe_shape_t& s, const float* logits, int32_t* idx,
                       float* gate, float* prob_part, float* prob_sum, int32_t* alt, int32_t* hist) {
  // with alt: k alternates after the k selected experts (2k picks in all)
  const int ksel = alt ? 2 * s.k : s.k;
  // one token per wave; with the softmax sums requested, kTopkTokPerWaveProb tokens per wave
  // so the per-block partial sums stay small
  const int tpw = prob_sum ? kTopkTokPerWaveProb : 1;
  const int nblk = (s.T + 4 * tpw - 1) / (4 * tpw);
  const int epl = (s.E + 63) / 64;
  float* part = prob_sum ? prob_part : nullptr;
  if (nblk > 0) {
    TimedLaunch tl(MOE_K_TOPK, c.stream);
#define MOE_TOPK(N)                                                                                  \
  if (prob_sum)                                                                                      \
    hipLaunchKernelGGL((topk_softmax<N, kTopkTokPerWaveProb>), dim3(nblk), dim3(256), 0, c.stream,    \
                       logits, s.T, s.E, ksel, s.k, idx, gate, alt, part, hist);                     \
  else                                                                                               \
    hipLaunchKernelGGL((topk_softmax<N, 1>), dim3(nblk), dim3(256), 0, c.stream, logits, s.T, s.E,    \
                       ksel, s.k, idx, gate, alt, part, hist)
    if (epl <= 1) MOE_TOPK(1);
    else if (epl <= 2) MOE_TOPK(2);
    else if (epl <= 4) MOE_TOPK(4);
    else if (epl <= 8) MOE_TOPK(8);
    else if (epl <= 14) MOE_TOPK(14);
    else MOE_TOPK(16);
#undef MOE_TOPK
  }
  hipError_t err = hipGetLastError();
  if (err != hipSuccess || !prob_sum) return err;
  TimedLaunch tl(MOE_K_PROB_REDUCE, c.stream);
  hipLaunchKernelGGL(prob_reduce, dim3((s.E + kReduceE - 1) / kReduceE), dim3(1024), 0, c.stream, part, nblk, s.E,
                     prob_sum);
  return hipGetLastError();
}

// ------------------------------------------------------ load-balance loss ---

// out[1] = E * sum_e (counts[e] / (T k)) (prob_sum[e] / T); out[0] = coef out[1].
// One block; fixed-shape tree reduction in double.
__global__ __launch_bounds__(1024) void aux_loss_kernel(const int32_t* __restrict__ counts,
                                                        const float* __restrict__ prob_sum, int T,
                                                        int k, int E, float coef,
                                                        float* __restrict__ out) {
  __shared__ double red[1024];
  const int e = threadIdx.x;
  double v = 0.0;
  if (e < E && T > 0) v = ((double)counts[e] / ((double)T * k)) * ((double)prob_sum[e] / T);
  red[e] = v;
  __syncthreads();
  for (int h = 512; h >= 1; h >>= 1) {
    if (e < h) red[e] += red[e + h];
    __syncthreads();
  }
  if (e == 0) {
    const double raw = (double)E * red[0];
    out[1] = (float)raw;
    out[0] = (float)(coef * raw);
  }
}

hipError_t launch_aux(const Ctx& c, const moe_shape_t& s, const int32_t* counts,
                      const float* prob_sum, float coef, float* out) {
  TimedLaunch tl(MOE_K_AUX, c.stream);
  hipLaunchKernelGGL(aux_loss_kernel, dim3(1), dim3(1024), 0, c.stream, counts, prob_sum, s.T, s.k,
                     s.E, coef, out);
  return hipGetLastError();
}

}  // namespace moe
