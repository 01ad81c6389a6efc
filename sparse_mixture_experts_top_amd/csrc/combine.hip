// Combine: y[t] = sum_j g[t, j] * y_perm[slot[t, j]] over the token's kept,
// local slots, summed in j order in fp32 ("Adapting Trillion-Parameter MoE
// Models for LoRA Fine-Tuning: A Full-Stack Engineering Guide", §2.1: results
// are gathered back and weighted by the gate; "Trillion-Parameter MoE Model
// Training Adaptation: Full-Stack Optimization Practices", §3: unpermute).
//
// One workgroup per TB consecutive tokens (grid-stride beyond that). A wave
// per token loads its k slots and gates (one load per lane) and compacts the
// kept ones, in j order, into LDS with a ballot; a token with none kept (a
// dropped or non-local one) then costs only its zero store. Each thread owns
// 8 consecutive columns and
// reads them from each selected row with one 16-byte load (bf16), so a row is
// read by the workgroup as contiguous 4-8 KB. The loads of 8 rows are issued
// together and then accumulated in j order (the summation order is part of
// the definition), so their latencies overlap.
#include "common.h"

namespace moe {

// Adds entries j0 .. j0 + min(NB, nb) - 1 of a token's compacted list to
// acc in j order. All NB loads are issued before the first use (entries past
// nb re-read the last valid row and contribute 0 * 0 through selects, not
// branches, which would let the compiler sink each load to its use).
template <int NB>
__device__ __forceinline__ void combine_batch(float (&acc)[8], const bf16_t* __restrict__ y_perm,
                                              const int* s_slot, const float* s_gate, int j0, int nb,
                                              int d, int v) {
  int rs[NB];
#pragma unroll
  for (int b = 0; b < NB; ++b) rs[b] = s_slot[j0 + min(b, nb - 1)];
  uint4 raw[NB];
#pragma unroll
  for (int b = 0; b < NB; ++b) raw[b] = *reinterpret_cast<const uint4*>(y_perm + (int64_t)rs[b] * d + v * 8);
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    const bool in = b < nb;
    const float g = in ? s_gate[j0 + b] : 0.f;
    const uint32_t w[4] = {in ? raw[b].x : 0u, in ? raw[b].y : 0u, in ? raw[b].z : 0u, in ? raw[b].w : 0u};
#pragma unroll
    for (int u = 0; u < 8; ++u)
      acc[u] = fmaf(g, bf16_to_f32(static_cast<bf16_t>(w[u >> 1] >> ((u & 1) * 16))), acc[u]);
  }
}

template <int TB>
__global__ __launch_bounds__(256) void combine_bf16(const bf16_t* __restrict__ y_perm,
                                                    const int32_t* __restrict__ slot,
                                                    const float* __restrict__ gate, int T, int k,
                                                    int d, bf16_t* __restrict__ y) {
  constexpr int B = 8;  // rows per full batch, loaded before they are accumulated in order
  __shared__ int s_slot[TB][32];
  __shared__ float s_gate[TB][32];
  __shared__ int s_n[TB];
  const int nvec = d / 8;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  for (int t0 = blockIdx.x * TB; t0 < T; t0 += gridDim.x * TB) {
    const int nq = min(TB, T - t0);
    // wave w compacts the kept slots of tokens w, w + 4, ... in j order:
    // lane j loads entry j, a ballot gives its position among the kept ones
    for (int q = wave; q < nq; q += 4) {
      const int64_t e = (int64_t)(t0 + q) * k + lane;
      const int sl = lane < k ? slot[e] : -1;
      const float g = lane < k ? gate[e] : 0.f;
      const uint64_t kept = __ballot(sl >= 0);
      const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
      if (sl >= 0) {
        const int pos = __popcll(kept & below);
        s_slot[q][pos] = sl;
        s_gate[q][pos] = g;
      }
      if (lane == 0) s_n[q] = __popcll(kept);
    }
    __syncthreads();
    for (int q = 0; q < nq; ++q) {
      const int t = t0 + q;
      const int n = s_n[q];
      for (int v = threadIdx.x; v < nvec; v += blockDim.x) {
        float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
        int j0 = 0;
        for (; j0 + B <= n; j0 += B) combine_batch<B>(acc, y_perm, s_slot[q], s_gate[q], j0, B, d, v);
        for (; j0 < n; j0 += 2) combine_batch<2>(acc, y_perm, s_slot[q], s_gate[q], j0, n - j0, d, v);
        uint32_t o[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) o[u] = f32x2_to_bf16x2(acc[2 * u], acc[2 * u + 1]);
        *reinterpret_cast<uint4*>(y + (int64_t)t * d + v * 8) = make_uint4(o[0], o[1], o[2], o[3]);
      }
    }
    __syncthreads();
  }
}

__global__ __launch_bounds__(256) void combine_f32(const float* __restrict__ y_perm,
                                                   const int32_t* __restrict__ slot,
                                                   const float* __restrict__ gate, int T, int k,
                                                   int d, float* __restrict__ y) {
  __shared__ int s_slot[32];
  __shared__ float s_gate[32];
  for (int t = blockIdx.x; t < T; t += gridDim.x) {
    if (threadIdx.x < k) {
      s_slot[threadIdx.x] = slot[(int64_t)t * k + threadIdx.x];
      s_gate[threadIdx.x] = gate[(int64_t)t * k + threadIdx.x];
    }
    __syncthreads();
    for (int c = threadIdx.x; c < d; c += blockDim.x) {
      float acc = 0.f;
      for (int j = 0; j < k; ++j) {
        const int sl = s_slot[j];
        if (sl >= 0) acc = fmaf(s_gate[j], y_perm[(int64_t)sl * d + c], acc);
      }
      y[(int64_t)t * d + c] = acc;
    }
    __syncthreads();
  }
}

hipError_t launch_combine(const Ctx& c, const moe_shape_t& s, const void* y_perm,
                          const int32_t* slot, const float* gate, void* y) {
  TimedLaunch tl(MOE_K_COMBINE, c.stream);
  if (s.dtype == MOE_BF16) {
    // TB tokens per workgroup (their slot/gate loads are one round trip),
    // as many as keep >= 8 workgroups per CU; grid-stride beyond 64 per CU
    int tb = s.T / (c.num_cus * 8);
    tb = tb >= 8 ? 8 : tb >= 4 ? 4 : tb >= 2 ? 2 : 1;
    const int nblk = (s.T + tb - 1) / tb;
    const int grid = nblk < c.num_cus * 64 ? nblk : c.num_cus * 64;
#define MOE_COMBINE(N)                                                                          \
  hipLaunchKernelGGL(combine_bf16<N>, dim3(grid), dim3(256), 0, c.stream, (const bf16_t*)y_perm, \
                     slot, gate, s.T, s.k, s.d, (bf16_t*)y)
    if (tb == 8) MOE_COMBINE(8);
    else if (tb == 4) MOE_COMBINE(4);
    else if (tb == 2) MOE_COMBINE(2);
    else MOE_COMBINE(1);
#undef MOE_COMBINE
    return hipGetLastError();
  }
  const int grid = s.T < c.num_cus * 16 ? s.T : c.num_cus * 16;
  hipLaunchKernelGGL(combine_f32, dim3(grid), dim3(256), 0, c.stream, (const float*)y_perm, slot,
                     gate, s.T, s.k, s.d, (float*)y);
  return hipGetLastError();
}

}  // namespace moe
