// Combine: y[t] = sum_j g[t, j] * y_perm[slot[t, j]] over the token's kept,
// local slots, summed in j order in fp32 ("Adapting Trillion-Parameter MoE
// Models for LoRA Fine-Tuning: A Full-Stack Engineering Guide", §2.1: results
// are gathered back and weighted by the gate; "Trillion-Parameter MoE Model
// Training Adaptation: Full-Stack Optimization Practices", §3: unpermute).
//
// One workgroup per token (grid-stride over tokens). The token's slots and
// gates are staged in LDS; each thread then owns 8 consecutive columns and
// reads them from each selected row with one 16-byte load (bf16), so a row is
// read by the workgroup as contiguous 4-8 KB. The loads of 8 rows are issued
// together and then accumulated in j order (the summation order is part of
// the definition), so their latencies overlap.
#include "common.h"

namespace moe {

__global__ __launch_bounds__(256) void combine_bf16(const bf16_t* __restrict__ y_perm,
                                                    const int32_t* __restrict__ slot,
                                                    const float* __restrict__ gate, int T, int k,
                                                    int d, bf16_t* __restrict__ y) {
  constexpr int B = 8;  // rows loaded per batch, before they are accumulated in order
  __shared__ int s_slot[32];
  __shared__ float s_gate[32];
  const int nvec = d / 8;
  for (int t = blockIdx.x; t < T; t += gridDim.x) {
    if (threadIdx.x < k) {
      s_slot[threadIdx.x] = slot[(int64_t)t * k + threadIdx.x];
      s_gate[threadIdx.x] = gate[(int64_t)t * k + threadIdx.x];
    }
    __syncthreads();
    for (int v = threadIdx.x; v < nvec; v += blockDim.x) {
      float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
      for (int j0 = 0; j0 < k; j0 += B) {
        uint4 raw[B];
#pragma unroll
        for (int b = 0; b < B; ++b) {
          const int j = j0 + b;
          const int sl = j < k ? s_slot[j] : -1;
          raw[b] = sl >= 0 ? *reinterpret_cast<const uint4*>(y_perm + (int64_t)sl * d + v * 8)
                           : make_uint4(0u, 0u, 0u, 0u);
        }
#pragma unroll
        for (int b = 0; b < B; ++b) {
          const int j = j0 + b;
          if (j >= k || s_slot[j] < 0) continue;
          const float g = s_gate[j];
          const uint32_t w[4] = {raw[b].x, raw[b].y, raw[b].z, raw[b].w};
#pragma unroll
          for (int u = 0; u < 8; ++u)
            acc[u] = fmaf(g, bf16_to_f32(static_cast<bf16_t>(w[u >> 1] >> ((u & 1) * 16))), acc[u]);
        }
      }
      uint32_t o[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) o[u] = f32x2_to_bf16x2(acc[2 * u], acc[2 * u + 1]);
      *reinterpret_cast<uint4*>(y + (int64_t)t * d + v * 8) = make_uint4(o[0], o[1], o[2], o[3]);
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
  // one token per workgroup up to 64 workgroups per CU, grid-stride beyond
  const int grid = s.T < c.num_cus * 64 ? s.T : c.num_cus * 64;
  TimedLaunch tl(MOE_K_COMBINE, c.stream);
  if (s.dtype == MOE_BF16)
    hipLaunchKernelGGL(combine_bf16, dim3(grid), dim3(256), 0, c.stream, (const bf16_t*)y_perm, slot,
                       gate, s.T, s.k, s.d, (bf16_t*)y);
  else
    hipLaunchKernelGGL(combine_f32, dim3(grid), dim3(256), 0, c.stream, (const float*)y_perm, slot,
                       gate, s.T, s.k, s.d, (float*)y);
  return hipGetLastError();
}

}  // namespace moe
