// LoRA adapters on the expert up and down projections: rank-r projections for
// the forward and the four adapter gradients for the backward.
//
// "Adapting Trillion-Parameter MoE Models for LoRA Fine-Tuning: A Full-Stack
// Engineering Guide", §3: W' = W0 + (alpha/r) B A with W0 frozen, only the
// low-rank factors trained. With s = alpha/r and, for the rows of one expert,
// dO[p] = g_p dY[src_p], Z_u = X A_u^T, Z_d = H A_d^T:
//   db_down = s dO^T Z_d               da_down = s (dO B_d)^T H
//   dH = dO W_d + s (dO B_d) A_d,  dU = dH * silu(G)
//   db_up   = s dU^T Z_u               da_up   = s (dU B_u)^T X
//
// Kernels:
//   proj_mfma  the rank-r projections (Z_u, Z_d, dO B_d, dU B_u) on the matrix
//              cores, 16 dispatched rows per workgroup, K split over its
//              waves; fp32 out and/or s * (.) as bf16 high/low parts (the A
//              operand of the grouped GEMMs' extra adapter K step); several
//              independent projections in one launch
//   rowproj    the plain fallback (r > 16 or unaligned shapes): one wave per
//              row, fp32
//   transpose  [L, K, r] -> [L, r, K] (K-contiguous adapter rows for the
//              projections) and [L, r, N] -> [L, N, r] (the adapter rows of an
//              extra K step)
//   dh         the register-staged dH GEMM for unpacked W_d (the packed path
//              runs on the DMA engine in expert_gemm.hip): g dY W_d plus the
//              rank-r term, times silu(G) -> dU (fp32)
//   seg_mfma   per expert and 128 columns: sum over the expert's rows of
//              P[p, q] * V[p, c] -> the gradients, on the MFMAs for bf16 V
//              (rows staged per wave in LDS and read down the columns, P as
//              bf16 high + low parts), fixed-order reduction over the waves
//   seg_outer16  the same sums on the VALU for fp32 V (and shapes the MFMA
//              form does not take), 16 waves over the rows (seg_outer: the
//              plain fallback for r > 16)
#include <type_traits>

#include "common.h"
#include "mfma_tile.h"

namespace moe {

template <class TIn>
__device__ __forceinline__ void load8(const TIn* p, float (&v)[8]);
template <>
__device__ __forceinline__ void load8<bf16_t>(const bf16_t* p, float (&v)[8]) {
  const uint4 raw = *reinterpret_cast<const uint4*>(p);
  const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
  for (int u = 0; u < 8; ++u) v[u] = bf16_to_f32(static_cast<bf16_t>(w[u >> 1] >> ((u & 1) * 16)));
}
template <>
__device__ __forceinline__ void load8<float>(const float* p, float (&v)[8]) {
  const float4 a = *reinterpret_cast<const float4*>(p);
  const float4 b = *reinterpret_cast<const float4*>(p + 4);
  v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
  v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}

template <class TIn, int RMAX>
__global__ __launch_bounds__(256) void lora_rowproj(int L, const int32_t* __restrict__ offsets,
                                                    const TIn* __restrict__ in, int64_t in_stride,
                                                    const int32_t* __restrict__ src,
                                                    const float* __restrict__ row_scale, int K,
                                                    const bf16_t* __restrict__ M, int m_qk, int r,
                                                    float* __restrict__ out) {
  const int R = offsets[L];
  const int lane = threadIdx.x & 63;
  const int nwaves = gridDim.x * 4;
  for (int p = blockIdx.x * 4 + (threadIdx.x >> 6); p < R; p += nwaves) {
    const int le = segment_of(offsets, L, p);
    const int64_t srow = src ? src[p] : p;
    const float sc = row_scale ? row_scale[p] : 1.f;
    const TIn* x = in + srow * in_stride;
    const bf16_t* Mb = M + (int64_t)le * r * K;
    float acc[RMAX];
#pragma unroll
    for (int q = 0; q < RMAX; ++q) acc[q] = 0.f;
    for (int i0 = lane * 8; i0 < K; i0 += 512) {
      float xv[8];
      load8<TIn>(x + i0, xv);
      if (m_qk) {
#pragma unroll
        for (int q = 0; q < RMAX; ++q) {
          if (q >= r) break;
          float mv[8];
          load8<bf16_t>(Mb + (int64_t)q * K + i0, mv);
#pragma unroll
          for (int u = 0; u < 8; ++u) acc[q] = fmaf(xv[u], mv[u], acc[q]);
        }
      } else {
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const bf16_t* mrow = Mb + (int64_t)(i0 + u) * r;
#pragma unroll
          for (int q = 0; q < RMAX; ++q) {
            if (q >= r) break;
            acc[q] = fmaf(xv[u], bf16_to_f32(mrow[q]), acc[q]);
          }
        }
      }
    }
    float mine = 0.f;
#pragma unroll
    for (int q = 0; q < RMAX; ++q) {
      const float v = wave_sum(acc[q]);
      if (lane == q) mine = v;
    }
    if (lane < r) out[(int64_t)p * r + lane] = sc * mine;
  }
}

// Largest le with off[le] <= p (off[0] <= p < off[L]), wave-uniform: a
// binary search on scalar loads.
__device__ __forceinline__ int segment_of_uniform(const int32_t* off, int L, int p) {
  int lo = 0, hi = L;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (ld_uniform(off, mid) <= p) lo = mid; else hi = mid;
  }
  return lo;
}

// Eight consecutive K values of one row as an MFMA operand: bf16 as is; fp32
// split into a bf16 high part and the bf16 rounding of the remainder (their
// sum carries about 16 significant bits).
__device__ __forceinline__ void frag_load(const bf16_t* p, bf16x8& hi, bf16x8& lo) {
  hi = *reinterpret_cast<const bf16x8*>(p);
  (void)lo;
}
__device__ __forceinline__ void frag_load(const float* p, bf16x8& hi, bf16x8& lo) {
  const float4 a = *reinterpret_cast<const float4*>(p);
  const float4 b = *reinterpret_cast<const float4*>(p + 4);
  const float v[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
  uint32_t h[4], l[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    h[u] = f32x2_to_bf16x2(v[2 * u], v[2 * u + 1]);
    const float r0 = v[2 * u] - bf16_to_f32(static_cast<bf16_t>(h[u]));
    const float r1 = v[2 * u + 1] - bf16_to_f32(static_cast<bf16_t>(h[u] >> 16));
    l[u] = f32x2_to_bf16x2(r0, r1);
  }
  hi = __builtin_bit_cast(bf16x8, u32x4{h[0], h[1], h[2], h[3]});
  lo = __builtin_bit_cast(bf16x8, u32x4{l[0], l[1], l[2], l[3]});
}

// out[p, q] = scale_p * in[src_p] . Mt[le][q] for q < r <= 16 on the matrix
// cores. One workgroup per kProjRowGroups x 16 consecutive dispatched rows
// (the row fragments share each B fragment); its 8 waves take
// the K steps of 32 in turn (wave w: steps w, w + 8, ...) and their 16 x 16
// partial sums are added in wave order through LDS. A group that spans an
// expert boundary is computed once per expert it touches, each pass storing
// that expert's rows. Lane l supplies row l % 16 of the in-rows and of Mt
// (ranks) at K offset 8 (l / 16) and receives rows 4 (l / 16) + i, rank l % 16.
constexpr int kProjWaves = 8;
// 16-row groups per workgroup (sharing each B fragment load); two measured
// slower on the 14-expert LoRA step (fewer workgroups outweigh the halved
// adapter re-reads from L2)
constexpr int kProjRowGroups = 1;
#ifndef MOE_PROJ_U
#define MOE_PROJ_U 4
#endif

// One projection: out[p, q] = row_scale_p * in[src_p] . Mt[le(p)][q] (and
// out_hl, see launch_lora_rowproj).
template <class TIn>
struct ProjJob {
  const TIn* in;
  int64_t in_stride;
  const int32_t* src;
  const float* row_scale;
  int K;
  const bf16_t* Mt;
  float* out;
  bf16_t* out_hl;
  float hl_scale;
};
// NJ independent projections over the same dispatched rows in one launch
// (blockIdx.y selects the job), so they share the GPU instead of each
// leaving it partly idle.
template <class TIn, int NJ>
struct ProjJobs {
  ProjJob<TIn> j[NJ];
};

template <class TIn, int NJ>
__global__ __launch_bounds__(64 * kProjWaves) void lora_proj_mfma(int L, const int32_t* __restrict__ offsets, int r,
                                                                  ProjJobs<TIn, NJ> jobs) {
  constexpr bool kSplit = sizeof(TIn) == 4;
  constexpr int U = MOE_PROJ_U;  // K steps per load batch
  constexpr int RG = kProjRowGroups;
  __shared__ f32x4 part[kProjWaves][RG][64];
  const ProjJob<TIn>& jb = jobs.j[NJ == 1 ? 0 : blockIdx.y];
  const TIn* __restrict__ in = jb.in;
  const int64_t in_stride = jb.in_stride;
  const int32_t* __restrict__ src = jb.src;
  const float* __restrict__ row_scale = jb.row_scale;
  const int K = jb.K;
  const bf16_t* __restrict__ Mt = jb.Mt;
  float* __restrict__ out = jb.out;
  bf16_t* __restrict__ out_hl = jb.out_hl;
  const float hl_scale = jb.hl_scale;
  const int R = ld_uniform(offsets, L);
  const int p0 = blockIdx.x * 16 * RG;
  if (p0 >= R) return;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int row = lane & 15, kc = lane >> 4;
  const int le_first = segment_of_uniform(offsets, L, p0);
  const int le_last = segment_of_uniform(offsets, L, min(p0 + 16 * RG - 1, R - 1));
  const TIn* a_ptr[RG];
#pragma unroll
  for (int g = 0; g < RG; ++g) {
    const int prow = min(p0 + 16 * g + row, R - 1);
    const int64_t srow = src ? (int64_t)src[prow] : (int64_t)prow;
    a_ptr[g] = in + srow * in_stride + kc * 8;
  }
  const int nsteps = K / 32;
  for (int le = le_first; le <= le_last; ++le) {
    const int seg0 = ld_uniform(offsets, le), seg1 = ld_uniform(offsets, le + 1);
    if (seg0 == seg1) continue;  // wave-uniform
    const bf16_t* b_ptr = Mt + ((int64_t)le * r + min(row, r - 1)) * K + kc * 8;
    f32x4 acc[RG];
#pragma unroll
    for (int g = 0; g < RG; ++g) acc[g] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int s0 = wave; s0 < nsteps; s0 += kProjWaves * U) {
      bf16x8 ah[U][RG], al[U][RG], b[U];
#pragma unroll
      for (int j = 0; j < U; ++j) {
        const int st = s0 + kProjWaves * j;
        if (st < nsteps) {
          b[j] = *reinterpret_cast<const bf16x8*>(b_ptr + (int64_t)st * 32);
#pragma unroll
          for (int g = 0; g < RG; ++g) frag_load(a_ptr[g] + (int64_t)st * 32, ah[j][g], al[j][g]);
        }
      }
#pragma unroll
      for (int j = 0; j < U; ++j) {
        if (s0 + kProjWaves * j < nsteps) {
#pragma unroll
          for (int g = 0; g < RG; ++g) {
            acc[g] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah[j][g], b[j], acc[g], 0, 0, 0);
            if constexpr (kSplit) acc[g] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al[j][g], b[j], acc[g], 0, 0, 0);
          }
        }
      }
    }
#pragma unroll
    for (int g = 0; g < RG; ++g) part[wave][g][lane] = acc[g];
    __syncthreads();
    if (wave < RG) {  // wave g finishes row group g
      const int g = wave;
      f32x4 t = part[0][g][lane];
#pragma unroll
      for (int w = 1; w < kProjWaves; ++w) t += part[w][g][lane];
      const int q = lane & 15;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int p = p0 + 16 * g + 4 * kc + i;
        if (q < r && p >= seg0 && p < seg1) {
          if (out_hl) {
            // hl_scale t (before the row scale) as a bf16 high part and the
            // bf16 rounding of the rest
            const float sv = hl_scale * t[i];
            const bf16_t hi = f32_to_bf16(sv);
            out_hl[(int64_t)p * 2 * r + q] = hi;
            out_hl[(int64_t)p * 2 * r + r + q] = f32_to_bf16(sv - bf16_to_f32(hi));
          }
          if (out) out[(int64_t)p * r + q] = (row_scale ? row_scale[p] : 1.f) * t[i];
        }
      }
    }
    __syncthreads();
  }
}

// At[le][n][q] = A[le][q][n]: an [L, r, N] adapter as [L, N, r] rows (the
// B operand of an extra adapter K step).
__global__ __launch_bounds__(256) void lora_transpose_rn(const bf16_t* __restrict__ A, int L, int r, int N,
                                                         bf16_t* __restrict__ At) {
  const int64_t id = (int64_t)blockIdx.x * 256 + threadIdx.x;  // over L * r * N, N fastest
  if (id >= (int64_t)L * r * N) return;
  const int64_t n = id % N, q = (id / N) % r, le = id / ((int64_t)N * r);
  At[(le * N + n) * r + q] = A[id];
}

hipError_t launch_lora_transpose_rn(const Ctx& c, const bf16_t* A, int L, int r, int N, bf16_t* At) {
  const int64_t n = (int64_t)L * r * N;
  if (n == 0) return hipSuccess;
  TimedLaunch tl(MOE_K_LORA_PROJ, c.stream);
  hipLaunchKernelGGL(lora_transpose_rn, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, c.stream, A, L, r, N, At);
  return hipGetLastError();
}

// Mt[le][q][k] = M[le][k][q]: a [L, K, r] adapter made K-contiguous.
__global__ __launch_bounds__(256) void lora_transpose_kr(const bf16_t* __restrict__ M, int L, int K, int r,
                                                         bf16_t* __restrict__ Mt) {
  const int64_t id = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (id >= (int64_t)L * K) return;
  const int64_t le = id / K, k = id % K;
  for (int q = 0; q < r; ++q) Mt[(le * r + q) * K + k] = M[id * r + q];
}

// The adapter backward's three re-layouts in one launch (blockIdx.y picks
// the job, threads past a job's rows return): B_d [L, d, r] and B_u [L, f, r]
// made K-contiguous ([L, r, d], [L, r, f]) for the projections dO B_d and
// dU B_u, and, with ad_t, A_d [L, r, f] as [L, f, r] rows for the dH
// product's extra K step. One thread per adapter row (le, k): its r values
// are contiguous on the [., r] side, read or written as 16-byte vectors when
// r = 16 and the rows are 16-byte aligned, and strided by K on the other
// side, where consecutive threads touch consecutive elements.
__global__ __launch_bounds__(256) void lora_transpose_bwd(const bf16_t* __restrict__ bd, const bf16_t* __restrict__ bu,
                                                          const bf16_t* __restrict__ ad, int L, int d, int f, int r,
                                                          bf16_t* __restrict__ bd_t, bf16_t* __restrict__ bu_t,
                                                          bf16_t* __restrict__ ad_t) {
  const int64_t id = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int K = blockIdx.y == 0 ? d : f;
  if (id >= (int64_t)L * K) return;
  const int64_t le = id / K, k = id % K;
  if (blockIdx.y < 2) {  // [le][k][q] -> [le][q][k]
    const bf16_t* M = blockIdx.y == 0 ? bd : bu;
    bf16_t* Mt = blockIdx.y == 0 ? bd_t : bu_t;
    if (r == 16 && (reinterpret_cast<uintptr_t>(M) & 15) == 0) {
      const uint4 v0 = reinterpret_cast<const uint4*>(M + id * 16)[0];
      const uint4 v1 = reinterpret_cast<const uint4*>(M + id * 16)[1];
      const uint32_t w[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
#pragma unroll
      for (int q = 0; q < 16; ++q)
        Mt[(le * 16 + q) * K + k] = static_cast<bf16_t>(w[q >> 1] >> (16 * (q & 1)));
    } else {
      for (int q = 0; q < r; ++q) Mt[(le * r + q) * K + k] = M[id * r + q];
    }
    return;
  }
  if (!ad_t) return;  // [le][q][n] -> [le][n][q], n = k < f
  if (r == 16 && (reinterpret_cast<uintptr_t>(ad_t) & 15) == 0) {
    uint32_t w[8];
#pragma unroll
    for (int q2 = 0; q2 < 8; ++q2)
      w[q2] = (uint32_t)ad[(le * 16 + 2 * q2) * f + k] | ((uint32_t)ad[(le * 16 + 2 * q2 + 1) * f + k] << 16);
    reinterpret_cast<uint4*>(ad_t + id * 16)[0] = make_uint4(w[0], w[1], w[2], w[3]);
    reinterpret_cast<uint4*>(ad_t + id * 16)[1] = make_uint4(w[4], w[5], w[6], w[7]);
  } else {
    for (int q = 0; q < r; ++q) ad_t[id * r + q] = ad[(le * r + q) * f + k];
  }
}

template <class TIn>
hipError_t launch_lora_rowproj(const Ctx& c, int L, const int32_t* offsets, int64_t rmax_rows,
                               const TIn* in, int64_t in_stride, const int32_t* src,
                               const float* row_scale, int K, const bf16_t* M, bool m_qk, int r,
                               float* out, bf16_t* mt, bf16_t* out_hl, float hl_scale) {
  if (rmax_rows <= 0) return hipSuccess;
  if (r <= 16 && K % 32 == 0 && in_stride % 8 == 0 && (m_qk || mt)) {
    TimedLaunch tl(MOE_K_LORA_PROJ, c.stream);
    if (!m_qk) {
      const int64_t n = (int64_t)L * K;
      hipLaunchKernelGGL(lora_transpose_kr, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, c.stream, M, L, K, r,
                         mt);
      M = mt;
    }
    ProjJobs<TIn, 1> jobs{{{in, in_stride, src, row_scale, K, M, out, out_hl, hl_scale}}};
    hipLaunchKernelGGL((lora_proj_mfma<TIn, 1>), dim3((unsigned)((rmax_rows + 16 * kProjRowGroups - 1) /
                                                                  (16 * kProjRowGroups))),
                       dim3(64 * kProjWaves), 0,
                       c.stream, L, offsets, r, jobs);
    return hipGetLastError();
  }
  if (out_hl) return hipErrorInvalidValue;  // the high/low output exists on the matrix-core path only
  const int64_t want = (rmax_rows + 3) / 4;
  const int grid = (int)(want < (int64_t)c.num_cus * 8 ? (want > 0 ? want : 1) : (int64_t)c.num_cus * 8);
  TimedLaunch tl(MOE_K_LORA_PROJ, c.stream);
#define MOE_RP(N)                                                                          \
  hipLaunchKernelGGL((lora_rowproj<TIn, N>), dim3(grid), dim3(256), 0, c.stream, L, offsets, in, \
                     in_stride, src, row_scale, K, M, (int)m_qk, r, out)
  if (r <= 16) MOE_RP(16);
  else if (r <= 32) MOE_RP(32);
  else MOE_RP(64);
#undef MOE_RP
  return hipGetLastError();
}

template hipError_t launch_lora_rowproj<bf16_t>(const Ctx&, int, const int32_t*, int64_t,
                                                const bf16_t*, int64_t, const int32_t*,
                                                const float*, int, const bf16_t*, bool, int, float*,
                                                bf16_t*, bf16_t*, float);
template hipError_t launch_lora_rowproj<float>(const Ctx&, int, const int32_t*, int64_t,
                                               const float*, int64_t, const int32_t*, const float*,
                                               int, const bf16_t*, bool, int, float*, bf16_t*, bf16_t*,
                                               float);

// out[le] = s * sum_{p in rows of le} P[p, q] * qscale_p * in[qsrc_p, c], for
// q < r, c < C; stored [L, r, C] (out_qc) or [L, C, r].
template <class TIn, int RMAX>
__global__ __launch_bounds__(256) void lora_seg_outer(const int32_t* __restrict__ offsets,
                                                      const float* __restrict__ P, int r,
                                                      const TIn* __restrict__ in, int64_t in_stride,
                                                      const int32_t* __restrict__ qsrc,
                                                      const float* __restrict__ qscale, int C,
                                                      float s, int out_qc, float* __restrict__ out) {
  constexpr int CH = 64;
  __shared__ float sp[CH][RMAX];
  __shared__ float ssc[CH];
  __shared__ int64_t ssrc[CH];
  const int le = blockIdx.y;
  const int c = blockIdx.x * 256 + threadIdx.x;
  const int a = offsets[le], b = offsets[le + 1];
  float acc[RMAX];
#pragma unroll
  for (int q = 0; q < RMAX; ++q) acc[q] = 0.f;
  for (int p0 = a; p0 < b; p0 += CH) {
    const int n = min(CH, b - p0);
    for (int i = threadIdx.x; i < n * r; i += 256) sp[i / r][i % r] = P[(int64_t)(p0 + i / r) * r + i % r];
    if (threadIdx.x < n) {
      const int p = p0 + threadIdx.x;
      ssc[threadIdx.x] = qscale ? qscale[p] : 1.f;
      ssrc[threadIdx.x] = qsrc ? (int64_t)qsrc[p] : (int64_t)p;
    }
    __syncthreads();
    if (c < C) {
      for (int pp = 0; pp < n; ++pp) {
        const float v = ssc[pp] * load_f<TIn>(in + ssrc[pp] * in_stride + c);
#pragma unroll
        for (int q = 0; q < RMAX; ++q)
          if (q < r) acc[q] = fmaf(sp[pp][q], v, acc[q]);
      }
    }
    __syncthreads();
  }
  if (c >= C) return;
#pragma unroll
  for (int q = 0; q < RMAX; ++q) {
    if (q >= r) break;
    if (out_qc) out[((int64_t)le * r + q) * C + c] = s * acc[q];
    else out[((int64_t)le * C + c) * r + q] = s * acc[q];
  }
}

// Same sums for r <= 16 and C % 4 == 0, with the rows spread over the
// workgroup: one workgroup per (64 CPL columns, expert), 16 waves, wave w
// taking the expert's rows w, w + 16, ... in order, each lane CPL
// consecutive columns x 16 ranks in registers. Rows go in batches of 8 (4
// for fp32 rows of 4 columns): a batch's loads (its rows of `in`, kept as
// loaded until their FMAs, and its P values, one per lane per 4 rows) are
// issued before the previous batch's FMAs; the source rows and row scales
// come 64 rows at a time in one vector load and are read per row with
// readlane. The 16 waves' partial sums are then added in a fixed tree order
// through LDS, so the result does not depend on timing.
typedef const __attribute__((address_space(4))) float* const_f32_ptr_t;

// N consecutive values (N = 1, 2 or 4) in one load, as floats.
template <int N>
__device__ __forceinline__ void load_vec(const bf16_t* p, float (&v)[N]) {
  if constexpr (N == 4) {
    const uint2 raw = *reinterpret_cast<const uint2*>(p);
    v[0] = bf16_to_f32(static_cast<bf16_t>(raw.x));
    v[1] = bf16_to_f32(static_cast<bf16_t>(raw.x >> 16));
    v[2] = bf16_to_f32(static_cast<bf16_t>(raw.y));
    v[3] = bf16_to_f32(static_cast<bf16_t>(raw.y >> 16));
  } else if constexpr (N == 2) {
    const uint32_t raw = *reinterpret_cast<const uint32_t*>(p);
    v[0] = bf16_to_f32(static_cast<bf16_t>(raw));
    v[1] = bf16_to_f32(static_cast<bf16_t>(raw >> 16));
  } else {
    v[0] = bf16_to_f32(*p);
  }
}
template <int N>
__device__ __forceinline__ void load_vec(const float* p, float (&v)[N]) {
  if constexpr (N == 4) {
    const float4 a = *reinterpret_cast<const float4*>(p);
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
  } else if constexpr (N == 2) {
    const float2 a = *reinterpret_cast<const float2*>(p);
    v[0] = a.x; v[1] = a.y;
  } else {
    v[0] = *p;
  }
}

// CPL consecutive row values as loaded (bf16 words, or fp32), widened one
// at a time where they are used.
template <class TIn, int N>
struct RawVec;
template <int N>
struct RawVec<bf16_t, N> {
  uint32_t w[(N + 1) / 2];
  __device__ __forceinline__ void load(const bf16_t* p) {
    if constexpr (N == 4) {
      const uint2 raw = *reinterpret_cast<const uint2*>(p);
      w[0] = raw.x;
      w[1] = raw.y;
    } else if constexpr (N == 2) {
      w[0] = *reinterpret_cast<const uint32_t*>(p);
    } else {
      w[0] = static_cast<uint32_t>(*p);
    }
  }
  __device__ __forceinline__ void zero() {
#pragma unroll
    for (int i = 0; i < (N + 1) / 2; ++i) w[i] = 0u;
  }
  __device__ __forceinline__ float at(int u) const {
    const uint32_t x = w[u >> 1];
    return __uint_as_float((u & 1) ? (x & 0xffff0000u) : (x << 16));
  }
};
template <int N>
struct RawVec<float, N> {
  float v[N];
  __device__ __forceinline__ void load(const float* p) { load_vec<N>(p, v); }
  __device__ __forceinline__ void zero() {
#pragma unroll
    for (int i = 0; i < N; ++i) v[i] = 0.f;
  }
  __device__ __forceinline__ float at(int u) const { return v[u]; }
};

constexpr int kSegWaves = 16;  // waves per workgroup
constexpr int kSegRq = 16;     // ranks held per lane
constexpr int kSegSlots = 8;   // LDS partial-sum slots of the reduction tree

// CPL columns per lane (1, 2 or 4), 64 CPL per workgroup: fewer columns per
// lane for narrow C, so that enough workgroups share the work.
template <class TIn, int CPL>
__global__ __launch_bounds__(64 * kSegWaves) void lora_seg_outer16(
    const int32_t* __restrict__ offsets, const float* __restrict__ P, int r, const TIn* __restrict__ in,
    int64_t in_stride, const int32_t* __restrict__ qsrc, const float* __restrict__ qscale, int C, float s,
    int out_qc, float* __restrict__ out) {
  // rows per batch: 8, or 4 where 8 fp32 rows of 4 columns would not fit in
  // registers; NH groups of 4 rows x 16 ranks of P per batch
  constexpr int B = (sizeof(TIn) == 4 && CPL == 4) ? 4 : 8;
  constexpr int NH = B / 4;
  constexpr int kSegCols = 64 * CPL;
  __shared__ float red[kSegSlots][kSegRq][kSegCols];
  const int le = blockIdx.y;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int cb = blockIdx.x * kSegCols;
  const int c0 = cb + lane * CPL;
  const bool cok = c0 < C;
  const int a = ld_uniform(offsets, le), b = ld_uniform(offsets, le + 1);
  // this wave's rows: a + wave + kSegWaves m, m < M
  const int M = b - a > wave ? (b - a - wave + kSegWaves - 1) / kSegWaves : 0;
  float acc[kSegRq][CPL];
#pragma unroll
  for (int q = 0; q < kSegRq; ++q)
#pragma unroll
    for (int u = 0; u < CPL; ++u) acc[q][u] = 0.f;
  // P values this lane fetches: rows jp + 4 h of a batch, rank qp
  const int jp = lane >> 4, qp = lane & 15;
  int srcv = 0;      // lane l: source row of window row l (64 rows per window)
  float sclv = 1.f;  // lane l: its scale
  RawVec<TIn, CPL> vc[B], vn[B];
  float sc_c[B], sc_n[B];  // row scales of the two batches (1 past M)
  float pc[NH], pn[NH];
#pragma unroll
  for (int h = 0; h < NH; ++h) pc[h] = pn[h] = 0.f;
  for (int m0 = 0; m0 < M + B; m0 += B) {
    // fetch batch m0 (if any) into (vn, pn) while batch m0 - B, in (vc, pc), is consumed
    if (m0 < M) {
      if ((m0 & 63) == 0) {
        const int m = m0 + lane;
        const int p = a + wave + kSegWaves * m;
        srcv = m < M ? (qsrc ? qsrc[p] : p) : 0;
        sclv = (m < M && qscale) ? qscale[p] : 1.f;
      }
#pragma unroll
      for (int h = 0; h < NH; ++h) {
        const int mp = m0 + jp + 4 * h;
        pn[h] = (mp < M && qp < r) ? P[(int64_t)(a + wave + kSegWaves * mp) * r + qp] : 0.f;
      }
#pragma unroll
      for (int j = 0; j < B; ++j) {
        const int src = __builtin_amdgcn_readlane(srcv, (m0 + j) & 63);
        if (m0 + j < M && cok) vn[j].load(in + (int64_t)src * in_stride + c0);
        else vn[j].zero();
        // rows past M have scale 1 and zeros
        sc_n[j] = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, sclv),
                                                                      (m0 + j) & 63));
      }
    }
    if (m0 > 0) {
#pragma unroll
      for (int j = 0; j < B; ++j) {
        float v[CPL];
#pragma unroll
        for (int u = 0; u < CPL; ++u) v[u] = vc[j].at(u) * sc_c[j];
#pragma unroll
        for (int q = 0; q < kSegRq; ++q) {
          const float pq = __builtin_bit_cast(
              float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, pc[j >> 2]), 16 * (j & 3) + q));
#pragma unroll
          for (int u = 0; u < CPL; ++u) acc[q][u] = fmaf(pq, v[u], acc[q][u]);
        }
      }
    }
#pragma unroll
    for (int j = 0; j < B; ++j) {
      vc[j] = vn[j];
      sc_c[j] = sc_n[j];
    }
#pragma unroll
    for (int h = 0; h < NH; ++h) pc[h] = pn[h];
  }
  // fixed-order tree over the waves: 16 -> 8 -> 4 -> 2 -> 1
  for (int half = kSegWaves / 2; half >= 1; half >>= 1) {
    if (wave >= half && wave < 2 * half) {
#pragma unroll
      for (int q = 0; q < kSegRq; ++q)
#pragma unroll
        for (int u = 0; u < CPL; ++u) red[wave - half][q][lane * CPL + u] = acc[q][u];
    }
    __syncthreads();
    if (wave < half) {
#pragma unroll
      for (int q = 0; q < kSegRq; ++q)
#pragma unroll
        for (int u = 0; u < CPL; ++u) acc[q][u] += red[wave][q][lane * CPL + u];
    }
    __syncthreads();
  }
  if (wave != 0 || !cok) return;
  if (out_qc) {
#pragma unroll
    for (int q = 0; q < kSegRq; ++q)
      if (q < r)
#pragma unroll
        for (int u = 0; u < CPL; ++u) out[((int64_t)le * r + q) * C + c0 + u] = s * acc[q][u];
  } else {
#pragma unroll
    for (int u = 0; u < CPL; ++u)
#pragma unroll
      for (int q = 0; q < kSegRq; ++q)
        if (q < r) out[((int64_t)le * C + c0 + u) * r + q] = s * acc[q][u];
  }
}

// The same sums on the matrix cores for bf16 rows, r <= 16 and C % 128 == 0:
// out[le] = s * sum over the expert's rows p of (scale_p P[p])^T in[src_p],
// as [r x 32] . [32 x kSmCols] MFMA products per step of 32 rows. One
// workgroup per (kSmCols columns, expert), kSmWaves waves, wave w taking the
// steps w, w + kSmWaves, ... A step's rows are staged in the wave's own LDS
// tile (32 x kSmCols bf16, each 16-byte chunk c of row j at chunk
// c ^ 2 (j / 8 % 4), so the column reads below hit 32 different banks); the
// B operand is read from it down the columns (8 rows of one column per
// lane), the A operand is the scaled P values split into bf16 high and low
// parts (two MFMAs, about 16 bits of P). The waves' 16 x kSmCols partial
// sums are then added in a fixed tree order through LDS, so the result does
// not depend on timing.
// 8 waves x 128 columns (two workgroups per CU) measured fastest on the
// 14-expert LoRA step; 8 x 256, 16 x 128, 8 x 64 and 4 x 128 were slower.
constexpr int kSmWaves = 8;
constexpr int kSmCols = 128;
constexpr int kSmFrags = kSmCols / 16;  // 16-column MFMA fragments
constexpr int kSmChunks = kSmCols / 8;  // 16-byte chunks per tile row

static_assert(kSmWaves * 32 * kSmCols * 2 <= 160 * 1024, "LDS tiles");
static_assert(kSmChunks <= 64 && kSmCols % 64 == 0, "tile rows");

// One gradient sum: out = s * sum over rows p (qscale_p P[p])^T in[qsrc_p]
// per expert, [L, r, C] (out_qc) or [L, C, r].
struct SegJob {
  const float* P;
  const bf16_t* in;
  int64_t in_stride;
  const int32_t* qsrc;
  const float* qscale;
  int C, out_qc;
  float* out;
};
// NJ independent sums over the same experts in one launch (blockIdx.z picks
// the job; workgroups past a job's columns return), so their latencies
// overlap instead of adding up.
template <int NJ>
struct SegJobs {
  SegJob j[NJ];
};

template <int NJ>
__global__ __launch_bounds__(64 * kSmWaves) void lora_seg_mfma(const int32_t* __restrict__ offsets, int r, float s,
                                                               SegJobs<NJ> jobs) {
  __shared__ __align__(16) bf16_t tile[kSmWaves * 32 * kSmCols];
  const SegJob& jb = jobs.j[NJ == 1 ? 0 : blockIdx.z];
  const float* __restrict__ P = jb.P;
  const bf16_t* __restrict__ in = jb.in;
  const int64_t in_stride = jb.in_stride;
  const int32_t* __restrict__ qsrc = jb.qsrc;
  const float* __restrict__ qscale = jb.qscale;
  const int C = jb.C, out_qc = jb.out_qc;
  float* __restrict__ out = jb.out;
  const int le = blockIdx.y;
  const int cb = blockIdx.x * kSmCols;
  if (cb >= C) return;  // workgroup-uniform, before any barrier
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int a = ld_uniform(offsets, le), b = ld_uniform(offsets, le + 1);
  const int nsteps = (b - a + 31) / 32;
  const int q = lane & 15, kg = lane >> 4;  // MFMA lane roles: row / column q, K group kg
  f32x4 acc[kSmFrags];
#pragma unroll
  for (int n = 0; n < kSmFrags; ++n) acc[n] = f32x4{0.f, 0.f, 0.f, 0.f};
  bf16_t* my = tile + wave * 32 * kSmCols;
  for (int st = wave; st < nsteps; st += kSmWaves) {
    const int p0 = a + st * 32;
    // lane l holds the source row of step row l % 32 (rows past the expert:
    // its last row, whose P values below are 0)
    const int pl = min(p0 + (lane & 31), b - 1);
    const int srcl = qsrc ? qsrc[pl] : pl;
    // this lane's chunks: rows (64 / kSmChunks) t + lane / kSmChunks, 8
    // columns at chunk lane % kSmChunks
    constexpr int RPT = 64 / kSmChunks, NT = 32 / RPT;
    uint4 v[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const int srow = __shfl(srcl, RPT * t + lane / kSmChunks, kWave);
      v[t] = *reinterpret_cast<const uint4*>(in + (int64_t)srow * in_stride + cb + (lane % kSmChunks) * 8);
    }
    // A: rank q of rows p0 + 8 kg + i, times the row scale, as bf16 hi + lo
    float pv[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int p = p0 + 8 * kg + i;
      pv[i] = (p < b && q < r) ? P[(int64_t)p * r + q] * (qscale ? qscale[p] : 1.f) : 0.f;
    }
    uint32_t h[4], l[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      h[u] = f32x2_to_bf16x2(pv[2 * u], pv[2 * u + 1]);
      l[u] = f32x2_to_bf16x2(pv[2 * u] - bf16_to_f32(static_cast<bf16_t>(h[u])),
                             pv[2 * u + 1] - bf16_to_f32(static_cast<bf16_t>(h[u] >> 16)));
    }
    const bf16x8 ah = __builtin_bit_cast(bf16x8, u32x4{h[0], h[1], h[2], h[3]});
    const bf16x8 al = __builtin_bit_cast(bf16x8, u32x4{l[0], l[1], l[2], l[3]});
    // (the previous step's reads of the tile precede these writes: one
    // wave's LDS accesses complete in order)
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const int row = RPT * t + lane / kSmChunks, cc = lane % kSmChunks;
      *reinterpret_cast<uint4*>(my + row * kSmCols + ((cc ^ (2 * ((row >> 3) & 3))) * 8)) = v[t];
    }
#pragma unroll
    for (int n = 0; n < kSmFrags; ++n) {
      // column 16 n + q, rows 8 kg .. 8 kg + 7 (their chunk key is kg)
      const int col = ((((2 * n + (q >> 3)) ^ (2 * kg))) * 8) + (q & 7);
      uint32_t w[4];
#pragma unroll
      for (int i2 = 0; i2 < 4; ++i2) {
        const uint32_t lo = my[(8 * kg + 2 * i2) * kSmCols + col];
        const uint32_t hi = my[(8 * kg + 2 * i2 + 1) * kSmCols + col];
        w[i2] = lo | (hi << 16);
      }
      const bf16x8 bv = __builtin_bit_cast(bf16x8, u32x4{w[0], w[1], w[2], w[3]});
      acc[n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bv, acc[n], 0, 0, 0);
      acc[n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al, bv, acc[n], 0, 0, 0);
    }
  }
  // fixed-order tree over the waves, halving (the tiles reused: half the
  // waves x 64 kSmFrags floats per lane)
  constexpr int kRed = kSmFrags * 4 * 64;
  static_assert((kSmWaves / 2) * kRed * 4 <= kSmWaves * 32 * kSmCols * 2, "reduction fits the tiles");
  float* red = reinterpret_cast<float*>(tile);
  __syncthreads();
  for (int half = kSmWaves / 2; half >= 1; half >>= 1) {
    if (wave >= half && wave < 2 * half) {
#pragma unroll
      for (int n = 0; n < kSmFrags; ++n)
#pragma unroll
        for (int j = 0; j < 4; ++j) red[(wave - half) * kRed + (n * 4 + j) * 64 + lane] = acc[n][j];
    }
    __syncthreads();
    if (wave < half) {
#pragma unroll
      for (int n = 0; n < kSmFrags; ++n)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[n][j] += red[wave * kRed + (n * 4 + j) * 64 + lane];
    }
    __syncthreads();
  }
  if (wave != 0) return;
  // lane: column cb + 16 n + q, ranks 4 kg + j
#pragma unroll
  for (int n = 0; n < kSmFrags; ++n)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int qo = 4 * kg + j, c = cb + 16 * n + q;
      if (qo < r) {
        if (out_qc) out[((int64_t)le * r + qo) * C + c] = s * acc[n][j];
        else out[((int64_t)le * C + c) * r + qo] = s * acc[n][j];
      }
    }
}

// The MFMA form takes bf16 rows, r <= 16, whole 128-column blocks and
// 16-byte aligned rows.
static bool seg_mfma_ok(int r, const bf16_t* in, int64_t in_stride, int C) {
  return r <= 16 && C % kSmCols == 0 && in_stride % 8 == 0 && (reinterpret_cast<uintptr_t>(in) & 15) == 0;
}

template <class TIn>
static hipError_t launch_seg_outer(const Ctx& c, int L, const int32_t* offsets, const float* P,
                                   int r, const TIn* in, int64_t in_stride, const int32_t* qsrc,
                                   const float* qscale, int C, float s, bool out_qc, float* out) {
  if constexpr (std::is_same<TIn, bf16_t>::value) {
    if (seg_mfma_ok(r, in, in_stride, C)) {
      TimedLaunch tl(MOE_K_LORA_GRAD, c.stream);
      SegJobs<1> jobs{{{P, in, in_stride, qsrc, qscale, C, (int)out_qc, out}}};
      hipLaunchKernelGGL((lora_seg_mfma<1>), dim3(C / kSmCols, L), dim3(64 * kSmWaves), 0, c.stream, offsets, r, s,
                         jobs);
      return hipGetLastError();
    }
  }
  if (r <= kSegRq && C % 4 == 0 && in_stride % 4 == 0) {
    TimedLaunch tl(MOE_K_LORA_GRAD, c.stream);
    // columns per lane: the widest that still gives about 200 workgroups
    const int64_t want = 200;
    const int cpl = (int64_t)((C + 255) / 256) * L >= want ? 4 : (int64_t)((C + 127) / 128) * L >= want ? 2 : 1;
#define MOE_SEG(N)                                                                                        \
  hipLaunchKernelGGL((lora_seg_outer16<TIn, N>), dim3((C + 64 * N - 1) / (64 * N), L), dim3(64 * kSegWaves), 0, \
                     c.stream, offsets, P, r, in, in_stride, qsrc, qscale, C, s, (int)out_qc, out)
    if (cpl == 4) MOE_SEG(4);
    else if (cpl == 2) MOE_SEG(2);
    else MOE_SEG(1);
#undef MOE_SEG
    return hipGetLastError();
  }
  dim3 grid((C + 255) / 256, L);
  TimedLaunch tl(MOE_K_LORA_GRAD, c.stream);
#define MOE_SO(N)                                                                             \
  hipLaunchKernelGGL((lora_seg_outer<TIn, N>), grid, dim3(256), 0, c.stream, offsets, P, r, in, \
                     in_stride, qsrc, qscale, C, s, (int)out_qc, out)
  if (r <= 16) MOE_SO(16);
  else if (r <= 32) MOE_SO(32);
  else MOE_SO(64);
#undef MOE_SO
  return hipGetLastError();
}

// dU[row, n] = (g_row * (dY[src_row] . W_d[:, n]) + s * wproj[row] . A_d[:, n])
//              * silu(G[row, n]), per (row tile, 128 FFN columns) item.
template <class Cfg>
struct DhProb {
  const bf16_t* dy;
  const int32_t* row_src;
  const float* row_gate;
  const int32_t* offsets;
  const int32_t* tiles;
  const bf16_t* w_down;
  int d, f, nt;
  const float* wproj;
  const bf16_t* a_down;
  int r;
  float s;
  const bf16_t* act_save;
  float* du;

  __device__ __forceinline__ void setup(int item, LoaderNN<Cfg>& ld) const {
    const int ti = item / nt, n0 = (item % nt) * Cfg::BN;
    const int le = ld_uniform(tiles, 2 * ti), r0 = ld_uniform(tiles, 2 * ti + 1);
    const int seg = ld_uniform(offsets, le);
    const int valid = min(Cfg::BM, ld_uniform(offsets, le + 1) - seg - r0);
    const int lrow = threadIdx.x / Cfg::CHUNKS_PER_ROW, lcol = (threadIdx.x % Cfg::CHUNKS_PER_ROW) * 8;
#pragma unroll
    for (int i = 0; i < Cfg::A_LOADS; ++i) {
      const int64_t row = (int64_t)seg + r0 + min(lrow + i * Cfg::ROWS_PER_PASS, valid - 1);
      ld.a[i] = dy + (int64_t)row_src[row] * d + lcol;
    }
    ld.b_base = w_down + (int64_t)le * d * f + n0;
    ld.ldb = f;
    ld.n_valid = min(Cfg::BN, f - n0);
  }

  __device__ __forceinline__ void epilogue(int item, Acc<Cfg>& acc) const {
    const int ti = item / nt, n0 = (item % nt) * Cfg::BN;
    const int le = ld_uniform(tiles, 2 * ti), r0 = ld_uniform(tiles, 2 * ti + 1);
    const int seg = ld_uniform(offsets, le);
    const int valid = min(Cfg::BM, ld_uniform(offsets, le + 1) - seg - r0);
    const int64_t row0 = (int64_t)seg + r0;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int wm = wave >> 1, wn = wave & 1;
#pragma unroll
    for (int j = 0; j < Cfg::FN; ++j) {
      const int n = n0 + frag_col<Cfg>(wn, j, lane);
      if (n >= f) continue;
#pragma unroll
      for (int i = 0; i < Cfg::FM; ++i)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int rin = frag_row<Cfg>(wm, i, lane, q);
          if (rin >= valid) continue;
          const int64_t row = row0 + rin;
          float t = 0.f;
          const float* w = wproj + row * r;
          const bf16_t* ad = a_down + (int64_t)le * r * f + n;
          for (int c = 0; c < r; ++c) t = fmaf(w[c], bf16_to_f32(ad[(int64_t)c * f]), t);
          const float dh = fmaf(row_gate[row], acc.v[i][j][q], s * t);
          const float g = bf16_to_f32(act_save[row * 3 * f + n]);
          du[row * f + n] = dh * silu_f(g);
        }
    }
  }
};

template <class Cfg>
__global__ __launch_bounds__(256, 2) void lora_dh_bf16(DhProb<Cfg> pb, int max_tiles) {
  extern __shared__ __align__(16) unsigned char smem_raw[];
  const int items = ld_uniform(pb.tiles, 2 * max_tiles) * pb.nt;
  persistent_gemm<Cfg, LoaderNN<Cfg>>(pb, items, pb.d / Cfg::BK, reinterpret_cast<bf16_t*>(smem_raw));
}

hipError_t launch_lora_bwd(const Ctx& c, const moe_shape_t& sh, const Workspace& ws,
                           const LoraArgs& lo, const bf16_t* dy, const int32_t* offsets,
                           const int32_t* row_src, const float* row_gate, const bf16_t* x_rows,
                           const int32_t* x_src, const bf16_t* act_save, const bf16_t* w_down, float* da_up,
                           float* db_up, float* da_down, float* db_down, const bf16_t* dgu_packed) {
  using Cfg = TileCfg<kGemmBM, 128>;
  const int L = sh.e_hi - sh.e_lo;
  const int d = sh.d, f = sh.f, r = lo.r;
  const int64_t rmax = max_rows(sh);
  const int max_tiles = gemm_max_tiles(sh);
  const bf16_t* H = act_save + f;  // rows of stride 3f (G | H | U)
  // Z_u, Z_d: kept by the forward in z_save, else projected here
  const bool have_z = lo.z_save != nullptr;
  float* zu = have_z ? lo.z_save : ws.zu;
  float* zd = have_z ? lo.z_save + rmax * r : ws.zd;
  hipError_t err;
#define MOE_TRY(x) \
  if ((err = (x)) != hipSuccess) return err
  MOE_TRY(launch_row_tiles(c, offsets, L, max_tiles, ws.gemm_tiles));
  // Z_u = X A_u^T, Z_d = H A_d^T, and dO B_d (row-scaled, fp32) plus, for the
  // packed dH product's extra K step, s dY B_d as bf16 high/low parts (the
  // row gate scales the whole dH there)
  const bool kx = dgu_packed && lo.r == 16 && ws.zx;
  // on the matrix-core path all three adapter re-layouts (B_d and B_u
  // K-contiguous, A_d as rows of the extra K step) go first, in one launch
  const bool mt_all = rmax > 0 && r <= 16 && d % 32 == 0 && f % 32 == 0 && ws.lora_mt && ws.lora_mt2 && ws.lora_mt3;
  if (mt_all) {
    TimedLaunch tl(MOE_K_LORA_PROJ, c.stream);
    const int64_t n = (int64_t)L * std::max(d, f);
    hipLaunchKernelGGL(lora_transpose_bwd, dim3((unsigned)((n + 255) / 256), 3), dim3(256), 0, c.stream, lo.b_down,
                       lo.b_up, lo.a_down, L, d, f, r, ws.lora_mt, ws.lora_mt2, kx ? ws.lora_mt3 : nullptr);
    MOE_TRY(hipGetLastError());
  }
  if (mt_all) {
    // the three projections are independent: one launch
    const ProjJob<bf16_t> j_dob{dy, d, row_src, row_gate, d, ws.lora_mt, ws.wproj, kx ? ws.zx : nullptr, lo.scale};
    const unsigned gx = (unsigned)((rmax + 16 * kProjRowGroups - 1) / (16 * kProjRowGroups));
    TimedLaunch tl(MOE_K_LORA_PROJ, c.stream);
    if (have_z) {
      ProjJobs<bf16_t, 1> jobs{{j_dob}};
      hipLaunchKernelGGL((lora_proj_mfma<bf16_t, 1>), dim3(gx), dim3(64 * kProjWaves), 0, c.stream, L, offsets, r,
                         jobs);
    } else {
      ProjJobs<bf16_t, 3> jobs{{{x_rows, d, x_src, nullptr, d, lo.a_up, zu, nullptr, 1.f},
                                {H, 3 * f, nullptr, nullptr, f, lo.a_down, zd, nullptr, 1.f},
                                j_dob}};
      hipLaunchKernelGGL((lora_proj_mfma<bf16_t, 3>), dim3(gx, 3), dim3(64 * kProjWaves), 0, c.stream, L, offsets,
                         r, jobs);
    }
    MOE_TRY(hipGetLastError());
  } else {
    if (!have_z) {
      MOE_TRY(launch_lora_rowproj<bf16_t>(c, L, offsets, rmax, x_rows, d, x_src, nullptr, d, lo.a_up, true, r, zu));
      MOE_TRY(launch_lora_rowproj<bf16_t>(c, L, offsets, rmax, H, 3 * f, nullptr, nullptr, f, lo.a_down, true, r, zd));
    }
    MOE_TRY(launch_lora_rowproj<bf16_t>(c, L, offsets, rmax, dy, d, row_src, row_gate, d, lo.b_down, false, r,
                                        ws.wproj, ws.lora_mt, kx ? ws.zx : nullptr, lo.scale));
  }
  if (dgu_packed) {
    if (kx && !mt_all) MOE_TRY(launch_lora_transpose_rn(c, lo.a_down, L, r, f, ws.lora_mt3));
    MOE_TRY(launch_lora_dh_packed(c, sh, ws, lo, dy, row_src, row_gate, offsets, act_save, dgu_packed,
                                  kx ? ws.lora_mt3 : nullptr));
  } else {
    TimedLaunch tl(MOE_K_LORA_DH, c.stream);
    DhProb<Cfg> pb{dy, row_src, row_gate, offsets, ws.gemm_tiles, w_down, d, f, (f + Cfg::BN - 1) / Cfg::BN,
                   ws.wproj, lo.a_down, r, lo.scale, act_save, ws.du};
    hipLaunchKernelGGL(lora_dh_bf16<Cfg>, dim3(c.num_cus * 2), dim3(256), Cfg::SMEM_BYTES, c.stream, pb,
                       max_tiles);
    MOE_TRY(hipGetLastError());
  }
  MOE_TRY(launch_lora_rowproj<float>(c, L, offsets, rmax, ws.du, f, nullptr, nullptr, f, mt_all ? ws.lora_mt2 : lo.b_up,
                                     mt_all, r, ws.vproj, ws.lora_mt));
  if (seg_mfma_ok(r, dy, d, d) && seg_mfma_ok(r, H, 3 * f, f) && seg_mfma_ok(r, x_rows, d, d)) {
    // db_down, da_down and da_up (bf16 rows) in one launch
    TimedLaunch tl(MOE_K_LORA_GRAD, c.stream);
    SegJobs<3> jobs{{{zd, dy, d, row_src, row_gate, d, 0, db_down},
                     {ws.wproj, H, 3 * f, nullptr, nullptr, f, 1, da_down},
                     {ws.vproj, x_rows, d, x_src, nullptr, d, 1, da_up}}};
    hipLaunchKernelGGL((lora_seg_mfma<3>), dim3(std::max(d, f) / kSmCols, L, 3), dim3(64 * kSmWaves), 0, c.stream,
                       offsets, r, lo.scale, jobs);
    MOE_TRY(hipGetLastError());
  } else {
    MOE_TRY(launch_seg_outer<bf16_t>(c, L, offsets, zd, r, dy, d, row_src, row_gate, d, lo.scale, false, db_down));
    MOE_TRY(launch_seg_outer<bf16_t>(c, L, offsets, ws.wproj, r, H, 3 * f, nullptr, nullptr, f, lo.scale, true,
                                     da_down));
    MOE_TRY(launch_seg_outer<bf16_t>(c, L, offsets, ws.vproj, r, x_rows, d, x_src, nullptr, d, lo.scale, true,
                                     da_up));
  }
  MOE_TRY(launch_seg_outer<float>(c, L, offsets, zu, r, ws.du, f, nullptr, nullptr, f, lo.scale, false, db_up));
#undef MOE_TRY
  return hipSuccess;
}

}  // namespace moe
