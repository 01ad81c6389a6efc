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
//   rowproj    one wave per row: out[p, 0..r) = scale_p * in[src_p] . M rows
//              (the rank-r projections Z_u, Z_d, dO B_d, dU B_u), fp32
//   dh         MFMA GEMM of the gathered dY rows against W_d (stored [d, f],
//              so B is transposed while staged into LDS), scaled by the row
//              gate, plus the rank-r term, times silu(G) -> dU (fp32)
//   seg_outer  per expert and column block: sum over the expert's rows of
//              P[p, q] * Q[p, c] -> the gradients, fp32, rows in order
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

template <class TIn>
hipError_t launch_lora_rowproj(const Ctx& c, int L, const int32_t* offsets, int64_t rmax_rows,
                               const TIn* in, int64_t in_stride, const int32_t* src,
                               const float* row_scale, int K, const bf16_t* M, bool m_qk, int r,
                               float* out) {
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
                                                const float*, int, const bf16_t*, bool, int, float*);
template hipError_t launch_lora_rowproj<float>(const Ctx&, int, const int32_t*, int64_t,
                                               const float*, int64_t, const int32_t*, const float*,
                                               int, const bf16_t*, bool, int, float*);

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

template <class TIn>
static hipError_t launch_seg_outer(const Ctx& c, int L, const int32_t* offsets, const float* P,
                                   int r, const TIn* in, int64_t in_stride, const int32_t* qsrc,
                                   const float* qscale, int C, float s, bool out_qc, float* out) {
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
                           float* db_up, float* da_down, float* db_down) {
  using Cfg = TileCfg<kGemmBM, 128>;
  const int L = sh.e_hi - sh.e_lo;
  const int d = sh.d, f = sh.f, r = lo.r;
  const int64_t rmax = max_rows(sh);
  const int max_tiles = gemm_max_tiles(sh);
  const bf16_t* H = act_save + f;  // rows of stride 3f (G | H | U)
  hipError_t err;
#define MOE_TRY(x) \
  if ((err = (x)) != hipSuccess) return err
  MOE_TRY(launch_row_tiles(c, offsets, L, max_tiles, ws.gemm_tiles));
  MOE_TRY(launch_lora_rowproj<bf16_t>(c, L, offsets, rmax, x_rows, d, x_src, nullptr, d, lo.a_up, true, r, ws.zu));
  MOE_TRY(launch_lora_rowproj<bf16_t>(c, L, offsets, rmax, H, 3 * f, nullptr, nullptr, f, lo.a_down, true, r, ws.zd));
  MOE_TRY(launch_lora_rowproj<bf16_t>(c, L, offsets, rmax, dy, d, row_src, row_gate, d, lo.b_down, false, r, ws.wproj));
  {
    TimedLaunch tl(MOE_K_LORA_DH, c.stream);
    DhProb<Cfg> pb{dy, row_src, row_gate, offsets, ws.gemm_tiles, w_down, d, f, (f + Cfg::BN - 1) / Cfg::BN,
                   ws.wproj, lo.a_down, r, lo.scale, act_save, ws.du};
    hipLaunchKernelGGL(lora_dh_bf16<Cfg>, dim3(c.num_cus * 2), dim3(256), Cfg::SMEM_BYTES, c.stream, pb,
                       max_tiles);
    MOE_TRY(hipGetLastError());
  }
  MOE_TRY(launch_lora_rowproj<float>(c, L, offsets, rmax, ws.du, f, nullptr, nullptr, f, lo.b_up, false, r, ws.vproj));
  MOE_TRY(launch_seg_outer<bf16_t>(c, L, offsets, ws.zd, r, dy, d, row_src, row_gate, d, lo.scale, false, db_down));
  MOE_TRY(launch_seg_outer<bf16_t>(c, L, offsets, ws.wproj, r, H, 3 * f, nullptr, nullptr, f, lo.scale, true, da_down));
  MOE_TRY(launch_seg_outer<float>(c, L, offsets, ws.zu, r, ws.du, f, nullptr, nullptr, f, lo.scale, false, db_up));
  MOE_TRY(launch_seg_outer<bf16_t>(c, L, offsets, ws.vproj, r, x_rows, d, x_src, nullptr, d, lo.scale, true, da_up));
#undef MOE_TRY
  return hipSuccess;
}

}  // namespace moe
