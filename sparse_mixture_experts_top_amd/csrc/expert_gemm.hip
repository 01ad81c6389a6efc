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
//   K8 gate_up  per (row tile, 64 FFN columns): the B tile interleaves 16 rows
//             of W_g and the same 16 rows of W_u, so each lane ends up holding
//             G and U of the same (row, column) and applies silu(G) * U in
//             registers; H is rounded to bf16.
//   K9 down   per (row tile, 128 output columns): O = H W_d^T (+ LoRA).
// Both are persistent: a grid of 2 workgroups per CU walks the items, each
// XCD taking a contiguous range so row tiles that share A or B stay in one L2.
// fp32 path (small parity shapes): one thread per output element.
#include "common.h"
#include "mfma_tile.h"

namespace moe {

using GemmCfg = TileCfg<kGemmBM, 128>;

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

template <class Cfg>
__global__ __launch_bounds__(256) void gate_up_bf16(
    const bf16_t* __restrict__ x_perm, const int32_t* __restrict__ offsets,
    const int32_t* __restrict__ tiles, int max_tiles, const bf16_t* __restrict__ w_gate,
    const bf16_t* __restrict__ w_up, int d, int f, const float* __restrict__ zu,
    const bf16_t* __restrict__ b_up, int r, float lora_scale, bf16_t* __restrict__ hbuf,
    bf16_t* __restrict__ act_save) {
  extern __shared__ __align__(16) unsigned char smem_raw[];
  bf16_t* smem = reinterpret_cast<bf16_t*>(smem_raw);
  constexpr int HALF = Cfg::BN / 2;  // FFN columns per item
  const int nt = f / HALF;
  const int ntiles = tiles[2 * max_tiles];
  const XcdSplit sp = xcd_split(ntiles * nt);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int lrow = tid / Cfg::CHUNKS_PER_ROW, lcol = (tid % Cfg::CHUNKS_PER_ROW) * 8;
  for (int item = sp.first; item < sp.end; item += sp.stride) {
    const int ti = item / nt, ni = item % nt;
    const int le = tiles[2 * ti], r0 = tiles[2 * ti + 1];
    const int seg = offsets[le];
    const int valid = min(Cfg::BM, offsets[le + 1] - seg - r0);
    const int64_t row0 = (int64_t)seg + r0;
    const bf16_t* a_rows[Cfg::A_LOADS];
    const bf16_t* b_rows[Cfg::B_LOADS];
#pragma unroll
    for (int i = 0; i < Cfg::A_LOADS; ++i)
      a_rows[i] = x_perm + (row0 + min(lrow + i * Cfg::ROWS_PER_PASS, valid - 1)) * d + lcol;
#pragma unroll
    for (int i = 0; i < Cfg::B_LOADS; ++i) {
      const int jb = lrow + i * Cfg::ROWS_PER_PASS;
      const int frag = jb >> 4;
      const int fcol = ni * HALF + (frag >> 1) * 16 + (jb & 15);
      const bf16_t* w = (frag & 1) ? w_up : w_gate;
      b_rows[i] = w + ((int64_t)le * f + fcol) * d + lcol;
    }
    Acc<Cfg> acc;
    acc.zero();
    mainloop_nt<Cfg>(a_rows, b_rows, d, acc, smem);
#pragma unroll
    for (int jj = 0; jj < Cfg::FN; jj += 2) {
      const int jg = wn * Cfg::FN + jj;  // even: G fragment, jg + 1: U fragment
      const int fcol = ni * HALF + (jg >> 1) * 16 + (lane & 15);
#pragma unroll
      for (int i = 0; i < Cfg::FM; ++i)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int rin = frag_row<Cfg>(wm, i, lane, q);
          if (rin >= valid) continue;
          const int64_t row = row0 + rin;
          const float g = acc.v[i][jj][q];
          float u = acc.v[i][jj + 1][q];
          if (zu) {
            const float* z = zu + row * r;
            const bf16_t* bu = b_up + ((int64_t)le * f + fcol) * r;
            float t = 0.f;
            for (int c = 0; c < r; ++c) t = fmaf(z[c], bf16_to_f32(bu[c]), t);
            u = fmaf(lora_scale, t, u);
          }
          const bf16_t h = f32_to_bf16(silu_f(g) * u);
          hbuf[row * f + fcol] = h;
          if (act_save) {
            act_save[row * 2 * f + fcol] = f32_to_bf16(g);
            act_save[row * 2 * f + f + fcol] = h;
          }
        }
    }
  }
}

template <class Cfg>
__global__ __launch_bounds__(256) void down_bf16(
    const bf16_t* __restrict__ hbuf, const int32_t* __restrict__ offsets,
    const int32_t* __restrict__ tiles, int max_tiles, const bf16_t* __restrict__ w_down, int d,
    int f, const float* __restrict__ zd, const bf16_t* __restrict__ b_down, int r,
    float lora_scale, bf16_t* __restrict__ y_perm) {
  extern __shared__ __align__(16) unsigned char smem_raw[];
  bf16_t* smem = reinterpret_cast<bf16_t*>(smem_raw);
  const int nt = (d + Cfg::BN - 1) / Cfg::BN;
  const int ntiles = tiles[2 * max_tiles];
  const XcdSplit sp = xcd_split(ntiles * nt);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int lrow = tid / Cfg::CHUNKS_PER_ROW, lcol = (tid % Cfg::CHUNKS_PER_ROW) * 8;
  for (int item = sp.first; item < sp.end; item += sp.stride) {
    const int ti = item / nt, ni = item % nt;
    const int le = tiles[2 * ti], r0 = tiles[2 * ti + 1];
    const int seg = offsets[le];
    const int valid = min(Cfg::BM, offsets[le + 1] - seg - r0);
    const int64_t row0 = (int64_t)seg + r0;
    const int n0 = ni * Cfg::BN;
    const bf16_t* a_rows[Cfg::A_LOADS];
    const bf16_t* b_rows[Cfg::B_LOADS];
#pragma unroll
    for (int i = 0; i < Cfg::A_LOADS; ++i)
      a_rows[i] = hbuf + (row0 + min(lrow + i * Cfg::ROWS_PER_PASS, valid - 1)) * f + lcol;
#pragma unroll
    for (int i = 0; i < Cfg::B_LOADS; ++i)
      b_rows[i] = w_down + ((int64_t)le * d + min(n0 + lrow + i * Cfg::ROWS_PER_PASS, d - 1)) * f + lcol;
    Acc<Cfg> acc;
    acc.zero();
    mainloop_nt<Cfg>(a_rows, b_rows, f, acc, smem);
#pragma unroll
    for (int j = 0; j < Cfg::FN; ++j) {
      const int n = n0 + frag_col<Cfg>(wn, j, lane);
      if (n >= d) continue;
#pragma unroll
      for (int i = 0; i < Cfg::FM; ++i)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int rin = frag_row<Cfg>(wm, i, lane, q);
          if (rin >= valid) continue;
          const int64_t row = row0 + rin;
          float o = acc.v[i][j][q];
          if (zd) {
            const float* z = zd + row * r;
            const bf16_t* bd = b_down + ((int64_t)le * d + n) * r;
            float t = 0.f;
            for (int c = 0; c < r; ++c) t = fmaf(z[c], bf16_to_f32(bd[c]), t);
            o = fmaf(lora_scale, t, o);
          }
          y_perm[row * d + n] = f32_to_bf16(o);
        }
    }
  }
}

// ------------------------------------------------------------- fp32 path ---

__global__ __launch_bounds__(256) void gate_up_f32(const float* __restrict__ x_perm,
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
    const float* xr = x_perm + (int64_t)p * d;
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
      act_save[(int64_t)p * 2 * f + c] = g;
      act_save[(int64_t)p * 2 * f + f + c] = h;
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
                            int32_t* tiles) {
  TimedLaunch tl(MOE_K_TILES, c.stream);
  hipLaunchKernelGGL(build_row_tiles, dim3(1), dim3(1024), 0, c.stream, offsets, L, kGemmBM,
                     max_tiles, tiles);
  return hipGetLastError();
}

hipError_t launch_expert_gemm(const Ctx& c, const moe_shape_t& s, const Workspace& ws,
                              const void* x_perm, const int32_t* offsets, const void* w_gate,
                              const void* w_up, const void* w_down, const LoraArgs* lora,
                              void* act_save, void* y_perm) {
  const int L = s.e_hi - s.e_lo;
  const int64_t rmax = max_rows(s);
  hipError_t err;
  if (s.dtype != MOE_BF16) {
    const int grid = c.num_cus * 4;
    {
      TimedLaunch tl(MOE_K_GATE_UP, c.stream);
      hipLaunchKernelGGL(gate_up_f32, dim3(grid), dim3(256), 0, c.stream, (const float*)x_perm,
                         offsets, L, rmax, (const float*)w_gate, (const float*)w_up, s.d, s.f,
                         (float*)ws.hbuf, (float*)act_save);
    }
    if ((err = hipGetLastError()) != hipSuccess) return err;
    TimedLaunch tl(MOE_K_DOWN, c.stream);
    hipLaunchKernelGGL(down_f32, dim3(grid), dim3(256), 0, c.stream, (const float*)ws.hbuf, offsets,
                       L, (const float*)w_down, s.d, s.f, (float*)y_perm);
    return hipGetLastError();
  }
  const int max_tiles = gemm_max_tiles(s);
  if ((err = launch_row_tiles(c, offsets, L, max_tiles, ws.gemm_tiles)) != hipSuccess) return err;
  const bf16_t* xp = (const bf16_t*)x_perm;
  if (lora) {
    err = launch_lora_rowproj<bf16_t>(c, L, offsets, rmax, xp, s.d, nullptr, nullptr, s.d,
                                      lora->a_up, true, lora->r, ws.zu);
    if (err != hipSuccess) return err;
  }
  const int grid = c.num_cus * 2;  // two 72 KB-LDS workgroups fit one CU
  {
    TimedLaunch tl(MOE_K_GATE_UP, c.stream);
    hipLaunchKernelGGL(gate_up_bf16<GemmCfg>, dim3(grid), dim3(256), GemmCfg::SMEM_BYTES, c.stream,
                       xp, offsets, ws.gemm_tiles, max_tiles, (const bf16_t*)w_gate,
                       (const bf16_t*)w_up, s.d, s.f, lora ? ws.zu : nullptr,
                       lora ? lora->b_up : nullptr, lora ? lora->r : 0,
                       lora ? lora->scale : 0.f, (bf16_t*)ws.hbuf, (bf16_t*)act_save);
  }
  if ((err = hipGetLastError()) != hipSuccess) return err;
  if (lora) {
    err = launch_lora_rowproj<bf16_t>(c, L, offsets, rmax, (const bf16_t*)ws.hbuf, s.f, nullptr,
                                      nullptr, s.f, lora->a_down, true, lora->r, ws.zd);
    if (err != hipSuccess) return err;
  }
  TimedLaunch tl(MOE_K_DOWN, c.stream);
  hipLaunchKernelGGL(down_bf16<GemmCfg>, dim3(grid), dim3(256), GemmCfg::SMEM_BYTES, c.stream,
                     (const bf16_t*)ws.hbuf, offsets, ws.gemm_tiles, max_tiles,
                     (const bf16_t*)w_down, s.d, s.f, lora ? ws.zd : nullptr,
                     lora ? lora->b_down : nullptr, lora ? lora->r : 0, lora ? lora->scale : 0.f,
                     (bf16_t*)y_perm);
  return hipGetLastError();
}

}  // namespace moe
