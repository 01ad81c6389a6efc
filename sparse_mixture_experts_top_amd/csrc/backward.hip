// Full backward of the layer for the loss sum(y * dY) + L_aux: the gradient
// of the gates and of the router logits, and dx through the frozen experts
// and the frozen router.
//
// "Adapting Trillion-Parameter MoE Models for LoRA Fine-Tuning: A Full-Stack
// Engineering Guide", §3: the adapters train through a frozen MoE layer, so
// the layers below need the input gradient; "Trillion-Parameter MoE Model
// Training Adaptation: Full-Stack Optimization Practices", §3: the backward
// runs the permute / grouped GEMM / unpermute stages in reverse; §2.1 of the
// guide: y = sum_i g_i E_i(x) with the auxiliary load-balance loss.
//
//   gate_bwd   one wave per token: dg_j = <dY_t, O[slot_tj]> for kept local
//              slots (8 rows' loads in flight per chunk); the softmax-over-
//              the-selection Jacobian dl_{idx_j} = g_j (dg_j - sum_i g_i dg_i);
//              with counts, the
//              load-balance term coef E / T * p_te (f_e - sum_e' f_e' p_te')
//              (p = softmax over all E, f = counts / (T k), held constant)
//   dgu        grouped GEMM, per (row tile, 128 FFN columns): dH = g_p dY[src_p]
//              W_d (+ s (dO B_d) A_d), then dG = dH U silu'(G), dU = dH silu(G)
//              from the saved G and U, stored bf16 [Rmax, 2f]
//   dx rows    grouped GEMM over K = 2f: dX = [dG dU] [W_g; W_u] (+ s (dU B_u)
//              A_u), fp32 rows
//   unpermute  dx[t] = sum over the token's kept slots, in j order (the
//              combine kernel with unit gates); the adding form after the
//              router's stored product (one wave per token) touches only
//              tokens with a kept slot
//   router     dx[t] += sum_e dl[t, e] W_r[e]: a dense GEMM with K = E on
//              bf16-rounded logit gradients (fp32 fallback kernels for the
//              small fp32 shapes or E % 64 != 0)
#include "common.h"
#include "mfma_tile.h"

namespace moe {

__device__ __forceinline__ float silu_grad_f(float a) {
  const float s = 1.0f / (1.0f + expf(-a));
  return s * (1.0f + a * (1.0f - s));
}

template <class T>
__device__ __forceinline__ void load8f(const T* p, float (&v)[8]);
template <>
__device__ __forceinline__ void load8f<bf16_t>(const bf16_t* p, float (&v)[8]) {
  const uint4 raw = *reinterpret_cast<const uint4*>(p);
  const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
  for (int u = 0; u < 8; ++u) v[u] = bf16_to_f32(static_cast<bf16_t>(w[u >> 1] >> ((u & 1) * 16)));
}
template <>
__device__ __forceinline__ void load8f<float>(const float* p, float (&v)[8]) {
  const float4 a = *reinterpret_cast<const float4*>(p);
  const float4 b = *reinterpret_cast<const float4*>(p + 4);
  v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
  v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}
__device__ __forceinline__ float load1f(const float* p) { return *p; }
__device__ __forceinline__ float load1f(const bf16_t* p) { return bf16_to_f32(*p); }

// ------------------------------------------------------------ gate bwd ---
// One wave per token (4 per workgroup). Lane j < k holds slot, gate and
// selected expert of assignment j; the dot products run 8 assignments at a
// time over 8-element chunks of the row (VEC, d % 8 == 0; otherwise single
// elements), lanes striding the chunks, and a group whose slots are all
// empty (dropped or not local) is skipped; lane l holds logits l, l + 64,
// ... (EPL of them). The load-balance fractions counts[e] / (T k) are staged
// once per workgroup in LDS.
template <class T, int EPL, bool VEC>
__global__ __launch_bounds__(256) void gate_bwd(const T* __restrict__ dy, const T* __restrict__ y_perm,
                                                const int32_t* __restrict__ slot,
                                                const int32_t* __restrict__ idx,
                                                const float* __restrict__ gate,
                                                const float* __restrict__ logits,
                                                const int32_t* __restrict__ counts, float aux_scale,
                                                float inv_tk, int Tn, int d, int E, int k,
                                                float* __restrict__ dgate, float* __restrict__ dlogits) {
  constexpr int G = 8;  // assignments per group of row loads
  __shared__ float s_fr[EPL * 64];
  const int lane = threadIdx.x & 63;
  if (counts) {
    for (int e = threadIdx.x; e < EPL * 64; e += 256) s_fr[e] = e < E ? (float)counts[e] * inv_tk : 0.f;
    __syncthreads();
  }
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= Tn) return;
  const int my_slot = lane < k ? slot[(int64_t)t * k + lane] : -1;
  const float my_g = lane < k ? gate[(int64_t)t * k + lane] : 0.f;
  const int my_e = lane < k ? idx[(int64_t)t * k + lane] : 0;
  const T* dyr = dy + (int64_t)t * d;
  float my_dg = 0.f;
  // the token's kept local slots, compacted in j order (slot and j per entry)
  __shared__ int s_cs[4][64], s_cj[4][64];
  const int wv = threadIdx.x >> 6;
  const uint64_t kept = __ballot(my_slot >= 0);
  const int n = __popcll(kept);
  if (my_slot >= 0) {
    const uint64_t below = lane == 0 ? 0ull : (~0ull >> (64 - lane));
    const int pos = __popcll(kept & below);
    s_cs[wv][pos] = my_slot;
    s_cj[wv][pos] = lane;
  }
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
  for (int j0 = 0; j0 < n; j0 += G) {
    // G entries (past n: the last kept row again, its sum discarded), the
    // G + 1 loads of a row chunk in flight before its FMAs
    int64_t rb[G];
#pragma unroll
    for (int q = 0; q < G; ++q) rb[q] = (int64_t)s_cs[wv][min(j0 + q, n - 1)] * d;
    float acc[G];
#pragma unroll
    for (int q = 0; q < G; ++q) acc[q] = 0.f;
    if (VEC) {
      for (int i0 = lane * 8; i0 < d; i0 += 64 * 8) {
        float a0[8], o0[G][8];
        load8f<T>(dyr + i0, a0);
#pragma unroll
        for (int q = 0; q < G; ++q) load8f<T>(y_perm + rb[q] + i0, o0[q]);
#pragma unroll
        for (int q = 0; q < G; ++q)
#pragma unroll
          for (int u = 0; u < 8; ++u) acc[q] = fmaf(a0[u], o0[q][u], acc[q]);
      }
    } else {
      for (int i = lane; i < d; i += 64) {
        const float a0 = load1f(dyr + i);
#pragma unroll
        for (int q = 0; q < G; ++q) acc[q] = fmaf(a0, load1f(y_perm + rb[q] + i), acc[q]);
      }
    }
#pragma unroll
    for (int q = 0; q < G; ++q) {
      if (j0 + q >= n) break;  // wave-uniform
      const float v = wave_sum(acc[q]);
      if (lane == s_cj[wv][j0 + q]) my_dg = v;
    }
  }
  if (dgate && lane < k) dgate[(int64_t)t * k + lane] = my_dg;
  // softmax over the selection: dl_{idx_j} = g_j (dg_j - sum_i g_i dg_i)
  const float inner = wave_sum(my_g * my_dg);
  const float contrib = my_g * (my_dg - inner);
  float val[EPL];
  if (counts) {
    float l[EPL], m = -INFINITY;
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
      const int e = lane + 64 * i;
      l[i] = e < E ? logits[(int64_t)t * E + e] : -INFINITY;
      m = fmaxf(m, l[i]);
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, kWave));
    float z = 0.f;
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
      l[i] = lane + 64 * i < E ? expf(l[i] - m) : 0.f;
      z += l[i];
    }
    const float inv_z = 1.0f / wave_sum(z);
    float fp = 0.f, fr[EPL];
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
      l[i] *= inv_z;  // p
      fr[i] = s_fr[lane + 64 * i];
      fp = fmaf(l[i], fr[i], fp);
    }
    fp = wave_sum(fp);
#pragma unroll
    for (int i = 0; i < EPL; ++i) val[i] = aux_scale * l[i] * (fr[i] - fp);
  } else {
#pragma unroll
    for (int i = 0; i < EPL; ++i) val[i] = 0.f;
  }
  for (int j = 0; j < k; ++j) {
    const int e = __shfl(my_e, j, kWave);
    const float cj = __shfl(contrib, j, kWave);
#pragma unroll
    for (int i = 0; i < EPL; ++i)
      if (e == lane + 64 * i) val[i] += cj;
  }
#pragma unroll
  for (int i = 0; i < EPL; ++i) {
    const int e = lane + 64 * i;
    if (e < E) dlogits[(int64_t)t * E + e] = val[i];
  }
}

hipError_t launch_gate_bwd(const Ctx& c, const moe_shape_t& s, const void* dy, const void* y_perm,
                           const int32_t* slot, const int32_t* idx, const float* gate,
                           const float* logits, const int32_t* counts, float aux_coef, float* dgate,
                           float* dlogits) {
  if (s.T == 0) return hipSuccess;
  const int epl = (s.E + 63) / 64;
  const bool aux = counts != nullptr && aux_coef != 0.f;
  const float aux_scale = aux ? aux_coef * (float)s.E / (float)s.T : 0.f;
  const float inv_tk = 1.0f / ((float)s.T * (float)s.k);
  const int grid = (s.T + 3) / 4;
  TimedLaunch tl(MOE_K_GATE_BWD, c.stream);
  const bool vec = s.d % 8 == 0;
#define MOE_GB(TT, N)                                                                                   \
  do {                                                                                                  \
    if (vec) MOE_GB2(TT, N, true)                                                                       \
    else MOE_GB2(TT, N, false)                                                                          \
  } while (0)
#define MOE_GB2(TT, N, V)                                                                               \
  hipLaunchKernelGGL((gate_bwd<TT, N, V>), dim3(grid), dim3(256), 0, c.stream, (const TT*)dy,           \
                     (const TT*)y_perm, slot, idx, gate, logits, aux ? counts : nullptr, aux_scale,    \
                     inv_tk, s.T, s.d, s.E, s.k, dgate, dlogits);
#define MOE_GB_E(TT)                      \
  if (epl <= 1) MOE_GB(TT, 1);            \
  else if (epl <= 2) MOE_GB(TT, 2);       \
  else if (epl <= 4) MOE_GB(TT, 4);       \
  else if (epl <= 8) MOE_GB(TT, 8);       \
  else if (epl <= 14) MOE_GB(TT, 14);     \
  else MOE_GB(TT, 16);
  if (s.dtype == MOE_BF16) {
    MOE_GB_E(bf16_t)
  } else {
    MOE_GB_E(float)
  }
#undef MOE_GB_E
#undef MOE_GB
#undef MOE_GB2
  return hipGetLastError();
}

// ---------------------------------------------------- expert dG / dU GEMM ---
// dH[row, n] = g_row * (dY[src_row] . W_d[:, n]) (+ s * wproj[row] . A_d[:, n]),
// per (row tile, 128 FFN columns) item; W_d is stored [d, f], so B is
// transposed while staged into LDS. The epilogue turns dH into dG and dU.
template <class Cfg>
struct DguProb {
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
  const bf16_t* act_save;  // [Rmax, 3f]: G | H | U
  bf16_t* dgu;             // [Rmax, 2f]: dG | dU

  __device__ __forceinline__ void tile(int item, int& le, int64_t& row0, int& valid, int& n0) const {
    const int ti = item / nt;
    n0 = (item % nt) * Cfg::BN;
    le = ld_uniform(tiles, 2 * ti);
    const int r0 = ld_uniform(tiles, 2 * ti + 1);
    const int seg = ld_uniform(offsets, le);
    valid = min(Cfg::BM, ld_uniform(offsets, le + 1) - seg - r0);
    row0 = (int64_t)seg + r0;
  }

  __device__ __forceinline__ void setup(int item, LoaderNN<Cfg>& ld) const {
    int le, valid, n0;
    int64_t row0;
    tile(item, le, row0, valid, n0);
    const int lrow = threadIdx.x / Cfg::CHUNKS_PER_ROW, lcol = (threadIdx.x % Cfg::CHUNKS_PER_ROW) * 8;
#pragma unroll
    for (int i = 0; i < Cfg::A_LOADS; ++i) {
      const int64_t row = row0 + min(lrow + i * Cfg::ROWS_PER_PASS, valid - 1);
      ld.a[i] = dy + (int64_t)row_src[row] * d + lcol;
    }
    ld.b_base = w_down + (int64_t)le * d * f + n0;
    ld.ldb = f;
    ld.n_valid = min(Cfg::BN, f - n0);
  }

  __device__ __forceinline__ void epilogue(int item, Acc<Cfg>& acc) const {
    int le, valid, n0;
    int64_t row0;
    tile(item, le, row0, valid, n0);
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
          float lo = 0.f;
          if (wproj) {
            const float* w = wproj + row * r;
            const bf16_t* ad = a_down + (int64_t)le * r * f + n;
            for (int cc = 0; cc < r; ++cc) lo = fmaf(w[cc], bf16_to_f32(ad[(int64_t)cc * f]), lo);
          }
          const float dh = fmaf(row_gate[row], acc.v[i][j][q], s * lo);
          const float g = bf16_to_f32(act_save[row * 3 * f + n]);
          const float u = bf16_to_f32(act_save[row * 3 * f + 2 * f + n]);
          dgu[row * 2 * f + n] = f32_to_bf16(dh * u * silu_grad_f(g));
          dgu[row * 2 * f + f + n] = f32_to_bf16(dh * silu_f(g));
        }
    }
  }
};

template <class Cfg>
__global__ __launch_bounds__(256, 2) void expert_dgu_bf16(DguProb<Cfg> pb, int max_tiles) {
  extern __shared__ __align__(16) unsigned char smem_raw[];
  const int items = ld_uniform(pb.tiles, 2 * max_tiles) * pb.nt;
  persistent_gemm<Cfg, LoaderNN<Cfg>>(pb, items, pb.d / Cfg::BK, reinterpret_cast<bf16_t*>(smem_raw));
}

// ------------------------------------------------------ expert dX GEMM ---
// B of dX = [dG dU] [W_g; W_u]: K steps below kt_split read W_g[le] ([f, d]),
// the others W_u[le]; both transposed into LDS like LoaderNN.
template <class Cfg>
struct LoaderNN2 {
  typedef RegsNN<Cfg> Regs;
  const bf16_t* a[Cfg::A_LOADS];
  const bf16_t* b0;
  const bf16_t* b1;
  int kt_split;
  int64_t ldb;
  int n_valid;
  __device__ __forceinline__ void load(Regs& r, int kt) const {
    const int k0 = kt * Cfg::BK;
    const int nk_row = threadIdx.x / Cfg::NN_CHUNKS_PER_K;
    const int nn_col = (threadIdx.x % Cfg::NN_CHUNKS_PER_K) * 8;
    gload_rows(r.a, a, k0);
    const bool first = kt < kt_split;
    gload_nn<Cfg>(r.b, first ? b0 : b1, ldb, first ? k0 : k0 - kt_split * Cfg::BK, nk_row, nn_col, n_valid,
                  nn_col + 8 <= n_valid);
  }
  __device__ __forceinline__ void store(bf16_t* As, bf16_t* Bs, const Regs& r) const {
    const int lrow = threadIdx.x / Cfg::CHUNKS_PER_ROW, lcol = (threadIdx.x % Cfg::CHUNKS_PER_ROW) * 8;
    sstore_rows<Cfg>(As, r.a, lrow, lcol);
    sstore_nn<Cfg>(Bs, r.b, threadIdx.x / Cfg::NN_CHUNKS_PER_K, (threadIdx.x % Cfg::NN_CHUNKS_PER_K) * 8);
  }
};

template <class Cfg>
struct DxProb {
  const bf16_t* dgu;  // [Rmax, 2f]
  const int32_t* offsets;
  const int32_t* tiles;
  const bf16_t* w_gate;
  const bf16_t* w_up;
  int d, f, nt;
  const float* vproj;  // [Rmax, r] dU B_u, or NULL
  const bf16_t* a_up;  // [L, r, d]
  int r;
  float s;
  float* dx_rows;  // [Rmax, d]

  __device__ __forceinline__ void tile(int item, int& le, int64_t& row0, int& valid, int& n0) const {
    const int ti = item / nt;
    n0 = (item % nt) * Cfg::BN;
    le = ld_uniform(tiles, 2 * ti);
    const int r0 = ld_uniform(tiles, 2 * ti + 1);
    const int seg = ld_uniform(offsets, le);
    valid = min(Cfg::BM, ld_uniform(offsets, le + 1) - seg - r0);
    row0 = (int64_t)seg + r0;
  }

  __device__ __forceinline__ void setup(int item, LoaderNN2<Cfg>& ld) const {
    int le, valid, n0;
    int64_t row0;
    tile(item, le, row0, valid, n0);
    const int lrow = threadIdx.x / Cfg::CHUNKS_PER_ROW, lcol = (threadIdx.x % Cfg::CHUNKS_PER_ROW) * 8;
#pragma unroll
    for (int i = 0; i < Cfg::A_LOADS; ++i)
      ld.a[i] = dgu + (row0 + min(lrow + i * Cfg::ROWS_PER_PASS, valid - 1)) * 2 * f + lcol;
    ld.b0 = w_gate + (int64_t)le * f * d + n0;
    ld.b1 = w_up + (int64_t)le * f * d + n0;
    ld.kt_split = f / Cfg::BK;
    ld.ldb = d;
    ld.n_valid = min(Cfg::BN, d - n0);
  }

  __device__ __forceinline__ void epilogue(int item, Acc<Cfg>& acc) const {
    int le, valid, n0;
    int64_t row0;
    tile(item, le, row0, valid, n0);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int wm = wave >> 1, wn = wave & 1;
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
          float v = acc.v[i][j][q];
          if (vproj) {
            const float* w = vproj + row * r;
            const bf16_t* au = a_up + (int64_t)le * r * d + n;
            float lo = 0.f;
            for (int cc = 0; cc < r; ++cc) lo = fmaf(w[cc], bf16_to_f32(au[(int64_t)cc * d]), lo);
            v = fmaf(s, lo, v);
          }
          dx_rows[row * d + n] = v;
        }
    }
  }
};

template <class Cfg>
__global__ __launch_bounds__(256, 2) void expert_dx_bf16(DxProb<Cfg> pb, int max_tiles) {
  extern __shared__ __align__(16) unsigned char smem_raw[];
  const int items = ld_uniform(pb.tiles, 2 * max_tiles) * pb.nt;
  persistent_gemm<Cfg, LoaderNN2<Cfg>>(pb, items, 2 * pb.f / Cfg::BK, reinterpret_cast<bf16_t*>(smem_raw));
}

// ------------------------------------------------------- fp32 expert path ---
// Small fp32 shapes: one thread per output element.
__global__ __launch_bounds__(256) void expert_dgu_f32(const float* __restrict__ dy,
                                                      const int32_t* __restrict__ row_src,
                                                      const float* __restrict__ row_gate,
                                                      const int32_t* __restrict__ offsets, int L,
                                                      const float* __restrict__ w_down,
                                                      const float* __restrict__ act_save, int d, int f,
                                                      float* __restrict__ dgu) {
  const int R = offsets[L];
  for (int64_t id = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; id < (int64_t)R * f;
       id += (int64_t)gridDim.x * blockDim.x) {
    const int p = (int)(id / f), n = (int)(id % f);
    const int le = segment_of(offsets, L, p);
    const float* dyr = dy + (int64_t)row_src[p] * d;
    const float* wd = w_down + (int64_t)le * d * f + n;
    float acc = 0.f;
    for (int i = 0; i < d; ++i) acc = fmaf(dyr[i], wd[(int64_t)i * f], acc);
    const float dh = row_gate[p] * acc;
    const float g = act_save[(int64_t)p * 3 * f + n], u = act_save[(int64_t)p * 3 * f + 2 * f + n];
    dgu[(int64_t)p * 2 * f + n] = dh * u * silu_grad_f(g);
    dgu[(int64_t)p * 2 * f + f + n] = dh * silu_f(g);
  }
}

__global__ __launch_bounds__(256) void expert_dx_f32(const float* __restrict__ dgu,
                                                     const int32_t* __restrict__ offsets, int L,
                                                     const float* __restrict__ w_gate,
                                                     const float* __restrict__ w_up, int d, int f,
                                                     float* __restrict__ dx_rows) {
  const int R = offsets[L];
  for (int64_t id = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; id < (int64_t)R * d;
       id += (int64_t)gridDim.x * blockDim.x) {
    const int p = (int)(id / d), n = (int)(id % d);
    const int le = segment_of(offsets, L, p);
    const float* gr = dgu + (int64_t)p * 2 * f;
    const float* wg = w_gate + (int64_t)le * f * d + n;
    const float* wu = w_up + (int64_t)le * f * d + n;
    float acc = 0.f;
    for (int cc = 0; cc < f; ++cc) acc = fmaf(gr[cc], wg[(int64_t)cc * d], acc);
    for (int cc = 0; cc < f; ++cc) acc = fmaf(gr[f + cc], wu[(int64_t)cc * d], acc);
    dx_rows[id] = acc;
  }
}

// dx[t] = sum over the token's kept slots j, in j order, of dx_rows[slot].
// Like the forward combine: TB tokens per workgroup, a wave per token
// compacts its kept slots (ballot, j order) into LDS, then each thread owns
// 4 consecutive columns and adds the rows in batches whose loads are all
// issued before the first use (a short batch re-reads its last row and adds
// it times 0 through selects).
template <int NB>
__device__ __forceinline__ void unpermute_batch(float4& acc, const float* __restrict__ rows, const int* s_slot,
                                                int j0, int nb, int d, int v) {
  float4 raw[NB];
#pragma unroll
  for (int b = 0; b < NB; ++b)
    raw[b] = *reinterpret_cast<const float4*>(rows + (int64_t)s_slot[j0 + min(b, nb - 1)] * d + v * 4);
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    const float m = b < nb ? 1.f : 0.f;
    acc.x = fmaf(m, raw[b].x, acc.x);
    acc.y = fmaf(m, raw[b].y, acc.y);
    acc.z = fmaf(m, raw[b].z, acc.z);
    acc.w = fmaf(m, raw[b].w, acc.w);
  }
}

template <int TB>
__global__ __launch_bounds__(256) void unpermute_sum_f32(const float* __restrict__ dx_rows,
                                                         const int32_t* __restrict__ slot, int T, int k,
                                                         int d, float* __restrict__ dx) {
  __shared__ int s_slot[TB][32];
  __shared__ int s_n[TB];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int nvec = d / 4;
  for (int t0 = blockIdx.x * TB; t0 < T; t0 += gridDim.x * TB) {
    const int nq = min(TB, T - t0);
    for (int q = wave; q < nq; q += 4) {
      const int sl = lane < k ? slot[(int64_t)(t0 + q) * k + lane] : -1;
      const uint64_t kept = __ballot(sl >= 0);
      const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
      if (sl >= 0) s_slot[q][__popcll(kept & below)] = sl;
      if (lane == 0) s_n[q] = __popcll(kept);
    }
    __syncthreads();
    for (int q = 0; q < nq; ++q) {
      const int n = s_n[q];
      if (d % 4 == 0) {
        for (int v = threadIdx.x; v < nvec; v += blockDim.x) {
          float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
          int j0 = 0;
          for (; j0 + 8 <= n; j0 += 8) unpermute_batch<8>(acc, dx_rows, s_slot[q], j0, 8, d, v);
          for (; j0 < n; j0 += 2) unpermute_batch<2>(acc, dx_rows, s_slot[q], j0, n - j0, d, v);
          *reinterpret_cast<float4*>(dx + (int64_t)(t0 + q) * d + v * 4) = acc;
        }
      } else {
        // rows not 16-byte aligned: one column per thread, same j order
        for (int c = threadIdx.x; c < d; c += blockDim.x) {
          float acc = 0.f;
          for (int j = 0; j < n; ++j) acc += dx_rows[(int64_t)s_slot[q][j] * d + c];
          dx[(int64_t)(t0 + q) * d + c] = acc;
        }
      }
    }
    __syncthreads();
  }
}

// dx[t] += sum over the token's kept slots (j order) of dx_rows[slot], one
// wave per token; U column chunks of 4 per lane, all loads of a slot pair in
// flight before the adds (a lone last slot re-reads its row, added times 0).
template <int U>
__global__ __launch_bounds__(256) void unpermute_add_wave(const float* __restrict__ rows,
                                                          const int32_t* __restrict__ slot, int T, int k, int d,
                                                          float* __restrict__ dx) {
  const int lane = threadIdx.x & 63;
  const int nw = gridDim.x * 4;
  for (int t = blockIdx.x * 4 + (int)(threadIdx.x >> 6); t < T; t += nw) {
    const int sl = lane < k ? slot[(int64_t)t * k + lane] : -1;
    const uint64_t kept = __ballot(sl >= 0);
    if (kept == 0) continue;
    for (int c0 = lane * 4; c0 < d; c0 += 64 * 4 * U) {
      float4 acc[U];
#pragma unroll
      for (int u = 0; u < U; ++u) acc[u] = make_float4(0.f, 0.f, 0.f, 0.f);
      uint64_t m = kept;
      while (m) {
        const int b0 = __ffsll((long long)m) - 1;
        m &= m - 1;
        const bool two = m != 0;
        const int b1 = two ? __ffsll((long long)m) - 1 : b0;
        if (two) m &= m - 1;
        const int64_t r0 = (int64_t)__builtin_amdgcn_readlane(sl, b0) * d;
        const int64_t r1 = (int64_t)__builtin_amdgcn_readlane(sl, b1) * d;
        float4 x0[U], x1[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int c = min(c0 + 256 * u, d - 4);
          x0[u] = *reinterpret_cast<const float4*>(rows + r0 + c);
          x1[u] = *reinterpret_cast<const float4*>(rows + r1 + c);
        }
        const float w1 = two ? 1.f : 0.f;
#pragma unroll
        for (int u = 0; u < U; ++u) {
          acc[u].x = fmaf(w1, x1[u].x, acc[u].x + x0[u].x);
          acc[u].y = fmaf(w1, x1[u].y, acc[u].y + x0[u].y);
          acc[u].z = fmaf(w1, x1[u].z, acc[u].z + x0[u].z);
          acc[u].w = fmaf(w1, x1[u].w, acc[u].w + x0[u].w);
        }
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int c = c0 + 256 * u;
        if (c < d) {
          float4* p = reinterpret_cast<float4*>(dx + (int64_t)t * d + c);
          const float4 o = *p;
          *p = make_float4(o.x + acc[u].x, o.y + acc[u].y, o.z + acc[u].z, o.w + acc[u].w);
        }
      }
    }
  }
}

hipError_t launch_unpermute(const Ctx& c, const moe_shape_t& s, const float* dx_rows, const int32_t* slot,
                            float* dx, bool add) {
  if (s.T == 0) return hipSuccess;
  TimedLaunch tl(MOE_K_UNPERMUTE, c.stream);
  if (add) {
    if (s.d % 4 != 0) return hipErrorInvalidValue;
    // one wave per token: tokens without a kept slot cost one ballot
    const int nblk = (s.T + 3) / 4;
    const int grid = nblk < c.num_cus * 16 ? nblk : c.num_cus * 16;
    hipLaunchKernelGGL(unpermute_add_wave<4>, dim3(grid), dim3(256), 0, c.stream, dx_rows, slot, s.T, s.k, s.d,
                       dx);
    return hipGetLastError();
  }
  int tb = s.T / (c.num_cus * 8);
  tb = tb >= 8 ? 8 : tb >= 4 ? 4 : tb >= 2 ? 2 : 1;
  const int nblk = (s.T + tb - 1) / tb;
  const int grid = nblk < c.num_cus * 64 ? nblk : c.num_cus * 64;
#define MOE_UNP(N)                                                                                  \
  hipLaunchKernelGGL((unpermute_sum_f32<N>), dim3(grid), dim3(256), 0, c.stream, dx_rows, slot, s.T, s.k, \
                     s.d, dx)
  if (tb == 8) MOE_UNP(8);
  else if (tb == 4) MOE_UNP(4);
  else if (tb == 2) MOE_UNP(2);
  else MOE_UNP(1);
#undef MOE_UNP
  return hipGetLastError();
}

hipError_t launch_expert_bwd(const Ctx& c, const moe_shape_t& s, const Workspace& ws, const LoraArgs* lo,
                             const void* dy, const int32_t* offsets, const int32_t* row_src,
                             const float* row_gate, const int32_t* slot, const void* act_save,
                             const void* w_gate, const void* w_up, const void* w_down,
                             const void* dgu_packed, const void* dx_packed, void* dgu, float* dx_rows,
                             float* dx) {
  const int L = s.e_hi - s.e_lo;
  const int d = s.d, f = s.f;
  const int64_t rmax = max_rows(s);
  hipError_t err;
#define MOE_TRY(x) \
  if ((err = (x)) != hipSuccess) return err
  if (s.dtype != MOE_BF16) {
    const int grid = c.num_cus * 4;
    {
      TimedLaunch tl(MOE_K_EXPERT_DGU, c.stream);
      hipLaunchKernelGGL(expert_dgu_f32, dim3(grid), dim3(256), 0, c.stream, (const float*)dy, row_src, row_gate,
                         offsets, L, (const float*)w_down, (const float*)act_save, d, f, (float*)dgu);
      MOE_TRY(hipGetLastError());
    }
    {
      TimedLaunch tl(MOE_K_EXPERT_DX, c.stream);
      hipLaunchKernelGGL(expert_dx_f32, dim3(grid), dim3(256), 0, c.stream, (const float*)dgu, offsets, L,
                         (const float*)w_gate, (const float*)w_up, d, f, dx_rows);
      MOE_TRY(hipGetLastError());
    }
  } else if (dgu_packed) {
    MOE_TRY(launch_bwd_gemms_packed(c, s, ws, lo, (const bf16_t*)dy, row_src, row_gate, offsets,
                                    (const bf16_t*)act_save, (const bf16_t*)dgu_packed,
                                    (const bf16_t*)dx_packed, (bf16_t*)dgu, dx_rows));
  } else {
    using Cfg = TileCfg<kGemmBM, 128>;
    const int max_tiles = gemm_max_tiles(s);
    MOE_TRY(launch_row_tiles(c, offsets, L, max_tiles, ws.gemm_tiles));
    const bf16_t* dyb = (const bf16_t*)dy;
    bf16_t* dgub = (bf16_t*)dgu;
    if (lo) {
      MOE_TRY(launch_lora_rowproj<bf16_t>(c, L, offsets, rmax, dyb, d, row_src, row_gate, d, lo->b_down, false,
                                          lo->r, ws.wproj, ws.lora_mt));
    }
    {
      TimedLaunch tl(MOE_K_EXPERT_DGU, c.stream);
      DguProb<Cfg> pb{dyb, row_src, row_gate, offsets, ws.gemm_tiles, (const bf16_t*)w_down, d, f,
                      (f + Cfg::BN - 1) / Cfg::BN, lo ? ws.wproj : nullptr, lo ? lo->a_down : nullptr,
                      lo ? lo->r : 0, lo ? lo->scale : 0.f, (const bf16_t*)act_save, dgub};
      hipLaunchKernelGGL(expert_dgu_bf16<Cfg>, dim3(c.num_cus * 2), dim3(256), Cfg::SMEM_BYTES, c.stream, pb,
                         max_tiles);
      MOE_TRY(hipGetLastError());
    }
    if (lo) {
      MOE_TRY(launch_lora_rowproj<bf16_t>(c, L, offsets, rmax, dgub + f, 2 * f, nullptr, nullptr, f, lo->b_up,
                                          false, lo->r, ws.vproj, ws.lora_mt));
    }
    {
      TimedLaunch tl(MOE_K_EXPERT_DX, c.stream);
      DxProb<Cfg> pb{dgub, offsets, ws.gemm_tiles, (const bf16_t*)w_gate, (const bf16_t*)w_up, d, f,
                     (d + Cfg::BN - 1) / Cfg::BN, lo ? ws.vproj : nullptr, lo ? lo->a_up : nullptr,
                     lo ? lo->r : 0, lo ? lo->scale : 0.f, dx_rows};
      hipLaunchKernelGGL(expert_dx_bf16<Cfg>, dim3(c.num_cus * 2), dim3(256), Cfg::SMEM_BYTES, c.stream, pb,
                         max_tiles);
      MOE_TRY(hipGetLastError());
    }
  }
  if (s.T > 0 && dx) MOE_TRY(launch_unpermute(c, s, dx_rows, slot, dx, false));
#undef MOE_TRY
  return hipSuccess;
}

// ---------------------------------------------------------- router bwd ---
// dx[t, n] += sum_e dl[t, e] W_r[e, n]. bf16 with E % 64 == 0: the logit
// gradients are rounded to bf16 rows and multiplied on the MFMAs (W_r is
// [E, d], K = E, so B is transposed into LDS); otherwise one thread per
// output element in fp32.
__global__ __launch_bounds__(256) void to_bf16_rows(const float* __restrict__ in, int64_t n,
                                                    bf16_t* __restrict__ out) {
  for (int64_t i = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) * 8; i < n;
       i += (int64_t)gridDim.x * blockDim.x * 8) {
    const float4 a = *reinterpret_cast<const float4*>(in + i);
    const float4 b = *reinterpret_cast<const float4*>(in + i + 4);
    *reinterpret_cast<uint4*>(out + i) =
        make_uint4(f32x2_to_bf16x2(a.x, a.y), f32x2_to_bf16x2(a.z, a.w), f32x2_to_bf16x2(b.x, b.y),
                   f32x2_to_bf16x2(b.z, b.w));
  }
}

template <class Cfg>
struct RouterBwdProb {
  const bf16_t* dl;  // [T, E] bf16
  const bf16_t* w;   // [E, d]
  int T, E, d, nt;
  float* dx;  // [T, d], accumulated

  __device__ __forceinline__ void setup(int item, LoaderNN<Cfg>& ld) const {
    const int m0 = (item / nt) * Cfg::BM, n0 = (item % nt) * Cfg::BN;
    const int lrow = threadIdx.x / Cfg::CHUNKS_PER_ROW, lcol = (threadIdx.x % Cfg::CHUNKS_PER_ROW) * 8;
#pragma unroll
    for (int i = 0; i < Cfg::A_LOADS; ++i)
      ld.a[i] = dl + (int64_t)min(m0 + lrow + i * Cfg::ROWS_PER_PASS, T - 1) * E + lcol;
    ld.b_base = w + n0;
    ld.ldb = d;
    ld.n_valid = min(Cfg::BN, d - n0);
  }

  __device__ __forceinline__ void epilogue(int item, Acc<Cfg>& acc) const {
    const int m0 = (item / nt) * Cfg::BM, n0 = (item % nt) * Cfg::BN;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int wm = wave >> 1, wn = wave & 1;
#pragma unroll
    for (int j = 0; j < Cfg::FN; ++j) {
      const int n = n0 + frag_col<Cfg>(wn, j, lane);
      if (n >= d) continue;
#pragma unroll
      for (int i = 0; i < Cfg::FM; ++i)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int m = m0 + frag_row<Cfg>(wm, i, lane, q);
          if (m < T) dx[(int64_t)m * d + n] += acc.v[i][j][q];
        }
    }
  }
};

template <class Cfg>
__global__ __launch_bounds__(256, 2) void router_bwd_bf16(RouterBwdProb<Cfg> pb, int items) {
  extern __shared__ __align__(16) unsigned char smem_raw[];
  persistent_gemm<Cfg, LoaderNN<Cfg>>(pb, items, pb.E / Cfg::BK, reinterpret_cast<bf16_t*>(smem_raw));
}

template <class TW>
__global__ __launch_bounds__(256) void router_bwd_simple(const float* __restrict__ dl, const TW* __restrict__ w,
                                                         int T, int E, int d, float* __restrict__ dx) {
  for (int64_t id = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; id < (int64_t)T * d;
       id += (int64_t)gridDim.x * blockDim.x) {
    const int t = (int)(id / d), n = (int)(id % d);
    float acc = 0.f;
    for (int e = 0; e < E; ++e) acc = fmaf(dl[(int64_t)t * E + e], load_f<TW>(w + (int64_t)e * d + n), acc);
    dx[id] += acc;
  }
}

hipError_t launch_router_bwd(const Ctx& c, const moe_shape_t& s, const Workspace& ws, const float* dlogits,
                             const void* w_router, const void* wr_packed, float* dx, const float* dx_rows,
                             const int32_t* slot) {
  if (s.T == 0) return hipSuccess;
  if (slot) {
    // dx = the product (stored, not added), then the expert rows added where
    // a token has any: dx is read only for those tokens
    if (s.dtype != MOE_BF16 || s.E % 64 != 0 || !wr_packed) return hipErrorInvalidValue;
    {
      TimedLaunch tl(MOE_K_ROUTER_BWD, c.stream);
      bf16_t* dlb = reinterpret_cast<bf16_t*>(ws.logits);
      const int64_t n = (int64_t)s.T * s.E;
      const int cgrid = (int)std::min<int64_t>((n / 8 + 255) / 256, (int64_t)c.num_cus * 16);
      hipLaunchKernelGGL(to_bf16_rows, dim3(cgrid), dim3(256), 0, c.stream, dlogits, n, dlb);
      hipError_t err = hipGetLastError();
      if (err != hipSuccess) return err;
      err = launch_router_bwd_packed(c, s, dlb, (const bf16_t*)wr_packed, dx, true);
      if (err != hipSuccess) return err;
    }
    return launch_unpermute(c, s, dx_rows, slot, dx, true);
  }
  TimedLaunch tl(MOE_K_ROUTER_BWD, c.stream);
  if (s.dtype == MOE_BF16 && s.E % 64 == 0) {
    using Cfg = TileCfg<128, 128>;
    bf16_t* dlb = reinterpret_cast<bf16_t*>(ws.logits);  // [T, E] f32 scratch holds the bf16 rows
    const int64_t n = (int64_t)s.T * s.E;                 // a multiple of 64
    const int cgrid = (int)std::min<int64_t>((n / 8 + 255) / 256, (int64_t)c.num_cus * 16);
    hipLaunchKernelGGL(to_bf16_rows, dim3(cgrid), dim3(256), 0, c.stream, dlogits, n, dlb);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    if (wr_packed) return launch_router_bwd_packed(c, s, dlb, (const bf16_t*)wr_packed, dx);
    const int nt = (s.d + Cfg::BN - 1) / Cfg::BN;
    const int items = ((s.T + Cfg::BM - 1) / Cfg::BM) * nt;
    const int grid = std::min(((items + 7) / 8) * 8, c.num_cus * 2);
    RouterBwdProb<Cfg> pb{dlb, (const bf16_t*)w_router, s.T, s.E, s.d, nt, dx};
    hipLaunchKernelGGL(router_bwd_bf16<Cfg>, dim3(grid), dim3(256), Cfg::SMEM_BYTES, c.stream, pb, items);
    return hipGetLastError();
  }
  const int grid = c.num_cus * 4;
  if (s.dtype == MOE_BF16)
    hipLaunchKernelGGL(router_bwd_simple<bf16_t>, dim3(grid), dim3(256), 0, c.stream, dlogits,
                       (const bf16_t*)w_router, s.T, s.E, s.d, dx);
  else
    hipLaunchKernelGGL(router_bwd_simple<float>, dim3(grid), dim3(256), 0, c.stream, dlogits,
                       (const float*)w_router, s.T, s.E, s.d, dx);
  return hipGetLastError();
}

}  // namespace moe
