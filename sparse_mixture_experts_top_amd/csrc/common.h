// Internal declarations shared by the kernels and the host entry points.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>

#include <algorithm>
#include <stdint.h>

#include "moe.h"

namespace moe {

typedef uint16_t bf16_t;  // bfloat16 bit pattern in memory
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
// 16 bytes as a native vector (HIP's uint4 is a struct, which keeps arrays of
// it from being promoted to registers).
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

// ---------------------------------------------------------------- numbers ---

__device__ __forceinline__ float bf16_to_f32(bf16_t h) {
  return __uint_as_float(static_cast<uint32_t>(h) << 16);
}

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

// Round to nearest, ties to even: gfx950's packed convert instruction
// (v_cvt_pk_bf16_f32), which rounds exactly like the textbook bit
// manipulation (u + 0x7fff + lsb) >> 16 for every finite value and infinity.
__device__ __forceinline__ uint32_t f32x2_to_bf16x2(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t{a, b}), bf16x2_t));
}
__device__ __forceinline__ bf16_t f32_to_bf16(float v) {
  return static_cast<bf16_t>(f32x2_to_bf16x2(v, 0.f));
}

template <class T> __device__ __forceinline__ float load_f(const T* p);
template <> __device__ __forceinline__ float load_f<float>(const float* p) { return *p; }
template <> __device__ __forceinline__ float load_f<bf16_t>(const bf16_t* p) { return bf16_to_f32(*p); }

template <class T> __device__ __forceinline__ void store_f(T* p, float v);
template <> __device__ __forceinline__ void store_f<float>(float* p, float v) { *p = v; }
template <> __device__ __forceinline__ void store_f<bf16_t>(bf16_t* p, float v) { *p = f32_to_bf16(v); }

__device__ __forceinline__ float silu_f(float a) { return a / (1.0f + expf(-a)); }

// A 16-byte store with the non-temporal hint: the L2 keeps the line only
// until it needs the space, so rows written once and read by a later
// kernel do not push out data the writing kernel still reuses.
__device__ __forceinline__ void store16_nt(void* p, uint4 v) {
  __builtin_nontemporal_store(u32x4{v.x, v.y, v.z, v.w}, reinterpret_cast<u32x4*>(p));
}

// Four floats -> four bf16 (round to nearest even) packed in 8 bytes.
__device__ __forceinline__ uint2 pack4_bf16(float a, float b, float c, float d) {
  return make_uint2(f32x2_to_bf16x2(a, b), f32x2_to_bf16x2(c, d));
}

// LoRA terms of one lane's four consecutive output columns n .. n+3 for one
// row with rank-r projection z (fp32, r values): t[q] = sum_c z[c] W[n+q][c]
// for an adapter W stored [N, r] (w_n = W + n r), or t[q] = sum_c z[c]
// A[c][n+q] for one stored [r, N] with row stride lda (a_n = A + n). At r = 16
// the operands arrive in 16-byte (z, W) or 8-byte (A) loads.
__device__ __forceinline__ float bf16_lane(uint32_t w, int hi) {
  return bf16_to_f32(static_cast<bf16_t>(hi ? (w >> 16) : w));
}
__device__ __forceinline__ void lora_term_rows(const float* z, const bf16_t* w_n, int r, float (&t)[4]) {
  t[0] = t[1] = t[2] = t[3] = 0.f;
  if (r == 16) {
    // four ranks at a time: one 16-byte load of z, one 8-byte load per column
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const float4 zz = reinterpret_cast<const float4*>(z)[u];
      uint2 wv[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) wv[q] = *reinterpret_cast<const uint2*>(w_n + q * 16 + 4 * u);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        t[q] = fmaf(zz.x, bf16_lane(wv[q].x, 0), t[q]);
        t[q] = fmaf(zz.y, bf16_lane(wv[q].x, 1), t[q]);
        t[q] = fmaf(zz.z, bf16_lane(wv[q].y, 0), t[q]);
        t[q] = fmaf(zz.w, bf16_lane(wv[q].y, 1), t[q]);
      }
    }
    return;
  }
  for (int c = 0; c < r; ++c)
#pragma unroll
    for (int q = 0; q < 4; ++q) t[q] = fmaf(z[c], bf16_to_f32(w_n[q * r + c]), t[q]);
}
__device__ __forceinline__ void lora_term_cols(const float* z, const bf16_t* a_n, int64_t lda, int r,
                                               float (&t)[4]) {
  t[0] = t[1] = t[2] = t[3] = 0.f;
  if (r == 16) {
    // four ranks at a time: one 16-byte load of z, one 8-byte load per rank
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const float4 zz = reinterpret_cast<const float4*>(z)[u];
      const float zc[4] = {zz.x, zz.y, zz.z, zz.w};
      uint2 av[4];
#pragma unroll
      for (int c = 0; c < 4; ++c) av[c] = *reinterpret_cast<const uint2*>(a_n + (4 * u + c) * lda);
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        t[0] = fmaf(zc[c], bf16_lane(av[c].x, 0), t[0]);
        t[1] = fmaf(zc[c], bf16_lane(av[c].x, 1), t[1]);
        t[2] = fmaf(zc[c], bf16_lane(av[c].y, 0), t[2]);
        t[3] = fmaf(zc[c], bf16_lane(av[c].y, 1), t[3]);
      }
    }
    return;
  }
  for (int c = 0; c < r; ++c)
#pragma unroll
    for (int q = 0; q < 4; ++q) t[q] = fmaf(z[c], bf16_to_f32(a_n[c * lda + q]), t[q]);
}

// Index of the row block containing row p: largest le with off[le] <= p
// (off has L+1 non-decreasing entries, off[0] = 0, p < off[L]).
__device__ __forceinline__ int segment_of(const int32_t* off, int L, int p) {
  int lo = 0, hi = L;  // invariant: off[lo] <= p < off[hi]
  while (hi - lo > 1) {
    int mid = (lo + hi) >> 1;
    if (off[mid] <= p) lo = mid; else hi = mid;
  }
  return lo;
}

// Wave-uniform read of data no kernel writes while this one runs (written by
// an earlier kernel on the stream): through the constant address space with a
// uniform index, so it becomes a scalar load and never waits on vector memory.
typedef const __attribute__((address_space(4))) int32_t* const_i32_ptr_t;
typedef int32_t i32x16_t __attribute__((ext_vector_type(16), aligned(4)));
typedef const __attribute__((address_space(4))) i32x16_t* const_i32x16_ptr_t;
__device__ __forceinline__ int ld_uniform(const int32_t* p, int idx) {
  return ((const_i32_ptr_t)p)[__builtin_amdgcn_readfirstlane(idx)];
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, kWave);
  return v;
}

// ------------------------------------------------------------- host side ---

struct Ctx {
  hipStream_t stream;
  int num_cus;
};

// Kernel timing hooks (api.cpp). begin/end bracket one launch.
void timing_begin(int kid, hipStream_t s);
void timing_end(int kid, hipStream_t s);

struct TimedLaunch {
  int kid;
  hipStream_t s;
  TimedLaunch(int k, hipStream_t st) : kid(k), s(st) { timing_begin(kid, s); }
  ~TimedLaunch() { timing_end(kid, s); }
};

// Workspace carve-up (api.cpp).
struct Workspace {
  int32_t* tile_counts;  // [ntok_tiles, E]
  int32_t* tile_base;    // [ntok_tiles, E]
  int32_t* cseg;         // [L+1]   candidate segment offsets (capacity)
  uint32_t* cand_key;    // [T*k]   gate bits of candidates (capacity)
  int32_t* cand_idx;     // [T*k]   assignment index t*k+j (capacity)
  int32_t* gemm_tiles;   // [max_tiles*2 + 1] (expert, row0) pairs + count at the end
  void* hbuf;            // H in the shape's dtype: [Rmax, f], or tile-packed (bf16 without adapters)
  float* zu;             // [Rmax, rmax] LoRA X A_up^T
  float* zd;             // [Rmax, rmax] LoRA H A_down^T
  float* wproj;          // [Rmax, rmax] LoRA dO B_down
  float* vproj;          // [Rmax, rmax] LoRA dU B_up
  float* du;             // [Rmax, f]   LoRA backward dU (f32)
  bf16_t* lora_mt;       // [L, r, max(d, f)] a [K, r] adapter transposed for the rank-r projections
  bf16_t* lora_mt2;      // [L, r, max(d, f)] the adapter backward's B_up made K-contiguous
  bf16_t* lora_mt3;      // [L, max(d, f), r] the adapter backward's A_down as [L, f, r] rows
  bf16_t* zx;            // [Rmax, 2r] s Z as bf16 high | low parts (the extra adapter K step)
  float* logits;         // [T, E]
  float* prob_part;      // [prob_blocks, E]
  // token remapping (capacity > 0): the all-expert pass and the proposals
  int32_t* rm_offsets1;  // [E+1]
  int32_t* rm_slot1;     // [T*k]
  int32_t* rm_src1;      // [min(T*k, E*C)]
  float* rm_gate1;       // [min(T*k, E*C)]
  int32_t* rm_idx2;      // [T*k]
  float* rm_key2;        // [T*k]
  int32_t* rm_counts2;   // [E]
  int64_t dispatch_bytes;  // the leading part dispatch uses (tile_counts .. cand_idx)
  int64_t bytes;           // all of it (0 when carved with dispatch_only)
};

constexpr int kTokTile = 32;       // tokens per dispatch tile (one 32-bit mask per expert)
constexpr int kTopkTokPerWaveProb = 2;  // tokens per top-k wave when softmax sums are kept
constexpr int kGemmBM = 128;       // grouped GEMM row tile

// dispatch_only: lay out the leading dispatch part only (no pointer past it
// is formed), for a scratch area that holds just that part.
Workspace carve_workspace(const moe_shape_t& s, int lora_r, void* base, bool dispatch_only = false);
int64_t max_rows(const moe_shape_t& s);
int gemm_max_tiles(const moe_shape_t& s);
// Row-tile height of the forward grouped GEMMs for a shape (128, or 320
// where each expert expects a few hundred rows), and the bf16 elements of
// H in its tile-packed layout (each 320-row tile owns BM x f elements; 0 for
// the 128-row tiles, which keep H row-major).
int gemm_tile_rows(const moe_shape_t& s);
int64_t packed_h_elems(const moe_shape_t& s);

// ------------------------------------------------------ kernel launchers ---
// Each returns hipSuccess or the launch error.

// zero / zero_n: an int32 buffer the router kernel clears on the side (the
// per-tile expert histogram that the top-k kernel then fills).
hipError_t launch_router(const Ctx& c, const moe_shape_t& s, const void* x, const void* w,
                         const float* bias, float* logits, int32_t* zero = nullptr, int64_t zero_n = 0);
hipError_t launch_router_mnk(const Ctx& c, int M, int N, int K, const bf16_t* x, const bf16_t* w,
                             const float* bias, float* logits, bf16_t* out_b, int32_t* zero = nullptr,
                             int64_t zero_n = 0);
// hist: per 32-token tile expert counts [ceil(T/32), E], cleared beforehand,
// to which each token adds its k selections.
hipError_t launch_topk(const Ctx& c, const moe_shape_t& s, const float* logits, int32_t* idx,
                       float* gate, float* prob_part, float* prob_sum, int32_t* alt = nullptr,
                       int32_t* hist = nullptr);
hipError_t launch_aux(const Ctx& c, const moe_shape_t& s, const int32_t* counts,
                      const float* prob_sum, float coef, float* out);

hipError_t launch_dispatch_remap(const Ctx& c, const moe_shape_t& s, const Workspace& ws, const int32_t* idx,
                                 const float* gate, const int32_t* alt, const void* x, int32_t* counts,
                                 int32_t* offsets, int32_t* slot, int32_t* row_src, float* row_gate, void* x_perm,
                                 int32_t* moved, int32_t* dropped);
hipError_t launch_dispatch(const Ctx& c, const moe_shape_t& s, const Workspace& ws,
                           const int32_t* idx, const float* gate, const void* x, int32_t* counts,
                           int32_t* offsets, int32_t* slot, int32_t* row_src, float* row_gate,
                           void* x_perm, int32_t* dropped, bool hist_done = false);

struct LoraArgs {
  int r;
  float scale;
  const bf16_t* a_up;
  const bf16_t* b_up;
  const bf16_t* a_down;
  const bf16_t* b_down;
  float* z_save;  // [2, Rmax, r] f32 | NULL: Z_u then Z_d, kept from forward to backward
};

hipError_t launch_expert_gemm(const Ctx& c, const moe_shape_t& s, const Workspace& ws,
                              const void* x_rows, const int32_t* row_src, const int32_t* offsets,
                              const void* gu_packed, const void* d_packed, const void* w_gate,
                              const void* w_up, const void* w_down, const LoraArgs* lora,
                              void* act_save, void* y_perm);

hipError_t launch_pack(const Ctx& c, const moe_shape_t& s, const void* w_gate, const void* w_up,
                       const void* w_down, void* gu_packed, void* d_packed);

// Row tiles of bm rows (kGemmBM unless the GEMM that reads the list uses
// another tile height; max_tiles from gemm_max_tiles bounds any bm >= kGemmBM).
hipError_t launch_row_tiles(const Ctx& c, const int32_t* offsets, int L, int max_tiles,
                            int32_t* tiles, int bm = kGemmBM);

hipError_t launch_combine(const Ctx& c, const moe_shape_t& s, const void* y_perm,
                          const int32_t* slot, const float* gate, void* y);

hipError_t launch_lora_bwd(const Ctx& c, const moe_shape_t& s, const Workspace& ws,
                           const LoraArgs& lo, const bf16_t* dy, const int32_t* offsets,
                           const int32_t* row_src, const float* row_gate, const bf16_t* x_rows,
                           const int32_t* x_src,
                           const bf16_t* act_save, const bf16_t* w_down, float* da_up,
                           float* db_up, float* da_down, float* db_down,
                           const bf16_t* dgu_packed = nullptr);
// dU of the LoRA backward on the packed W_d^T (expert_gemm.hip)
// adt: A_d^T [L, f, 16] (lora_transpose_rn) to carry the adapter term as an
// extra K step whose A operand is ws.zx (s dY B_d, high/low), or NULL for the
// fp32 epilogue term from ws.wproj
hipError_t launch_lora_dh_packed(const Ctx& c, const moe_shape_t& s, const Workspace& ws, const LoraArgs& lo,
                                 const bf16_t* dy, const int32_t* row_src, const float* row_gate,
                                 const int32_t* offsets, const bf16_t* act_save, const bf16_t* dgu_packed,
                                 const bf16_t* adt);
hipError_t launch_lora_transpose_rn(const Ctx& c, const bf16_t* A, int L, int r, int N, bf16_t* At);

hipError_t launch_gate_bwd(const Ctx& c, const moe_shape_t& s, const void* dy, const void* y_perm,
                           const int32_t* slot, const int32_t* idx, const float* gate,
                           const float* logits, const int32_t* counts, float aux_coef, float* dgate,
                           float* dlogits);

hipError_t launch_expert_bwd(const Ctx& c, const moe_shape_t& s, const Workspace& ws, const LoraArgs* lo,
                             const void* dy, const int32_t* offsets, const int32_t* row_src,
                             const float* row_gate, const int32_t* slot, const void* act_save,
                             const void* w_gate, const void* w_up, const void* w_down,
                             const void* dgu_packed, const void* dx_packed, void* dgu, float* dx_rows,
                             float* dx);

hipError_t launch_bwd_gemms_packed(const Ctx& c, const moe_shape_t& s, const Workspace& ws, const LoraArgs* lo,
                                   const bf16_t* dy, const int32_t* row_src, const float* row_gate,
                                   const int32_t* offsets, const bf16_t* act_save, const bf16_t* dgu_packed,
                                   const bf16_t* dx_packed, bf16_t* dgu, float* dx_rows);

hipError_t launch_pack_bwd(const Ctx& c, const moe_shape_t& s, const void* w_gate, const void* w_up,
                           const void* w_down, void* dgu_packed, void* dx_packed);

hipError_t launch_pack_router_bwd(const Ctx& c, const moe_shape_t& s, const void* w_router, void* wr_packed);
// dx += dl . W_r, or with store set dx = dl . W_r (dx not read)
hipError_t launch_router_bwd_packed(const Ctx& c, const moe_shape_t& s, const bf16_t* dl, const bf16_t* wr_packed,
                                    float* dx, bool store = false);

// dx[t] = sum over the token's kept slots j, in j order, of dx_rows[slot];
// with add, dx[t] += that sum for tokens with a kept slot, others untouched
hipError_t launch_unpermute(const Ctx& c, const moe_shape_t& s, const float* dx_rows, const int32_t* slot,
                            float* dx, bool add);

hipError_t launch_router_bwd(const Ctx& c, const moe_shape_t& s, const Workspace& ws, const float* dlogits,
                             const void* w_router, const void* wr_packed, float* dx,
                             const float* dx_rows = nullptr, const int32_t* slot = nullptr);

// LoRA building blocks shared by the forward (expert_gemm) and the backward.
// out[p, q] = scale_p * sum_i in[src(p), i] * M(le(p), q, i) for rows p < R.
//   m_qk: M stored [L, r, K] (true) or [L, K, r] (false)
//   mt:   scratch of L * r * K bf16 for M transposed to [L, r, K] when it is
//         stored [L, K, r] (the matrix-core path reads K-contiguous rows), or
//         NULL (then such an M takes the plain per-row path)
//   out_hl: if not NULL, hl_scale * in[src_p] . M (without the row scale)
//         is also written there as [rows, 2r] bf16: the bf16 rounding in
//         columns [0, r) and the bf16 rounding of the remainder in [r, 2r)
//         (matrix-core path only; hipErrorInvalidValue otherwise); out may
//         then be NULL
template <class TIn>
hipError_t launch_lora_rowproj(const Ctx& c, int L, const int32_t* offsets, int64_t rmax_rows,
                               const TIn* in, int64_t in_stride, const int32_t* src,
                               const float* row_scale, int K, const bf16_t* M, bool m_qk, int r,
                               float* out, bf16_t* mt = nullptr, bf16_t* out_hl = nullptr,
                               float hl_scale = 1.f);

}  // namespace moe
