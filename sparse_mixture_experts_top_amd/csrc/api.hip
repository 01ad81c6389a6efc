// Host side of the C ABI declared in include/moe.h: argument validation,
// workspace layout, per-device launch context, kernel timing, error text.
#include <algorithm>
#include <mutex>
#include <string>
#include <vector>

#include "common.h"

namespace moe {

static thread_local std::string g_error;

static moe_status_t fail(moe_status_t st, const std::string& msg) {
  g_error = msg;
  return st;
}

static int64_t align256(int64_t b) { return (b + 255) & ~int64_t(255); }

int64_t max_rows(const moe_shape_t& s) {
  const int64_t L = s.e_hi - s.e_lo;
  int64_t r = (int64_t)s.T * std::min<int64_t>(s.k, L);
  if (s.capacity > 0) r = std::min<int64_t>(r, L * (int64_t)s.capacity);
  return r;
}

int gemm_max_tiles(const moe_shape_t& s) {
  return (int)((max_rows(s) + kGemmBM - 1) / kGemmBM + (s.e_hi - s.e_lo));
}

Workspace carve_workspace(const moe_shape_t& s, int lora_r, void* base, bool dispatch_only) {
  Workspace w{};
  char* p = static_cast<char*>(base);
  int64_t off = 0;
  auto take = [&](int64_t bytes) -> void* {
    void* q = p ? static_cast<void*>(p + off) : nullptr;
    off += align256(bytes > 0 ? bytes : 1);
    return q;
  };
  const int64_t L = s.e_hi - s.e_lo;
  const int64_t ntok_tiles = (s.T + kTokTile - 1) / kTokTile;
  const int64_t rmax = max_rows(s);
  const int64_t elt = s.dtype == MOE_BF16 ? 2 : 4;
  w.tile_counts = static_cast<int32_t*>(take(ntok_tiles * s.E * 4));
  w.tile_base = static_cast<int32_t*>(take(ntok_tiles * s.E * 4));
  // E + 1 (not L + 1): the all-expert pass of token remapping uses it too
  w.cseg = static_cast<int32_t*>(take(((int64_t)s.E + 1) * 4));
  if (s.capacity > 0) {
    w.cand_key = static_cast<uint32_t*>(take((int64_t)s.T * s.k * 4));
    w.cand_idx = static_cast<int32_t*>(take((int64_t)s.T * s.k * 4));
  }
  // everything dispatch uses lies before this point
  w.dispatch_bytes = off;
  if (dispatch_only) return w;
  if (s.capacity > 0) {
    const int64_t tk = (int64_t)s.T * s.k;
    const int64_t r1 = std::min<int64_t>(tk, (int64_t)s.E * s.capacity);
    w.rm_offsets1 = static_cast<int32_t*>(take(((int64_t)s.E + 1) * 4));
    w.rm_slot1 = static_cast<int32_t*>(take(tk * 4));
    w.rm_src1 = static_cast<int32_t*>(take(r1 * 4));
    w.rm_gate1 = static_cast<float*>(take(r1 * 4));
    w.rm_idx2 = static_cast<int32_t*>(take(tk * 4));
    w.rm_key2 = static_cast<float*>(take(tk * 4));
    w.rm_counts2 = static_cast<int32_t*>(take((int64_t)s.E * 4));
  }
  w.gemm_tiles = static_cast<int32_t*>(take((2 * (int64_t)gemm_max_tiles(s) + 1) * 4));
  w.hbuf = take(std::max(rmax * s.f * elt, s.dtype == MOE_BF16 ? packed_h_elems(s) * 2 : 0));
  if (lora_r > 0) {
    w.zu = static_cast<float*>(take(rmax * lora_r * 4));
    w.zd = static_cast<float*>(take(rmax * lora_r * 4));
    w.wproj = static_cast<float*>(take(rmax * lora_r * 4));
    w.vproj = static_cast<float*>(take(rmax * lora_r * 4));
    w.du = static_cast<float*>(take(rmax * s.f * 4));
    w.lora_mt = static_cast<bf16_t*>(take(L * lora_r * std::max(s.d, s.f) * 2));
    w.lora_mt2 = static_cast<bf16_t*>(take(L * lora_r * std::max(s.d, s.f) * 2));
    w.lora_mt3 = static_cast<bf16_t*>(take(L * lora_r * std::max(s.d, s.f) * 2));
    w.zx = static_cast<bf16_t*>(take(rmax * 2 * lora_r * 2));
  }
  w.logits = static_cast<float*>(take((int64_t)s.T * s.E * 4));
  const int64_t tok_per_blk = 4 * kTopkTokPerWaveProb;
  w.prob_part = static_cast<float*>(take(((int64_t)s.T + tok_per_blk - 1) / tok_per_blk * s.E * 4));
  w.bytes = off;
  return w;
}

// ------------------------------------------------------------ validation ---

static moe_status_t check_shape(const moe_shape_t* s) {
  if (!s) return fail(MOE_ERR_INVALID_ARG, "shape is NULL");
  if (s->T < 0) return fail(MOE_ERR_INVALID_ARG, "T < 0");
  if (s->d < 1 || s->E < 1 || s->f < 1) return fail(MOE_ERR_INVALID_ARG, "d, E and f must be >= 1");
  if (s->k < 1 || s->k > s->E) return fail(MOE_ERR_INVALID_ARG, "k must be in [1, E]");
  if (s->e_lo < 0 || s->e_hi > s->E || s->e_lo >= s->e_hi)
    return fail(MOE_ERR_INVALID_ARG, "local experts [e_lo, e_hi) must be a non-empty range inside [0, E)");
  if (s->dtype != MOE_F32 && s->dtype != MOE_BF16) return fail(MOE_ERR_INVALID_ARG, "dtype must be MOE_F32 or MOE_BF16");
  if ((int64_t)s->T * s->k >= (int64_t(1) << 31)) return fail(MOE_ERR_INVALID_ARG, "T*k must be < 2^31");
  if (s->E > 1024) return fail(MOE_ERR_UNSUPPORTED, "E > 1024");
  if (s->k > 32) return fail(MOE_ERR_UNSUPPORTED, "k > 32");
  if (s->dtype == MOE_BF16 && (s->d % 64 != 0 || s->f % 64 != 0))
    return fail(MOE_ERR_UNSUPPORTED, "bf16 needs d % 64 == 0 and f % 64 == 0");
  return MOE_OK;
}

static LoraArgs lora_args(const moe_lora_t* lo) {
  LoraArgs la{};
  if (!lo) return la;
  la.r = lo->r;
  la.scale = lo->alpha / (float)lo->r;
  la.a_up = static_cast<const bf16_t*>(lo->a_up);
  la.b_up = static_cast<const bf16_t*>(lo->b_up);
  la.a_down = static_cast<const bf16_t*>(lo->a_down);
  la.b_down = static_cast<const bf16_t*>(lo->b_down);
  la.z_save = lo->z_save;
  return la;
}

static moe_status_t check_lora(const moe_shape_t& s, const moe_lora_t* lo) {
  if (!lo) return MOE_OK;
  if (lo->r < 1) return fail(MOE_ERR_INVALID_ARG, "LoRA rank must be >= 1");
  if (!lo->a_up || !lo->b_up || !lo->a_down || !lo->b_down)
    return fail(MOE_ERR_INVALID_ARG, "LoRA adapter pointer is NULL");
  if (lo->r > 64) return fail(MOE_ERR_UNSUPPORTED, "LoRA rank > 64");
  if (s.dtype != MOE_BF16) return fail(MOE_ERR_UNSUPPORTED, "LoRA needs dtype MOE_BF16");
  return MOE_OK;
}

#define MOE_REQUIRE(ptr, name) \
  if (!(ptr)) return fail(MOE_ERR_INVALID_ARG, std::string(name) + " is NULL")
// Buffers sized by T (or by the row bound) may be NULL when that size is 0.
#define MOE_REQUIRE_IF(cond, ptr, name) \
  if ((cond) && !(ptr)) return fail(MOE_ERR_INVALID_ARG, std::string(name) + " is NULL")

static moe_status_t check_ws(const moe_shape_t& s, int lora_r, const void* ws, size_t ws_bytes) {
  const int64_t need = carve_workspace(s, lora_r, nullptr).bytes;
  if (!ws) return fail(MOE_ERR_INVALID_ARG, "ws is NULL");
  if ((reinterpret_cast<uintptr_t>(ws) & 255) != 0) return fail(MOE_ERR_INVALID_ARG, "ws must be 256-byte aligned");
  if ((int64_t)ws_bytes < need)
    return fail(MOE_ERR_WORKSPACE, "ws has " + std::to_string(ws_bytes) + " bytes, needs " + std::to_string(need));
  return MOE_OK;
}

// ----------------------------------------------------------- device info ---

static moe_status_t make_ctx(moe_stream_t stream, Ctx* c) {
  static std::mutex mu;
  static int cus[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64)
    return fail(MOE_ERR_HIP, "hipGetDevice failed (no HIP device?)");
  {
    std::lock_guard<std::mutex> g(mu);
    if (cus[dev] == 0) {
      int n = 0;
      if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
        return fail(MOE_ERR_HIP, "hipDeviceGetAttribute(MultiprocessorCount) failed");
      cus[dev] = (n + 3) & ~3;  // persistent grids of 2 per CU stay a multiple of 8
    }
    c->num_cus = cus[dev];
  }
  c->stream = reinterpret_cast<hipStream_t>(stream);
  return MOE_OK;
}

static moe_status_t hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return MOE_OK;
  return fail(MOE_ERR_HIP, std::string(what) + ": " + hipGetErrorString(e));
}

// ---------------------------------------------------------------- timing ---

namespace {
struct Timing {
  std::mutex mu;
  bool on = false;
  uint32_t mask = 0;  // bit k: kernel kind k is timed
  std::vector<hipEvent_t> pool;
  std::vector<std::pair<hipEvent_t, hipEvent_t>> pending[MOE_K_COUNT];
  double total_ms[MOE_K_COUNT] = {};
  int64_t launches[MOE_K_COUNT] = {};
};
Timing& timing() {
  static Timing t;
  return t;
}
thread_local hipEvent_t t_open[MOE_K_COUNT] = {};

// Events come only from the pool moe_timing_enable fills, so an entry point
// never creates one; with every pooled event pending, the sample is skipped.
hipEvent_t take_event(Timing& t) {
  if (t.pool.empty()) return nullptr;
  hipEvent_t e = t.pool.back();
  t.pool.pop_back();
  return e;
}

void drain(Timing& t, int kid) {
  for (auto& pr : t.pending[kid]) {
    float ms = 0.f;
    if (hipEventSynchronize(pr.second) == hipSuccess &&
        hipEventElapsedTime(&ms, pr.first, pr.second) == hipSuccess) {
      t.total_ms[kid] += ms;
      t.launches[kid] += 1;
    }
    t.pool.push_back(pr.first);
    t.pool.push_back(pr.second);
  }
  t.pending[kid].clear();
}
}  // namespace

void timing_begin(int kid, hipStream_t s) {
  Timing& t = timing();
  std::lock_guard<std::mutex> g(t.mu);
  if (!t.on || !((t.mask >> kid) & 1u)) return;
  hipEvent_t e = take_event(t);
  if (!e) return;
  if (hipEventRecord(e, s) == hipSuccess) t_open[kid] = e;
  else t.pool.push_back(e);
}

void timing_end(int kid, hipStream_t s) {
  Timing& t = timing();
  std::lock_guard<std::mutex> g(t.mu);
  hipEvent_t start = t_open[kid];
  t_open[kid] = nullptr;
  if (!t.on || !start) return;
  hipEvent_t e = take_event(t);
  if (e && hipEventRecord(e, s) == hipSuccess) {
    t.pending[kid].push_back({start, e});
    return;
  }
  // no end event: the sample is dropped and its events go back to the pool
  t.pool.push_back(start);
  if (e) t.pool.push_back(e);
}

// ------------------------------------------- library-owned dispatch scratch ---
// moe_dispatch_noalloc's scratch: the leading dispatch part of the workspace
// layout (per-tile expert histograms, their scan, with a capacity the
// candidate keys), in a device array the library owns. Each device holds its
// own copy from the first use until the process ends. In host code the name
// `scratch` is only a host-side stand-in for the symbol: its device address
// comes from hipGetSymbolAddress, once per device, and only that address is
// handed to kernels.
static __device__ __align__(256) unsigned char scratch[MOE_DISPATCH_NOALLOC_SCRATCH_BYTES];

static moe_status_t scratch_on_current_device(void** out) {
  static std::mutex mu;
  static void* ptr[64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64)
    return fail(MOE_ERR_HIP, "hipGetDevice failed (no HIP device?)");
  std::lock_guard<std::mutex> g(mu);
  if (!ptr[dev]) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(MOE_ERR_HIP, std::string("hipGetSymbolAddress(scratch): ") + hipGetErrorString(e));
    ptr[dev] = p;
  }
  *out = ptr[dev];
  return MOE_OK;
}

}  // namespace moe

using namespace moe;

// ============================================================== C ABI ======

extern "C" {

size_t moe_workspace_bytes(const moe_shape_t* shape, int32_t lora_r) {
  if (check_shape(shape) != MOE_OK || lora_r < 0 || lora_r > 64) return 0;
  return (size_t)carve_workspace(*shape, lora_r, nullptr).bytes;
}

int64_t moe_max_rows(const moe_shape_t* shape) {
  if (check_shape(shape) != MOE_OK) return -1;
  return max_rows(*shape);
}

const char* moe_last_error(void) { return g_error.c_str(); }

moe_status_t moe_route(const moe_shape_t* shape, const void* x, const void* w_router,
                       const float* bias, int32_t* topk_idx, float* topk_gate, float* logits,
                       float* prob_sum, void* ws, size_t ws_bytes, moe_stream_t stream) {
  moe_status_t st = check_shape(shape);
  if (st != MOE_OK) return st;
  const moe_shape_t& s = *shape;
  MOE_REQUIRE_IF(s.T > 0, x, "x");
  MOE_REQUIRE(w_router, "w_router");
  MOE_REQUIRE_IF(s.T > 0, topk_idx, "topk_idx");
  MOE_REQUIRE_IF(s.T > 0, topk_gate, "topk_gate");
  if ((st = check_ws(s, 0, ws, ws_bytes)) != MOE_OK) return st;
  Ctx c;
  if ((st = make_ctx(stream, &c)) != MOE_OK) return st;
  const Workspace w = carve_workspace(s, 0, ws);
  float* lg = logits ? logits : w.logits;
  if (s.T > 0) {
    if ((st = hip_status(launch_router(c, s, x, w_router, bias, lg), "router GEMM")) != MOE_OK) return st;
  }
  return hip_status(launch_topk(c, s, lg, topk_idx, topk_gate, w.prob_part, prob_sum), "top-k");
}

moe_status_t moe_route_alt(const moe_shape_t* shape, const void* x, const void* w_router, const float* bias,
                           int32_t* topk_idx, float* topk_gate, int32_t* alt_idx, float* logits, float* prob_sum,
                           void* ws, size_t ws_bytes, moe_stream_t stream) {
  moe_status_t st = check_shape(shape);
  if (st != MOE_OK) return st;
  const moe_shape_t& s = *shape;
  if (2 * s.k > s.E || 2 * s.k > 32)
    return fail(MOE_ERR_UNSUPPORTED, "alternates need 2k <= E and 2k <= 32");
  MOE_REQUIRE_IF(s.T > 0, x, "x");
  MOE_REQUIRE(w_router, "w_router");
  MOE_REQUIRE_IF(s.T > 0, topk_idx, "topk_idx");
  MOE_REQUIRE_IF(s.T > 0, topk_gate, "topk_gate");
  MOE_REQUIRE_IF(s.T > 0, alt_idx, "alt_idx");
  if ((st = check_ws(s, 0, ws, ws_bytes)) != MOE_OK) return st;
  Ctx c;
  if ((st = make_ctx(stream, &c)) != MOE_OK) return st;
  const Workspace w = carve_workspace(s, 0, ws);
  float* lg = logits ? logits : w.logits;
  if (s.T > 0) {
    if ((st = hip_status(launch_router(c, s, x, w_router, bias, lg), "router GEMM")) != MOE_OK) return st;
  }
  return hip_status(launch_topk(c, s, lg, topk_idx, topk_gate, w.prob_part, prob_sum, alt_idx), "top-k");
}

moe_status_t moe_route_latent(const moe_shape_t* shape, int32_t d_c, const void* x, const void* w_latent,
                              const void* w_router, const float* bias, void* z, int32_t* topk_idx,
                              float* topk_gate, float* logits, float* prob_sum, void* ws, size_t ws_bytes,
                              moe_stream_t stream) {
  moe_status_t st = check_shape(shape);
  if (st != MOE_OK) return st;
  const moe_shape_t& s = *shape;
  if (s.dtype != MOE_BF16) return fail(MOE_ERR_UNSUPPORTED, "the latent router needs dtype MOE_BF16");
  if (d_c < 64 || d_c % 64 != 0) return fail(MOE_ERR_UNSUPPORTED, "the latent width d_c must be a positive multiple of 64");
  MOE_REQUIRE_IF(s.T > 0, x, "x");
  MOE_REQUIRE(w_latent, "w_latent");
  MOE_REQUIRE(w_router, "w_router");
  MOE_REQUIRE_IF(s.T > 0, z, "z");
  MOE_REQUIRE_IF(s.T > 0, topk_idx, "topk_idx");
  MOE_REQUIRE_IF(s.T > 0, topk_gate, "topk_gate");
  if ((st = check_ws(s, 0, ws, ws_bytes)) != MOE_OK) return st;
  Ctx c;
  if ((st = make_ctx(stream, &c)) != MOE_OK) return st;
  const Workspace w = carve_workspace(s, 0, ws);
  float* lg = logits ? logits : w.logits;
  if (s.T > 0) {
    bf16_t* zb = static_cast<bf16_t*>(z);
    if ((st = hip_status(launch_router_mnk(c, s.T, d_c, s.d, (const bf16_t*)x, (const bf16_t*)w_latent, nullptr,
                                           nullptr, zb),
                         "latent projection")) != MOE_OK)
      return st;
    if ((st = hip_status(launch_router_mnk(c, s.T, s.E, d_c, zb, (const bf16_t*)w_router, bias, lg, nullptr),
                         "router GEMM")) != MOE_OK)
      return st;
  }
  return hip_status(launch_topk(c, s, lg, topk_idx, topk_gate, w.prob_part, prob_sum), "top-k");
}

moe_status_t moe_dispatch_remap(const moe_shape_t* shape, const int32_t* topk_idx, const float* topk_gate,
                                const int32_t* alt_idx, const void* x, int32_t* counts, int32_t* offsets,
                                int32_t* slot, int32_t* row_src, float* row_gate, void* x_perm, int32_t* moved,
                                int32_t* dropped, void* ws, size_t ws_bytes, moe_stream_t stream) {
  moe_status_t st = check_shape(shape);
  if (st != MOE_OK) return st;
  const moe_shape_t& s = *shape;
  if (s.capacity <= 0) return fail(MOE_ERR_INVALID_ARG, "token remapping needs a capacity > 0");
  if (2 * s.k > s.E) return fail(MOE_ERR_UNSUPPORTED, "alternates need 2k <= E");
  const bool rows = max_rows(s) > 0;
  MOE_REQUIRE_IF(s.T > 0, topk_idx, "topk_idx");
  MOE_REQUIRE_IF(s.T > 0, topk_gate, "topk_gate");
  MOE_REQUIRE_IF(s.T > 0, alt_idx, "alt_idx");
  MOE_REQUIRE_IF(s.T > 0 && x_perm, x, "x");
  MOE_REQUIRE(counts, "counts");
  MOE_REQUIRE(offsets, "offsets");
  MOE_REQUIRE_IF(s.T > 0, slot, "slot");
  MOE_REQUIRE_IF(rows, row_src, "row_src");
  MOE_REQUIRE_IF(rows, row_gate, "row_gate");
  if ((st = check_ws(s, 0, ws, ws_bytes)) != MOE_OK) return st;
  Ctx c;
  if ((st = make_ctx(stream, &c)) != MOE_OK) return st;
  const Workspace w = carve_workspace(s, 0, ws);
  return hip_status(launch_dispatch_remap(c, s, w, topk_idx, topk_gate, alt_idx, x, counts, offsets, slot, row_src,
                                          row_gate, x_perm, moved, dropped),
                    "dispatch with remapping");
}

moe_status_t moe_dispatch(const moe_shape_t* shape, const int32_t* topk_idx,
                          const float* topk_gate, const void* x, int32_t* counts,
                          int32_t* offsets, int32_t* slot, int32_t* row_src, float* row_gate,
                          void* x_perm, int32_t* dropped, void* ws, size_t ws_bytes,
                          moe_stream_t stream) {
  moe_status_t st = check_shape(shape);
  if (st != MOE_OK) return st;
  const moe_shape_t& s = *shape;
  const bool rows = max_rows(s) > 0;
  MOE_REQUIRE_IF(s.T > 0, topk_idx, "topk_idx");
  MOE_REQUIRE_IF(s.T > 0, topk_gate, "topk_gate");
  MOE_REQUIRE_IF(s.T > 0 && x_perm, x, "x");
  MOE_REQUIRE(counts, "counts");
  MOE_REQUIRE(offsets, "offsets");
  MOE_REQUIRE_IF(s.T > 0, slot, "slot");
  MOE_REQUIRE_IF(rows, row_src, "row_src");
  MOE_REQUIRE_IF(rows, row_gate, "row_gate");
  if ((st = check_ws(s, 0, ws, ws_bytes)) != MOE_OK) return st;
  Ctx c;
  if ((st = make_ctx(stream, &c)) != MOE_OK) return st;
  const Workspace w = carve_workspace(s, 0, ws);
  return hip_status(launch_dispatch(c, s, w, topk_idx, topk_gate, x, counts, offsets, slot, row_src,
                                    row_gate, x_perm, dropped),
                    "dispatch");
}

moe_status_t moe_route_dispatch(const moe_shape_t* shape, const void* x, const void* w_router,
                                const float* bias, int32_t* topk_idx, float* topk_gate, float* logits,
                                float* prob_sum, int32_t* counts, int32_t* offsets, int32_t* slot,
                                int32_t* row_src, float* row_gate, void* x_perm, int32_t* dropped,
                                void* ws, size_t ws_bytes, moe_stream_t stream) {
  moe_status_t st = check_shape(shape);
  if (st != MOE_OK) return st;
  const moe_shape_t& s = *shape;
  const bool rows = max_rows(s) > 0;
  MOE_REQUIRE_IF(s.T > 0, x, "x");
  MOE_REQUIRE(w_router, "w_router");
  MOE_REQUIRE_IF(s.T > 0, topk_idx, "topk_idx");
  MOE_REQUIRE_IF(s.T > 0, topk_gate, "topk_gate");
  MOE_REQUIRE(counts, "counts");
  MOE_REQUIRE(offsets, "offsets");
  MOE_REQUIRE_IF(s.T > 0, slot, "slot");
  MOE_REQUIRE_IF(rows, row_src, "row_src");
  MOE_REQUIRE_IF(rows, row_gate, "row_gate");
  if ((st = check_ws(s, 0, ws, ws_bytes)) != MOE_OK) return st;
  Ctx c;
  if ((st = make_ctx(stream, &c)) != MOE_OK) return st;
  const Workspace w = carve_workspace(s, 0, ws);
  float* lg = logits ? logits : w.logits;
  const int64_t hist_n = (int64_t)((s.T + kTokTile - 1) / kTokTile) * s.E;
  if (s.T > 0) {
    if ((st = hip_status(launch_router(c, s, x, w_router, bias, lg, w.tile_counts, hist_n), "router GEMM")) !=
        MOE_OK)
      return st;
  }
  if ((st = hip_status(launch_topk(c, s, lg, topk_idx, topk_gate, w.prob_part, prob_sum, nullptr, w.tile_counts),
                       "top-k")) != MOE_OK)
    return st;
  return hip_status(launch_dispatch(c, s, w, topk_idx, topk_gate, x, counts, offsets, slot, row_src, row_gate,
                                    x_perm, dropped, true),
                    "dispatch");
}

moe_status_t moe_dispatch_noalloc(const moe_shape_t* shape, const int32_t* topk_idx,
                                  const float* topk_gate, const void* x, int32_t* counts,
                                  int32_t* offsets, int32_t* slot, int32_t* row_src, float* row_gate,
                                  void* x_perm, int32_t* dropped, moe_stream_t stream) {
  moe_status_t st = check_shape(shape);
  if (st != MOE_OK) return st;
  const moe_shape_t& s = *shape;
  const bool rows = max_rows(s) > 0;
  MOE_REQUIRE_IF(s.T > 0, topk_idx, "topk_idx");
  MOE_REQUIRE_IF(s.T > 0, topk_gate, "topk_gate");
  MOE_REQUIRE_IF(s.T > 0 && x_perm, x, "x");
  MOE_REQUIRE(counts, "counts");
  MOE_REQUIRE(offsets, "offsets");
  MOE_REQUIRE_IF(s.T > 0, slot, "slot");
  MOE_REQUIRE_IF(rows, row_src, "row_src");
  MOE_REQUIRE_IF(rows, row_gate, "row_gate");
  const int64_t need = carve_workspace(s, 0, nullptr, true).dispatch_bytes;
  if (need > (int64_t)MOE_DISPATCH_NOALLOC_SCRATCH_BYTES)
    return fail(MOE_ERR_WORKSPACE, "moe_dispatch_noalloc: this shape needs " + std::to_string(need) +
                                       " bytes of scratch, more than the library's " +
                                       std::to_string((int64_t)MOE_DISPATCH_NOALLOC_SCRATCH_BYTES) +
                                       "; use moe_dispatch with a workspace");
  Ctx c;
  if ((st = make_ctx(stream, &c)) != MOE_OK) return st;
  void* base = nullptr;
  if ((st = scratch_on_current_device(&base)) != MOE_OK) return st;
  const Workspace w = carve_workspace(s, 0, base, true);
  return hip_status(launch_dispatch(c, s, w, topk_idx, topk_gate, x, counts, offsets, slot, row_src,
                                    row_gate, x_perm, dropped),
                    "dispatch (no allocation)");
}

moe_status_t moe_expert_gemm(const moe_shape_t* shape, const void* x, const int32_t* row_src,
                             const int32_t* offsets, const void* w_gate, const void* w_up,
                             const void* w_down, const moe_lora_t* lora, void* act_save,
                             void* y_perm, void* ws, size_t ws_bytes, moe_stream_t stream) {
  moe_status_t st = check_shape(shape);
  if (st != MOE_OK) return st;
  const moe_shape_t& s = *shape;
  const bool rows = max_rows(s) > 0;
  MOE_REQUIRE_IF(rows, x, "x");
  MOE_REQUIRE(offsets, "offsets");
  MOE_REQUIRE(w_gate, "w_gate");
  MOE_REQUIRE(w_up, "w_up");
  MOE_REQUIRE(w_down, "w_down");
  MOE_REQUIRE_IF(rows, y_perm, "y_perm");
  if ((st = check_lora(s, lora)) != MOE_OK) return st;
  const int r = lora ? lora->r : 0;
  if ((st = check_ws(s, r, ws, ws_bytes)) != MOE_OK) return st;
  Ctx c;
  if ((st = make_ctx(stream, &c)) != MOE_OK) return st;
  const Workspace w = carve_workspace(s, r, ws);
  const LoraArgs la = lora_args(lora);
  return hip_status(launch_expert_gemm(c, s, w, x, row_src, offsets, nullptr, nullptr, w_gate, w_up, w_down,
                                       lora ? &la : nullptr, act_save, y_perm),
                    "expert GEMM");
}

static moe_status_t check_packable(const moe_shape_t& s) {
  if (s.dtype != MOE_BF16) return fail(MOE_ERR_UNSUPPORTED, "packed weights need dtype MOE_BF16");
  if (s.d % 128 != 0) return fail(MOE_ERR_UNSUPPORTED, "packed weights need d % 128 == 0");
  return MOE_OK;
}

moe_status_t moe_pack_expert_weights(const moe_shape_t* shape, const void* w_gate, const void* w_up,
                                     const void* w_down, void* gu_packed, void* down_packed,
                                     moe_stream_t stream) {
  moe_status_t st = check_shape(shape);
  if (st != MOE_OK) return st;
  const moe_shape_t& s = *shape;
  if ((st = check_packable(s)) != MOE_OK) return st;
  if (!gu_packed && !down_packed) return fail(MOE_ERR_INVALID_ARG, "no output requested");
  MOE_REQUIRE_IF(gu_packed, w_gate, "w_gate");
  MOE_REQUIRE_IF(gu_packed, w_up, "w_up");
  MOE_REQUIRE_IF(down_packed, w_down, "w_down");
  Ctx c;
  if ((st = make_ctx(stream, &c)) != MOE_OK) return st;
  return hip_status(launch_pack(c, s, w_gate, w_up, w_down, gu_packed, down_packed), "pack");
}

moe_status_t moe_expert_gemm_packed(const moe_shape_t* shape, const void* x, const int32_t* row_src,
                                    const int32_t* offsets, const void* gu_packed,
                                    const void* down_packed, const moe_lora_t* lora, void* act_save,
                                    void* y_perm, void* ws, size_t ws_bytes, moe_stream_t stream) {
  moe_status_t st = check_shape(shape);
  if (st != MOE_OK) return st;
  const moe_shape_t& s = *shape;
  if ((st = check_packable(s)) != MOE_OK) return st;
  const bool rows = max_rows(s) > 0;
  MOE_REQUIRE_IF(rows, x, "x");
  MOE_REQUIRE(offsets, "offsets");
  MOE_REQUIRE(gu_packed, "gu_packed");
  MOE_REQUIRE(down_packed, "down_packed");
  MOE_REQUIRE_IF(rows, y_perm, "y_perm");
  if ((st = check_lora(s, lora)) != MOE_OK) return st;
  const int r = lora ? lora->r : 0;
  if ((st = check_ws(s, r, ws, ws_bytes)) != MOE_OK) return st;
  Ctx c;
  if ((st = make_ctx(stream, &c)) != MOE_OK) return st;
  const Workspace w = carve_workspace(s, r, ws);
  const LoraArgs la = lora_args(lora);
  return hip_status(launch_expert_gemm(c, s, w, x, row_src, offsets, gu_packed, down_packed, nullptr,
                                       nullptr, nullptr, lora ? &la : nullptr, act_save, y_perm),
                    "expert GEMM (packed)");
}

moe_status_t moe_combine(const moe_shape_t* shape, const void* y_perm, const int32_t* slot,
                         const float* topk_gate, void* y, moe_stream_t stream) {
  moe_status_t st = check_shape(shape);
  if (st != MOE_OK) return st;
  const moe_shape_t& s = *shape;
  if (s.T == 0) return MOE_OK;
  MOE_REQUIRE_IF(max_rows(s) > 0, y_perm, "y_perm");
  MOE_REQUIRE(slot, "slot");
  MOE_REQUIRE(topk_gate, "topk_gate");
  MOE_REQUIRE(y, "y");
  Ctx c;
  if ((st = make_ctx(stream, &c)) != MOE_OK) return st;
  return hip_status(launch_combine(c, s, y_perm, slot, topk_gate, y), "combine");
}

moe_status_t moe_aux_loss(const moe_shape_t* shape, const int32_t* counts,
                          const float* prob_sum, float coef, float* out, moe_stream_t stream) {
  moe_status_t st = check_shape(shape);
  if (st != MOE_OK) return st;
  MOE_REQUIRE(counts, "counts");
  MOE_REQUIRE(prob_sum, "prob_sum");
  MOE_REQUIRE(out, "out");
  Ctx c;
  if ((st = make_ctx(stream, &c)) != MOE_OK) return st;
  return hip_status(launch_aux(c, *shape, counts, prob_sum, coef, out), "aux loss");
}

moe_status_t moe_lora_bwd(const moe_shape_t* shape, const moe_lora_t* lora, const void* dy,
                          const int32_t* offsets, const int32_t* row_src, const float* row_gate,
                          const void* x, const int32_t* x_src, const void* act_save,
                          const void* w_down, float* da_up, float* db_up, float* da_down, float* db_down, void* ws,
                          size_t ws_bytes, moe_stream_t stream) {
  moe_status_t st = check_shape(shape);
  if (st != MOE_OK) return st;
  const moe_shape_t& s = *shape;
  MOE_REQUIRE(lora, "lora");
  if ((st = check_lora(s, lora)) != MOE_OK) return st;
  const bool rows = max_rows(s) > 0;
  MOE_REQUIRE_IF(s.T > 0, dy, "dy");
  MOE_REQUIRE(offsets, "offsets");
  MOE_REQUIRE_IF(rows, row_src, "row_src");
  MOE_REQUIRE_IF(rows, row_gate, "row_gate");
  MOE_REQUIRE_IF(rows, x, "x");
  MOE_REQUIRE_IF(rows, act_save, "act_save");
  MOE_REQUIRE(w_down, "w_down");
  MOE_REQUIRE(da_up, "da_up");
  MOE_REQUIRE(db_up, "db_up");
  MOE_REQUIRE(da_down, "da_down");
  MOE_REQUIRE(db_down, "db_down");
  if ((st = check_ws(s, lora->r, ws, ws_bytes)) != MOE_OK) return st;
  Ctx c;
  if ((st = make_ctx(stream, &c)) != MOE_OK) return st;
  const Workspace w = carve_workspace(s, lora->r, ws);
  const LoraArgs la = lora_args(lora);
  return hip_status(
      launch_lora_bwd(c, s, w, la, static_cast<const bf16_t*>(dy), offsets, row_src, row_gate,
                      static_cast<const bf16_t*>(x), x_src, static_cast<const bf16_t*>(act_save),
                      static_cast<const bf16_t*>(w_down), da_up, db_up, da_down, db_down),
      "LoRA backward");
}

moe_status_t moe_lora_bwd_packed(const moe_shape_t* shape, const moe_lora_t* lora, const void* dy,
                          const int32_t* offsets, const int32_t* row_src, const float* row_gate,
                          const void* x, const int32_t* x_src, const void* act_save,
                          const void* dgu_packed, float* da_up, float* db_up, float* da_down, float* db_down, void* ws,
                          size_t ws_bytes, moe_stream_t stream) {
  moe_status_t st = check_shape(shape);
  if (st != MOE_OK) return st;
  const moe_shape_t& s = *shape;
  if ((st = check_packable(s)) != MOE_OK) return st;
  if (s.f % 128 != 0) return fail(MOE_ERR_UNSUPPORTED, "packed backward weights need f % 128 == 0");
  MOE_REQUIRE(lora, "lora");
  if ((st = check_lora(s, lora)) != MOE_OK) return st;
  const bool rows = max_rows(s) > 0;
  MOE_REQUIRE_IF(s.T > 0, dy, "dy");
  MOE_REQUIRE(offsets, "offsets");
  MOE_REQUIRE_IF(rows, row_src, "row_src");
  MOE_REQUIRE_IF(rows, row_gate, "row_gate");
  MOE_REQUIRE_IF(rows, x, "x");
  MOE_REQUIRE_IF(rows, act_save, "act_save");
  MOE_REQUIRE(dgu_packed, "dgu_packed");
  MOE_REQUIRE(da_up, "da_up");
  MOE_REQUIRE(db_up, "db_up");
  MOE_REQUIRE(da_down, "da_down");
  MOE_REQUIRE(db_down, "db_down");
  if ((st = check_ws(s, lora->r, ws, ws_bytes)) != MOE_OK) return st;
  Ctx c;
  if ((st = make_ctx(stream, &c)) != MOE_OK) return st;
  const Workspace w = carve_workspace(s, lora->r, ws);
  const LoraArgs la = lora_args(lora);
  return hip_status(
      launch_lora_bwd(c, s, w, la, static_cast<const bf16_t*>(dy), offsets, row_src, row_gate,
                      static_cast<const bf16_t*>(x), x_src, static_cast<const bf16_t*>(act_save),
                      nullptr, da_up, db_up, da_down, db_down, static_cast<const bf16_t*>(dgu_packed)),
      "LoRA backward (packed)");
}

moe_status_t moe_gate_bwd(const moe_shape_t* shape, const void* dy, const void* y_perm,
                          const int32_t* slot, const int32_t* topk_idx, const float* topk_gate,
                          const float* logits, const int32_t* counts, float aux_coef, float* dgate,
                          float* dlogits, moe_stream_t stream) {
  moe_status_t st = check_shape(shape);
  if (st != MOE_OK) return st;
  const moe_shape_t& s = *shape;
  const bool tok = s.T > 0;
  MOE_REQUIRE_IF(tok, dy, "dy");
  MOE_REQUIRE_IF(tok && max_rows(s) > 0, y_perm, "y_perm");
  MOE_REQUIRE_IF(tok, slot, "slot");
  MOE_REQUIRE_IF(tok, topk_idx, "topk_idx");
  MOE_REQUIRE_IF(tok, topk_gate, "topk_gate");
  MOE_REQUIRE_IF(tok && counts && aux_coef != 0.f, logits, "logits");
  MOE_REQUIRE_IF(tok, dlogits, "dlogits");
  Ctx c;
  if ((st = make_ctx(stream, &c)) != MOE_OK) return st;
  return hip_status(launch_gate_bwd(c, s, dy, y_perm, slot, topk_idx, topk_gate, logits, counts, aux_coef,
                                    dgate, dlogits),
                    "gate backward");
}

moe_status_t moe_expert_bwd(const moe_shape_t* shape, const moe_lora_t* lora, const void* dy,
                            const int32_t* offsets, const int32_t* row_src, const float* row_gate,
                            const int32_t* slot, const void* act_save, const void* w_gate,
                            const void* w_up, const void* w_down, void* dgu, float* dx_rows, float* dx,
                            void* ws, size_t ws_bytes, moe_stream_t stream) {
  moe_status_t st = check_shape(shape);
  if (st != MOE_OK) return st;
  const moe_shape_t& s = *shape;
  if ((st = check_lora(s, lora)) != MOE_OK) return st;
  const bool rows = max_rows(s) > 0;
  MOE_REQUIRE_IF(s.T > 0, dy, "dy");
  MOE_REQUIRE(offsets, "offsets");
  MOE_REQUIRE_IF(rows, row_src, "row_src");
  MOE_REQUIRE_IF(rows, row_gate, "row_gate");
  MOE_REQUIRE_IF(s.T > 0, slot, "slot");
  MOE_REQUIRE_IF(rows, act_save, "act_save");
  MOE_REQUIRE(w_gate, "w_gate");
  MOE_REQUIRE(w_up, "w_up");
  MOE_REQUIRE(w_down, "w_down");
  MOE_REQUIRE_IF(rows, dgu, "dgu");
  MOE_REQUIRE_IF(rows, dx_rows, "dx_rows");
  MOE_REQUIRE_IF(s.T > 0, dx, "dx");
  if ((st = check_ws(s, lora ? lora->r : 0, ws, ws_bytes)) != MOE_OK) return st;
  Ctx c;
  if ((st = make_ctx(stream, &c)) != MOE_OK) return st;
  const Workspace w = carve_workspace(s, lora ? lora->r : 0, ws);
  const LoraArgs la = lora_args(lora);
  return hip_status(launch_expert_bwd(c, s, w, lora ? &la : nullptr, dy, offsets, row_src, row_gate, slot,
                                      act_save, w_gate, w_up, w_down, nullptr, nullptr, dgu, dx_rows, dx),
                    "expert backward");
}

moe_status_t moe_pack_backward_weights(const moe_shape_t* shape, const void* w_gate, const void* w_up,
                                       const void* w_down, void* dgu_packed, void* dx_packed,
                                       moe_stream_t stream) {
  moe_status_t st = check_shape(shape);
  if (st != MOE_OK) return st;
  const moe_shape_t& s = *shape;
  if ((st = check_packable(s)) != MOE_OK) return st;
  if (s.f % 128 != 0) return fail(MOE_ERR_UNSUPPORTED, "packed backward weights need f % 128 == 0");
  if (!dgu_packed && !dx_packed) return fail(MOE_ERR_INVALID_ARG, "no output requested");
  MOE_REQUIRE_IF(dx_packed, w_gate, "w_gate");
  MOE_REQUIRE_IF(dx_packed, w_up, "w_up");
  MOE_REQUIRE_IF(dgu_packed, w_down, "w_down");
  Ctx c;
  if ((st = make_ctx(stream, &c)) != MOE_OK) return st;
  return hip_status(launch_pack_bwd(c, s, w_gate, w_up, w_down, dgu_packed, dx_packed), "pack backward");
}

moe_status_t moe_expert_bwd_packed(const moe_shape_t* shape, const moe_lora_t* lora, const void* dy,
                                   const int32_t* offsets, const int32_t* row_src, const float* row_gate,
                                   const int32_t* slot, const void* act_save, const void* dgu_packed,
                                   const void* dx_packed, void* dgu, float* dx_rows, float* dx, void* ws,
                                   size_t ws_bytes, moe_stream_t stream) {
  moe_status_t st = check_shape(shape);
  if (st != MOE_OK) return st;
  const moe_shape_t& s = *shape;
  if ((st = check_packable(s)) != MOE_OK) return st;
  if (s.f % 128 != 0) return fail(MOE_ERR_UNSUPPORTED, "packed backward weights need f % 128 == 0");
  if ((st = check_lora(s, lora)) != MOE_OK) return st;
  const bool rows = max_rows(s) > 0;
  MOE_REQUIRE_IF(s.T > 0, dy, "dy");
  MOE_REQUIRE(offsets, "offsets");
  MOE_REQUIRE_IF(rows, row_src, "row_src");
  MOE_REQUIRE_IF(rows, row_gate, "row_gate");
  MOE_REQUIRE_IF(s.T > 0 && dx, slot, "slot");
  MOE_REQUIRE_IF(rows, act_save, "act_save");
  MOE_REQUIRE(dgu_packed, "dgu_packed");
  MOE_REQUIRE(dx_packed, "dx_packed");
  MOE_REQUIRE_IF(rows, dgu, "dgu");
  MOE_REQUIRE_IF(rows, dx_rows, "dx_rows");
  if ((st = check_ws(s, lora ? lora->r : 0, ws, ws_bytes)) != MOE_OK) return st;
  Ctx c;
  if ((st = make_ctx(stream, &c)) != MOE_OK) return st;
  const Workspace w = carve_workspace(s, lora ? lora->r : 0, ws);
  const LoraArgs la = lora_args(lora);
  // dx null: the per-token sum is left to moe_router_bwd_unpermute_packed
  return hip_status(launch_expert_bwd(c, s, w, lora ? &la : nullptr, dy, offsets, row_src, row_gate, slot,
                                      act_save, nullptr, nullptr, nullptr, dgu_packed, dx_packed, dgu, dx_rows,
                                      dx),
                    "expert backward (packed)");
}

moe_status_t moe_router_bwd(const moe_shape_t* shape, const float* dlogits, const void* w_router,
                            float* dx, void* ws, size_t ws_bytes, moe_stream_t stream) {
  moe_status_t st = check_shape(shape);
  if (st != MOE_OK) return st;
  const moe_shape_t& s = *shape;
  MOE_REQUIRE_IF(s.T > 0, dlogits, "dlogits");
  MOE_REQUIRE(w_router, "w_router");
  MOE_REQUIRE_IF(s.T > 0, dx, "dx");
  if ((st = check_ws(s, 0, ws, ws_bytes)) != MOE_OK) return st;
  Ctx c;
  if ((st = make_ctx(stream, &c)) != MOE_OK) return st;
  const Workspace w = carve_workspace(s, 0, ws);
  return hip_status(launch_router_bwd(c, s, w, dlogits, w_router, nullptr, dx), "router backward");
}

moe_status_t moe_pack_router_bwd(const moe_shape_t* shape, const void* w_router, void* wr_packed,
                                 moe_stream_t stream) {
  moe_status_t st = check_shape(shape);
  if (st != MOE_OK) return st;
  const moe_shape_t& s = *shape;
  if (s.dtype != MOE_BF16 || s.d % 128 != 0 || s.E % 64 != 0)
    return fail(MOE_ERR_UNSUPPORTED, "packed router weights need bf16, d % 128 == 0 and E % 64 == 0");
  MOE_REQUIRE(w_router, "w_router");
  MOE_REQUIRE(wr_packed, "wr_packed");
  Ctx c;
  if ((st = make_ctx(stream, &c)) != MOE_OK) return st;
  return hip_status(launch_pack_router_bwd(c, s, w_router, wr_packed), "pack router");
}

moe_status_t moe_router_bwd_packed(const moe_shape_t* shape, const float* dlogits, const void* wr_packed,
                                   float* dx, void* ws, size_t ws_bytes, moe_stream_t stream) {
  moe_status_t st = check_shape(shape);
  if (st != MOE_OK) return st;
  const moe_shape_t& s = *shape;
  if (s.dtype != MOE_BF16 || s.d % 128 != 0 || s.E % 64 != 0)
    return fail(MOE_ERR_UNSUPPORTED, "packed router weights need bf16, d % 128 == 0 and E % 64 == 0");
  MOE_REQUIRE_IF(s.T > 0, dlogits, "dlogits");
  MOE_REQUIRE(wr_packed, "wr_packed");
  MOE_REQUIRE_IF(s.T > 0, dx, "dx");
  if ((st = check_ws(s, 0, ws, ws_bytes)) != MOE_OK) return st;
  Ctx c;
  if ((st = make_ctx(stream, &c)) != MOE_OK) return st;
  const Workspace w = carve_workspace(s, 0, ws);
  return hip_status(launch_router_bwd(c, s, w, dlogits, nullptr, wr_packed, dx), "router backward (packed)");
}

moe_status_t moe_router_bwd_unpermute_packed(const moe_shape_t* shape, const float* dlogits,
                                             const void* wr_packed, const float* dx_rows, const int32_t* slot,
                                             float* dx, void* ws, size_t ws_bytes, moe_stream_t stream) {
  moe_status_t st = check_shape(shape);
  if (st != MOE_OK) return st;
  const moe_shape_t& s = *shape;
  if (s.dtype != MOE_BF16 || s.d % 128 != 0 || s.E % 64 != 0)
    return fail(MOE_ERR_UNSUPPORTED, "packed router weights need bf16, d % 128 == 0 and E % 64 == 0");
  MOE_REQUIRE_IF(s.T > 0, dlogits, "dlogits");
  MOE_REQUIRE(wr_packed, "wr_packed");
  MOE_REQUIRE_IF(max_rows(s) > 0, dx_rows, "dx_rows");
  MOE_REQUIRE_IF(s.T > 0, slot, "slot");
  MOE_REQUIRE_IF(s.T > 0, dx, "dx");
  if ((st = check_ws(s, 0, ws, ws_bytes)) != MOE_OK) return st;
  Ctx c;
  if ((st = make_ctx(stream, &c)) != MOE_OK) return st;
  const Workspace w = carve_workspace(s, 0, ws);
  return hip_status(launch_router_bwd(c, s, w, dlogits, nullptr, wr_packed, dx, dx_rows, slot),
                    "router backward + unpermute (packed)");
}

moe_status_t moe_timing_enable(int32_t mask) {
  Timing& t = timing();
  std::lock_guard<std::mutex> g(t.mu);
  for (int k = 0; k < MOE_K_COUNT; ++k) {
    drain(t, k);
    t.total_ms[k] = 0.0;
    t.launches[k] = 0;
  }
  if (mask && t.pool.size() < 512) {
    for (int i = 0; i < 512; ++i) {
      hipEvent_t e = nullptr;
      if (hipEventCreate(&e) != hipSuccess) return fail(MOE_ERR_HIP, "hipEventCreate failed");
      t.pool.push_back(e);
    }
  }
  t.on = mask != 0;
  t.mask = (uint32_t)mask;
  return MOE_OK;
}

moe_status_t moe_timing_read(int32_t kernel, double* total_ms, int64_t* launches) {
  if (kernel < 0 || kernel >= MOE_K_COUNT) return fail(MOE_ERR_INVALID_ARG, "unknown kernel id");
  if (!total_ms || !launches) return fail(MOE_ERR_INVALID_ARG, "output pointer is NULL");
  Timing& t = timing();
  std::lock_guard<std::mutex> g(t.mu);
  drain(t, kernel);
  *total_ms = t.total_ms[kernel];
  *launches = t.launches[kernel];
  return MOE_OK;
}

}  // extern "C"
