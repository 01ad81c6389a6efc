/*
 * moe.h -- C ABI of the MI355X (gfx950) sparse MoE layer library.
 *
 * The layer is y = sum_{i in TopK(x)} g_i(x) * E_i(x) ("Adapting Trillion-
 * Parameter MoE Models for LoRA Fine-Tuning: A Full-Stack Engineering Guide",
 * §2.1), with E routed experts of which each token uses k (896 and 16 on "Day-
 * Level Adaptation and LoRA Fine-Tuning of Ultra-Large-Scale Sparse MoE
 * Models", §2.1), computed in four calls that mirror the permute -> grouped
 * GEMM -> unpermute pipeline of "Trillion-Parameter MoE Model Training
 * Adaptation: Full-Stack Optimization Practices", §4.3:
 *
 *   moe_route        router GEMM, softmax, top-k, renormalised gates
 *   moe_dispatch     expert histogram, scan, stable scatter, capacity, row gather
 *   moe_expert_gemm  grouped SwiGLU expert FFN over ragged per-expert row blocks
 *   moe_combine      gate-weighted sum of each token's expert rows
 *
 * plus moe_aux_loss (load-balance loss) and moe_lora_bwd (gradients of the
 * LoRA adapters on the up and down projections).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Pointers are DEVICE pointers unless marked [host]. Matrices are dense and
 *   row-major with no padding; "[a,b]" gives the shape.
 * - Floating tensors use the dtype of moe_shape_t.dtype (fp32 or bf16) unless
 *   stated as f32; indices are int32.
 * - Every call enqueues kernels on `stream` and returns without waiting for
 *   them; nothing synchronises with the host and nothing is allocated or freed
 *   on the device. The caller owns every buffer; the library keeps no pointer
 *   after the call returns.
 * - Sizes that depend on the routing (the number R of dispatched rows) stay on
 *   the device: R = offsets[L]. Buffers sized by moe_max_rows() hold R valid
 *   rows; the rows after R are not written.
 * - `ws` is scratch memory of at least moe_workspace_bytes() bytes, 256-byte
 *   aligned, used by one call at a time; its contents on entry do not matter.
 * - Errors: arguments are validated on the host before anything is enqueued;
 *   a bad argument returns MOE_ERR_INVALID_ARG or MOE_ERR_UNSUPPORTED and
 *   enqueues nothing. A failed launch returns MOE_ERR_HIP. The library never
 *   aborts or prints; moe_last_error() gives the message of the calling
 *   thread's last failure.
 * - Device preconditions (not checked): inputs are finite; topk_idx entries
 *   are in [0, E). Results are deterministic: the same inputs give bitwise the
 *   same outputs on every call.
 * - T == 0 is a valid empty batch: buffers sized by T may be NULL; counts,
 *   offsets, prob_sum and the LoRA gradients are still written (as zeros).
 */
#ifndef MOE_MI355X_H
#define MOE_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ihipStream_t* moe_stream_t; /* a hipStream_t; NULL = the null stream */

typedef enum {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = 1, /* null pointer, inconsistent or out-of-range sizes */
  MOE_ERR_UNSUPPORTED = 2, /* valid but outside what the kernels implement    */
  MOE_ERR_WORKSPACE = 3,   /* ws smaller than moe_workspace_bytes()           */
  MOE_ERR_HIP = 4          /* a HIP runtime call or kernel launch failed      */
} moe_status_t;

typedef enum { MOE_F32 = 0, MOE_BF16 = 1 } moe_dtype_t;

/* Problem shape. Local experts are [e_lo, e_hi): the expert weights passed to
 * the library hold L = e_hi - e_lo experts (local expert le is global expert
 * e_lo + le), as one expert-parallel rank holds E/EP of them ("Fine-Tuning
 * Trillion-Parameter Sparse MoE Models: Challenges and Engineering Practices",
 * §4: 896 / 64 = 14 per rank). Assignments to other experts are not computed.
 *
 * capacity > 0 caps the rows kept per expert ("Adapting Ultra-Large MoE
 * Models: Engineering Practices and Optimization Pathways", §3.3): an expert
 * chosen more than `capacity` times keeps the assignments with the largest
 * gate, equal gates going to the lower token; the rest are dropped.
 *
 * Limits: 1 <= k <= E <= 1024, k <= 32, 0 <= e_lo < e_hi <= E, T*k < 2^31.
 * bf16 additionally needs d % 64 == 0 and f % 64 == 0 (MFMA tiles). */
typedef struct {
  int32_t T;        /* tokens                          */
  int32_t d;        /* hidden size                     */
  int32_t E;        /* routed experts                  */
  int32_t k;        /* experts per token               */
  int32_t f;        /* expert FFN width                */
  int32_t e_lo;     /* first local expert              */
  int32_t e_hi;     /* one past the last local expert  */
  int32_t capacity; /* rows kept per expert, <= 0: all */
  int32_t dtype;    /* moe_dtype_t                     */
} moe_shape_t;

/* LoRA adapters on the up and down projections of every local expert:
 * W' = W0 + (alpha/r) B A ("Adapting Trillion-Parameter MoE Models for LoRA
 * Fine-Tuning: A Full-Stack Engineering Guide", §3). bf16 only, 1 <= r <= 64.
 *   a_up   [L, r, d]   b_up   [L, f, r]     (U  += s (X A_up^T) B_up^T)
 *   a_down [L, r, f]   b_down [L, d, r]     (O  += s (H A_down^T) B_down^T)
 * with s = alpha / r.
 *   z_save [2, Rmax, r] f32 | NULL  (Rmax = moe_max_rows): the rank-r
 *          projections of the rows, Z_u = X A_up^T in z_save[0] and
 *          Z_d = H A_down^T in z_save[1]. moe_expert_gemm(_packed) writes
 *          them; moe_lora_bwd(_packed) then reads them instead of projecting
 *          X and H again (the caller keeps the buffer, the rows and the
 *          adapters unchanged between the two calls). NULL: the backward
 *          recomputes them. */
typedef struct {
  int32_t r;
  float alpha;
  const void* a_up;
  const void* b_up;
  const void* a_down;
  const void* b_down;
  float* z_save;
} moe_lora_t;

/* [host] Scratch bytes every entry point below needs for this shape
 * (lora_r = 0 when no adapters are used). Returns 0 for an invalid shape. */
size_t moe_workspace_bytes(const moe_shape_t* shape, int32_t lora_r);

/* [host] Upper bound on the dispatched rows R: T*min(k, L), or, with a
 * capacity, min(T*min(k, L), L*capacity). Buffers indexed by row (row_src,
 * row_gate, x_perm, act_save, y_perm) need this many rows. -1 if invalid. */
int64_t moe_max_rows(const moe_shape_t* shape);

/* [host] Message of the calling thread's last failed call ("" if none). */
const char* moe_last_error(void);

/* Routing ("Day-Level Adaptation ...", §2.1 and §3.3: routing score, Top-16
 * selection; "Full-Stack Engineering Guide", §2.1: gate score g_i).
 *   x         [T, d]          tokens
 *   w_router  [E, d]          router weight (out x in)
 *   bias      [E] f32 | NULL  per-expert logit bias, added before the softmax
 *   topk_idx  [T, k] int32    OUT: selected experts, descending logit, ties
 *                             to the lower expert id (-0.0 equals +0.0)
 *   topk_gate [T, k] f32      OUT: softmax of the selected logits (the full
 *                             softmax renormalised over the selection)
 *   logits    [T, E] f32|NULL OUT (optional): x w_router^T + bias, fp32
 *                             accumulation; NULL keeps them in ws
 *   prob_sum  [E] f32 | NULL  OUT (optional): sum over tokens of the full
 *                             softmax, for moe_aux_loss
 * Logits are fp32 (bf16 inputs, fp32 accumulation); selection compares the
 * fp32 logits exactly. */
moe_status_t moe_route(const moe_shape_t* shape, const void* x, const void* w_router,
                       const float* bias, int32_t* topk_idx, float* topk_gate,
                       float* logits, float* prob_sum, void* ws, size_t ws_bytes,
                       moe_stream_t stream);

/* moe_route plus the experts ranked next: alt_idx [T, k] int32 OUT holds,
 * for each token, the experts of rank k .. 2k-1 by logit (the same order and
 * tie rule as topk_idx), the candidates moe_dispatch_remap moves
 * overflowing assignments to. topk_idx, topk_gate, logits and prob_sum are
 * those of moe_route. Needs 2k <= E and 2k <= 32 (MOE_ERR_UNSUPPORTED).
 * ("Adapting Ultra-Large MoE Models: Engineering Practices and Optimization
 * Pathways", §3.3: excess tokens are remapped or dropped.) */
moe_status_t moe_route_alt(const moe_shape_t* shape, const void* x, const void* w_router,
                           const float* bias, int32_t* topk_idx, float* topk_gate, int32_t* alt_idx,
                           float* logits, float* prob_sum, void* ws, size_t ws_bytes,
                           moe_stream_t stream);

/* Routing from a low-dimensional projection of the tokens ("Day-Level
 * Adaptation and LoRA Fine-Tuning of Ultra-Large-Scale Sparse MoE Models",
 * §2.1: tokens are first mapped to a more stable low-dimensional
 * representation, then routed):
 *   z = x w_latent^T            z [T, d_c] bf16 OUT (fp32 accumulation,
 *                               rounded to bf16: it feeds the next product)
 *   logits = z w_router^T + bias, then top-k and gates as moe_route.
 *   d_c         latent width, a positive multiple of 64
 *   w_latent    [d_c, d]        w_router [E, d_c]
 * bf16 only (MOE_ERR_UNSUPPORTED otherwise). The other arguments are those
 * of moe_route. */
moe_status_t moe_route_latent(const moe_shape_t* shape, int32_t d_c, const void* x, const void* w_latent,
                              const void* w_router, const float* bias, void* z, int32_t* topk_idx,
                              float* topk_gate, float* logits, float* prob_sum, void* ws, size_t ws_bytes,
                              moe_stream_t stream);

/* Dispatch ("Trillion-Parameter ... Full-Stack Optimization Practices", §3
 * and §4.3: permute tokens by routing result).
 *   topk_idx, topk_gate       from moe_route
 *   x         [T, d]          tokens
 *   counts    [E] int32       OUT: assignments per expert over all T*k,
 *                             before capacity
 *   offsets   [L+1] int32     OUT: row block of local expert le is
 *                             [offsets[le], offsets[le+1]); R = offsets[L]
 *   slot      [T, k] int32    OUT: row of assignment (t, j), or -1 when its
 *                             expert is not local or it was dropped
 *   row_src   [Rmax] int32    OUT: token of each row
 *   row_gate  [Rmax] f32      OUT: gate of each row
 *   x_perm    [Rmax, d]|NULL  OUT (optional): x_perm[p] = x[row_src[p]]
 *                             (bitwise copy); NULL skips the copy, x may
 *                             then be NULL too
 *   dropped   [1] int32|NULL  OUT (optional): local assignments dropped by
 *                             the capacity rule
 * Rows are grouped by local expert ascending and, within an expert, by token
 * ascending; the order never depends on thread timing. */
moe_status_t moe_dispatch(const moe_shape_t* shape, const int32_t* topk_idx,
                          const float* topk_gate, const void* x, int32_t* counts,
                          int32_t* offsets, int32_t* slot, int32_t* row_src, float* row_gate,
                          void* x_perm, int32_t* dropped, void* ws, size_t ws_bytes,
                          moe_stream_t stream);

/* Routing and dispatch as one call ("Day-Level Adaptation and LoRA
 * Fine-Tuning of Ultra-Large-Scale Sparse MoE Models", §3.3: routing score,
 * Top-k selection and expert dispatch merged into a few large kernels). The
 * results equal those of moe_route followed by moe_dispatch with the same
 * arguments, bit for bit; fewer kernels run: the router GEMM also clears the
 * per-tile expert histogram in ws, the top-k kernel adds its selections into
 * it, and the dispatch starts from it (no histogram pass of its own).
 * Arguments: those of moe_route (x .. prob_sum), then those of moe_dispatch
 * (counts .. dropped), then the workspace and stream. */
moe_status_t moe_route_dispatch(const moe_shape_t* shape, const void* x, const void* w_router,
                                const float* bias, int32_t* topk_idx, float* topk_gate, float* logits,
                                float* prob_sum, int32_t* counts, int32_t* offsets, int32_t* slot,
                                int32_t* row_src, float* row_gate, void* x_perm, int32_t* dropped,
                                void* ws, size_t ws_bytes, moe_stream_t stream);

/* Dispatch with token remapping instead of dropping ("Adapting Ultra-Large
 * MoE Models: Engineering Practices and Optimization Pathways", §3.3: excess
 * tokens are remapped or dropped). With C = capacity (> 0, else
 * MOE_ERR_INVALID_ARG):
 *   1. every expert (all E, not only the local ones) keeps its C assignments
 *      with the largest gate, equal gates going to the lower token, as in
 *      moe_dispatch; the others overflow;
 *   2. the m-th overflowing assignment of a token (in j order) is proposed to
 *      alt_idx[t, m] (moe_route_alt), the expert ranked k + m;
 *   3. an expert accepts proposals into the room its kept assignments left,
 *      C - kept, preferring the larger gate, then the lower token; the other
 *      proposals are dropped.
 * An accepted assignment keeps its gate: slot[t, j] then names a row of the
 * alternate expert, and moe_combine / moe_expert_gemm work unchanged. Rows
 * are grouped by local expert and token as in moe_dispatch; a token has at
 * most one row per expert.
 *   counts   [E]        OUT: assignments per expert before capacity (the
 *                       original selection), as in moe_dispatch
 *   moved    [1] | NULL OUT: proposals accepted by local experts
 *   dropped  [1] | NULL OUT: proposals to local experts that were rejected
 * The other arguments are those of moe_dispatch; the workspace of
 * moe_workspace_bytes for a shape with capacity > 0 includes the scratch of
 * the all-expert pass. Needs 2k <= E. */
moe_status_t moe_dispatch_remap(const moe_shape_t* shape, const int32_t* topk_idx, const float* topk_gate,
                                const int32_t* alt_idx, const void* x, int32_t* counts, int32_t* offsets,
                                int32_t* slot, int32_t* row_src, float* row_gate, void* x_perm, int32_t* moved,
                                int32_t* dropped, void* ws, size_t ws_bytes, moe_stream_t stream);

/* moe_dispatch without a workspace argument, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc. Same arguments (minus ws, ws_bytes) and
 * bitwise the same outputs as moe_dispatch. It allocates and frees nothing,
 * not even on its first call: its scratch (per-tile expert histograms and
 * their scan; with a capacity, the candidate gate keys) is a device array of
 * MOE_DISPATCH_NOALLOC_SCRATCH_BYTES bytes that the library owns, one copy on
 * each device it runs on, held until the process ends. A shape needs
 *   2 * a(ceil(T / 32) * E * 4) + a((E + 1) * 4)
 *     + (capacity > 0 ? 2 * a(T * k * 4) : 0)   bytes, a(n) = n rounded up
 * to a multiple of 256; more returns MOE_ERR_WORKSPACE (T = 16384, E = 896:
 * about 3.7 MB). Every word of the scratch is written before it is read, so
 * its contents on entry do not matter; calls on one device share the one
 * array, so calls that overlap on one device (two streams, two threads)
 * race and must be serialised by the caller. */
#define MOE_DISPATCH_NOALLOC_SCRATCH_BYTES ((size_t)16 << 20)
moe_status_t moe_dispatch_noalloc(const moe_shape_t* shape, const int32_t* topk_idx,
                                  const float* topk_gate, const void* x, int32_t* counts,
                                  int32_t* offsets, int32_t* slot, int32_t* row_src, float* row_gate,
                                  void* x_perm, int32_t* dropped, moe_stream_t stream);

/* Grouped expert FFN ("Trillion-Parameter ... Full-Stack Optimization
 * Practices", §3: experts compute in grouped matrix multiplications; SwiGLU
 * expert network). For the rows of local expert le:
 *   G = X w_gate[le]^T, U = X w_up[le]^T (+ LoRA), H = silu(G) * U,
 *   O = H w_down[le]^T (+ LoRA),  silu(a) = a / (1 + exp(-a)).
 *   x        input rows: with row_src, the tokens [T, d] and row p reads
 *            x[row_src[p]] (the dispatch gather happens inside the GEMM's
 *            loads); with row_src == NULL, the permuted rows x_perm [Rmax, d]
 *   row_src  [Rmax] int32 | NULL   from moe_dispatch
 *   offsets  [L+1] int32           from moe_dispatch
 *   w_gate   [L, f, d]        w_up [L, f, d]        w_down [L, d, f]
 *   lora     [host] | NULL    adapters (bf16 only)
 *   act_save [Rmax, 3f]|NULL  OUT (optional): per row G (columns 0..f-1),
 *                             the H fed to the down projection (f..2f-1) and
 *                             U (2f..3f-1, LoRA term included);
 *                             moe_lora_bwd and moe_expert_bwd need it
 *   y_perm   [Rmax, d]        OUT: O per row (not gate-scaled)
 * Accumulation is fp32; in bf16 mode H is rounded to bf16 before the down
 * projection and O is stored as bf16. */
moe_status_t moe_expert_gemm(const moe_shape_t* shape, const void* x, const int32_t* row_src,
                             const int32_t* offsets, const void* w_gate, const void* w_up,
                             const void* w_down, const moe_lora_t* lora, void* act_save,
                             void* y_perm, void* ws, size_t ws_bytes, moe_stream_t stream);

/* Packed expert weights. The expert weights are frozen, so they can be stored
 * once in the order the grouped GEMM streams them: every weight tile one
 * GEMM step reads (128 rows x 32 K values, bf16) becomes one contiguous 8 KB
 * block laid out exactly as it sits in LDS. Packing is a pure permutation
 * (bitwise equal values); packed buffers have the sizes of the originals.
 *   gu_packed   [L, 2f, d] elements: tile (le, b, kt) for b < f/64, kt < d/32
 *               holds rows 16q..16q+15 of w_gate[le] block b and the same
 *               rows of w_up[le], interleaved per 16 (q = 0..3), K values
 *               32kt..32kt+31
 *   down_packed [L, d, f]  elements: tile (le, b, kt) for b < d/128, kt < f/32
 *               holds rows 128b..128b+127 of w_down[le], K values 32kt..32kt+31
 * Within a tile, row r's 16-byte chunk c (K values 8c..8c+7) is stored at
 * chunk position c ^ key(r) of the row, key(r) = (r >> 1) & 3.
 * bf16 only, d % 128 == 0. Either output may be NULL (that input is then
 * not read). */
moe_status_t moe_pack_expert_weights(const moe_shape_t* shape, const void* w_gate, const void* w_up,
                                     const void* w_down, void* gu_packed, void* down_packed,
                                     moe_stream_t stream);

/* moe_expert_gemm with packed weights (same results, bitwise): the weight
 * tiles are read as contiguous blocks. */
moe_status_t moe_expert_gemm_packed(const moe_shape_t* shape, const void* x, const int32_t* row_src,
                                    const int32_t* offsets, const void* gu_packed,
                                    const void* down_packed, const moe_lora_t* lora, void* act_save,
                                    void* y_perm, void* ws, size_t ws_bytes, moe_stream_t stream);

/* Combine ("Full-Stack Engineering Guide", §2.1: results are gathered back
 * and weighted by g_i).
 *   y_perm    [Rmax, d]        from moe_expert_gemm
 *   slot      [T, k] int32     from moe_dispatch
 *   topk_gate [T, k] f32       from moe_route
 *   y         [T, d]           OUT: y[t] = sum_j g[t,j] y_perm[slot[t,j]] over
 *                              slot >= 0, in j order, fp32 accumulation;
 *                              tokens with no slot get zeros */
moe_status_t moe_combine(const moe_shape_t* shape, const void* y_perm, const int32_t* slot,
                         const float* topk_gate, void* y, moe_stream_t stream);

/* Load-balance loss ("Full-Stack Engineering Guide", §2.1 and "Engineering
 * Practices and Optimization Pathways", §3.3: auxiliary loss that encourages
 * uniform routing), as load times probability:
 *   out[1] = E * sum_e (counts[e] / (T k)) * (prob_sum[e] / T),
 *   out[0] = coef * out[1].
 *   counts [E] int32 (moe_dispatch), prob_sum [E] f32 (moe_route), out [2] f32. */
moe_status_t moe_aux_loss(const moe_shape_t* shape, const int32_t* counts,
                          const float* prob_sum, float coef, float* out, moe_stream_t stream);

/* Gradients of the four LoRA adapters for the loss sum(y * dy), with the
 * router, the gates and the base weights frozen ("Full-Stack Engineering
 * Guide", §3; the routing of the forward is reused, never recomputed, as
 * "Day-Level Adaptation ...", §5 advises). With s = alpha/r, for the rows of
 * local expert le, dO[p] = row_gate[p] dy[row_src[p]], Z_u = X A_up^T,
 * Z_d = H A_down^T:
 *   db_down = s dO^T Z_d                 da_down = s (dO B_down)^T H
 *   dH = dO w_down + s (dO B_down) A_down,  dU = dH * silu(G)
 *   db_up   = s dU^T Z_u                 da_up   = s (dU B_up)^T X
 *   dy          [T, d]            upstream gradient of y
 *   offsets, row_src, row_gate    from moe_dispatch
 *   x, x_src                      input rows as for moe_expert_gemm: the
 *                                 tokens [T, d] with x_src = row_src, or
 *                                 x_perm [Rmax, d] with x_src = NULL
 *   act_save    [Rmax, 3f]        from moe_expert_gemm (G, H, U)
 *   w_down      [L, d, f]
 *   da_up [L,r,d], db_up [L,f,r], da_down [L,r,f], db_down [L,d,r]   OUT, f32
 * bf16 only. Every gradient element is written (zero for experts with no
 * rows). */
moe_status_t moe_lora_bwd(const moe_shape_t* shape, const moe_lora_t* lora, const void* dy,
                          const int32_t* offsets, const int32_t* row_src, const float* row_gate,
                          const void* x, const int32_t* x_src, const void* act_save,
                          const void* w_down, float* da_up, float* db_up, float* da_down,
                          float* db_down, void* ws, size_t ws_bytes, moe_stream_t stream);

/* moe_lora_bwd with the frozen w_down's transpose packed once: dgu_packed
 * [L, f, d] elements as written by moe_pack_backward_weights (its dx_packed
 * may be NULL). The dH product then streams contiguous weight tiles on the
 * DMA engine of the forward. Same arguments otherwise (w_down replaced);
 * same results up to the fp32 summation order. bf16 only, d % 128 == 0 and
 * f % 128 == 0 (MOE_ERR_UNSUPPORTED otherwise). */
moe_status_t moe_lora_bwd_packed(const moe_shape_t* shape, const moe_lora_t* lora, const void* dy,
                                 const int32_t* offsets, const int32_t* row_src, const float* row_gate,
                                 const void* x, const int32_t* x_src, const void* act_save,
                                 const void* dgu_packed, float* da_up, float* db_up, float* da_down,
                                 float* db_down, void* ws, size_t ws_bytes, moe_stream_t stream);

/* ---- full backward --------------------------------------------------------
 * Gradients of the loss sum(y * dy) + L_aux for training through the layer
 * ("Full-Stack Engineering Guide", §3: adapters are trained through the
 * frozen MoE layer, which therefore has to pass gradients down; "Full-Stack
 * Optimization Practices", §3: the permute / grouped GEMM / unpermute stages
 * run again in reverse). The router, the gates' selection and the expert
 * weights are frozen; the selection is held (it is piecewise constant).
 *
 * moe_gate_bwd: gate and router-logit gradients.
 *   dy        [T, d]      upstream gradient of y (the shape's dtype)
 *   y_perm    [Rmax, d]   the forward's expert output rows (moe_expert_gemm)
 *   slot      [T, k]      from moe_dispatch
 *   topk_idx, topk_gate   [T, k] from moe_route
 *   logits    [T, E] f32  from moe_route; read only with counts
 *   counts    [E] | NULL  from moe_dispatch: adds the load-balance loss
 *                         gradient (with aux_coef; NULL or coef 0: none)
 *   dgate     [T, k] f32 | NULL  OUT: dg[t,j] = <dy[t], y_perm[slot[t,j]]>
 *                         for kept local slots, else 0
 *   dlogits   [T, E] f32  OUT: dl[t, idx_j] = g_j (dg_j - sum_i g_i dg_i)
 *                         (the gates are the softmax over the selected
 *                         logits), plus, with counts, coef E / T * p_te
 *                         (f_e - sum_e' f_e' p_te'), p = softmax over all E,
 *                         f = counts / (T k) held constant.
 * Every element of dlogits is written. */
moe_status_t moe_gate_bwd(const moe_shape_t* shape, const void* dy, const void* y_perm,
                          const int32_t* slot, const int32_t* topk_idx, const float* topk_gate,
                          const float* logits, const int32_t* counts, float aux_coef, float* dgate,
                          float* dlogits, moe_stream_t stream);

/* moe_expert_bwd: dx through the frozen experts (gates held). Per row p of
 * local expert le, dO = g_p dy[row_src[p]]:
 *   dH = dO w_down[le] (+ s (dO B_down) A_down),
 *   dG = dH * U * silu'(G),  dU = dH * silu(G)   (G, U from act_save),
 *   dX = dG w_gate[le] + dU w_up[le] (+ s (dU B_up) A_up),
 * and dx[t] = sum over the token's kept local slots j, in j order, of dX.
 *   lora      [host] | NULL  adapters of the forward (bf16 only)
 *   dy        [T, d]         upstream gradient (the shape's dtype)
 *   offsets, row_src, row_gate, slot   from moe_dispatch
 *   act_save  [Rmax, 3f]     from moe_expert_gemm
 *   w_gate, w_up [L, f, d], w_down [L, d, f]   row-major (not packed)
 *   dgu       [Rmax, 2f]     scratch (the shape's dtype): dG | dU per row
 *   dx_rows   [Rmax, d] f32  scratch: dX per row
 *   dx        [T, d] f32     OUT (tokens with no kept local slot get 0)
 * bf16 rounds dG and dU to bf16 before the dX product; accumulation is
 * fp32 throughout. */
moe_status_t moe_expert_bwd(const moe_shape_t* shape, const moe_lora_t* lora, const void* dy,
                            const int32_t* offsets, const int32_t* row_src, const float* row_gate,
                            const int32_t* slot, const void* act_save, const void* w_gate,
                            const void* w_up, const void* w_down, void* dgu, float* dx_rows, float* dx,
                            void* ws, size_t ws_bytes, moe_stream_t stream);

/* Packed transposed weights for the backward's grouped GEMMs (frozen, so
 * packed once): the two products contract over the other index of each
 * weight than the forward does, so their streamed operands are the
 * transposes, stored in the tile format of moe_pack_expert_weights' down
 * tiles (128 rows x 32 K values, contiguous 8 KB, chunk c of row r at
 * position c ^ key(r)):
 *   dgu_packed [L, f, d] elements: tile (le, b, kt), b < f/128, kt < d/32:
 *              rows n = 128b..128b+127, K values k = 32kt.., element
 *              w_down[le][k][n]
 *   dx_packed  [L, d, 2f] elements: tile (le, b, kt), b < d/128, kt < 2f/32:
 *              rows n of d, K values k of 2f, element w_gate[le][k][n] for
 *              k < f and w_up[le][k - f][n] otherwise
 * bf16 only, d % 128 == 0 and f % 128 == 0. Either output may be NULL. */
moe_status_t moe_pack_backward_weights(const moe_shape_t* shape, const void* w_gate, const void* w_up,
                                       const void* w_down, void* dgu_packed, void* dx_packed,
                                       moe_stream_t stream);

/* moe_expert_bwd with the packed transposed weights: the two grouped GEMMs
 * stream contiguous weight tiles on the DMA engine of the forward. Same
 * arguments otherwise; same results up to the fp32 summation order. dx may
 * be NULL here (and slot with it): the per-token sum of dx_rows is then
 * skipped, for moe_router_bwd_unpermute_packed to form it. */
moe_status_t moe_expert_bwd_packed(const moe_shape_t* shape, const moe_lora_t* lora, const void* dy,
                                   const int32_t* offsets, const int32_t* row_src, const float* row_gate,
                                   const int32_t* slot, const void* act_save, const void* dgu_packed,
                                   const void* dx_packed, void* dgu, float* dx_rows, float* dx, void* ws,
                                   size_t ws_bytes, moe_stream_t stream);

/* moe_router_bwd: the router's part of dx, dx[t] += sum_e dlogits[t, e]
 * w_router[e] (logits = x w_router^T + bias).
 *   dlogits [T, E] f32 (moe_gate_bwd), w_router [E, d], dx [T, d] f32 IN/OUT.
 * bf16 with E % 64 == 0 rounds dlogits to bf16 (in the workspace's logits
 * area) and multiplies on the matrix cores with fp32 accumulation; other
 * shapes use an fp32 loop. */
moe_status_t moe_router_bwd(const moe_shape_t* shape, const float* dlogits, const void* w_router,
                            float* dx, void* ws, size_t ws_bytes, moe_stream_t stream);

/* The router's transpose packed once for moe_router_bwd_packed (the router
 * is frozen): wr_packed [d, E] elements in the tile format of the packed
 * expert weights, rows n < d, K values e < E, element w_router[e][n].
 * bf16 only, d % 128 == 0, E % 64 == 0. */
moe_status_t moe_pack_router_bwd(const moe_shape_t* shape, const void* w_router, void* wr_packed,
                                 moe_stream_t stream);

/* moe_router_bwd with the packed transpose: dx[t] += sum_e dlogits[t, e]
 * w_router[e] on the DMA engine (dlogits rounded to bf16 in the workspace,
 * fp32 accumulation). */
moe_status_t moe_router_bwd_packed(const moe_shape_t* shape, const float* dlogits, const void* wr_packed,
                                   float* dx, void* ws, size_t ws_bytes, moe_stream_t stream);

/* The two parts of dx in one call: the frozen layer passes gradients down
 * through the experts and through the router ("Adapting Trillion-Parameter
 * MoE Models for LoRA Fine-Tuning: A Full-Stack Engineering Guide", §2.1 and
 * §3), the unpermute and the router product of the reversed pipeline of
 * "Trillion-Parameter MoE Model Training Adaptation: Full-Stack Optimization
 * Practices", §3:
 *   dx[t] = sum over the token's slots j with slot[t, j] >= 0, in j order,
 *           of dx_rows[slot[t, j]]  +  sum_e dlogits[t, e] w_router[e]
 * bitwise equal to moe_expert_bwd_packed's unpermute followed by
 * moe_router_bwd_packed. The product is stored (dx is not read for it),
 * then the rows are added for the tokens that have a kept slot only: where
 * most slots are remote (a local expert range) most of dx is written once
 * and never read. Three kernels on the stream, in order: dlogits to bf16
 * (in the workspace), the product, the row sums.
 *   dlogits [T, E] f32, wr_packed as for moe_router_bwd_packed,
 *   dx_rows [Rmax, d] f32 (moe_expert_bwd_packed with dx NULL; read only
 *   through kept slots; NULL only when Rmax = 0),
 *   slot [T, k] int32 (moe_dispatch), dx [T, d] f32 OUT.
 * bf16 only, d % 128 == 0, E % 64 == 0, else MOE_ERR_UNSUPPORTED. */
moe_status_t moe_router_bwd_unpermute_packed(const moe_shape_t* shape, const float* dlogits,
                                             const void* wr_packed, const float* dx_rows, const int32_t* slot,
                                             float* dx, void* ws, size_t ws_bytes, moe_stream_t stream);

/* ---- kernel timing (profiling aid) -------------------------------------
 * When enabled for a kernel kind, the library records a pair of HIP events
 * on the launch stream around every kernel of that kind it enqueues.
 * moe_timing_read waits for the recorded events and returns the summed
 * duration and the launch count of one kind since the last reset. Each
 * event pair adds a little time between launches, so a measurement of the
 * whole step should enable only the kinds it needs. [host] */
typedef enum {
  MOE_K_ROUTER_GEMM = 0,
  MOE_K_TOPK = 1,
  MOE_K_PROB_REDUCE = 2,
  MOE_K_HIST = 3,
  MOE_K_SCAN = 4,
  MOE_K_SCATTER = 5,
  MOE_K_CAPACITY = 6,
  MOE_K_GATHER = 7,
  MOE_K_TILES = 8,
  MOE_K_GATE_UP = 9,
  MOE_K_DOWN = 10,
  MOE_K_COMBINE = 11,
  MOE_K_AUX = 12,
  MOE_K_LORA_PROJ = 13,
  MOE_K_LORA_DH = 14,
  MOE_K_LORA_GRAD = 15,
  MOE_K_GATE_BWD = 16,
  MOE_K_EXPERT_DGU = 17,
  MOE_K_EXPERT_DX = 18,
  MOE_K_UNPERMUTE = 19,
  MOE_K_ROUTER_BWD = 20,
  MOE_K_COUNT = 21
} moe_kernel_t;

/* mask: bit k (1 << moe_kernel_t) enables timing of kind k; 0 disables all,
 * -1 enables all. Also resets the totals. The events are created here (512
 * of them); the entry points only record pooled events, so they still
 * allocate nothing. A launch whose events find the pool empty (all pending,
 * i.e. more than 256 timed launches since the last moe_timing_read) is not
 * timed and not counted. */
moe_status_t moe_timing_enable(int32_t mask);
moe_status_t moe_timing_read(int32_t kernel, double* total_ms, int64_t* launches);

#ifdef __cplusplus
}
#endif
#endif /* MOE_MI355X_H */
