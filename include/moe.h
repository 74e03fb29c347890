/* moe.h -- C ABI of the MI355X (gfx950) fine-grained mixture-of-experts layer.
 *
 * The layer is the NanoColibri / HYV3 MoE FFN described in the seventnews
 * article "A relay race of rented GPUs trained NanoColibri's 2.7B MoE for $200"
 * (opening section, architecture paragraph): a sigmoid-plus-bias router over
 * E routed experts with top-k selection, fine-grained SwiGLU experts of width
 * F on hidden size d, an always-resident shared expert of width Fs, a weighted
 * combine, and the aux-loss-free balancing step bias += gamma*sign(target-load).
 *
 * Conventions shared by every entry point
 *  - Every data pointer is a DEVICE pointer owned by the caller, unless the
 *    comment says (host).  The caller keeps buffers alive until the work on
 *    `stream` has finished.
 *  - `stream` is a hipStream_t passed as void*; NULL is the default stream.
 *    Every call only enqueues work on it and returns: no synchronisation, no
 *    allocation, no host<->device copies.  The one exception is the expert
 *    cache (moe_cache_*), which keeps its own host bookkeeping and enqueues
 *    host -> device fills of the experts it streams.
 *  - Arguments are checked on the host before anything is enqueued.  A failed
 *    check returns an error status and enqueues nothing.  MOE_E_DEVICE means a
 *    launch was rejected by the runtime (hipGetLastError after enqueueing).
 *  - Layouts are row-major with the contraction dimension last ("weight rows
 *    are dot-product rows").  act = MOE_F32 means float32, MOE_BF16 bfloat16.
 *  - Supported shapes: 0 <= T, 1 <= E <= 64, 1 <= k <= min(E, 8),
 *    d % 128 == 0, F % 64 == 0, Fs % 64 == 0, T*k*max(d, 2F) < 2^31.
 *  - Outputs may not overlap inputs or each other (MOE_E_ALIAS).
 *  - Non-finite inputs give undefined (but memory-safe) results.
 */
#ifndef FGMOE_MOE_H
#define FGMOE_MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOE_OK = 0,
  MOE_E_ARG = 1,          /* null pointer, negative or inconsistent size        */
  MOE_E_UNSUPPORTED = 2,  /* valid but outside the supported shapes / dtypes    */
  MOE_E_WORKSPACE = 3,    /* workspace missing or smaller than required         */
  MOE_E_ALIAS = 4,        /* an output overlaps an input or another output      */
  MOE_E_DEVICE = 5        /* the HIP runtime rejected a launch                  */
} moe_status;

typedef enum { MOE_F32 = 0, MOE_BF16 = 1, MOE_INT4_G128 = 2, MOE_BF16_STAGED = 3 } moe_dtype;

/* (host) Layer sizes.  T tokens, d hidden, E routed experts of width F, one
 * shared expert of width Fs, top-k.  act: dtype of x, y, the router and the
 * shared expert.  w_routed: dtype of the routed expert weights, equal to act,
 * or MOE_INT4_G128 (requires act = MOE_BF16 and k = 1: top-1 serving), or
 * MOE_BF16_STAGED: bf16 routed weights in the stage-major layout written by
 * moe_pack_routed_bf16 (requires act = MOE_BF16, d % 256 == 0, F % 128 == 0;
 * inference only: moe_backward and training forwards return
 * MOE_E_UNSUPPORTED). */
typedef struct {
  int32_t T, d, E, F, Fs, k;
  int32_t act;
  int32_t w_routed;
} moe_dims;

/* (host struct of device pointers) Layer weights.
 *  w_router     [E, d]                       act
 *  w_gate_up    [E, 2F, d]                   act; rows 0..F-1 gate, F..2F-1 up
 *               int4: packed uint8 [E, 2F, d/2], element 2i in the low nibble
 *  w_down       [E, d, F]                    act; int4: packed uint8 [E, d, F/2]
 *  s_gate_up    int4 only: bf16 scales [E, 2F, d/128]   (else ignored)
 *  s_down       int4 only: bf16 scales [E, d, F/128]    (else ignored)
 *  w_sh_gate_up [2Fs, d]                     act; rows 0..Fs-1 gate, Fs.. up
 *  w_sh_down    [d, Fs]                      act
 * int4 format (an assumed container; the article says only "int4"):
 * symmetric, one bf16 scale per 128 consecutive elements of a row,
 * w = q * scale with q a two's-complement nibble in [-8, 7]. */
typedef struct moe_weights {
  const void* w_router;
  const void* w_gate_up;
  const void* w_down;
  const void* s_gate_up;
  const void* s_down;
  const void* w_sh_gate_up;
  const void* w_sh_down;
  /* Optional (null: none).  The weights of the layer the caller runs next on
   * the same stream, with the same dims: a prefetch hint for a stack of
   * layers, whose weights do not depend on the activations.  The int4 top-1
   * serving path (w_routed = MOE_INT4_G128, T <= 64) reads next's router and
   * shared gate/up rows during its last launch, each weight block through
   * the XCD whose L2 the next layer's first launch reads it through, so the
   * next call finds them in cache.  Results never depend on it; other paths
   * ignore it.  The struct is read during the call only (a captured graph
   * keeps the device pointers it held). */
  const struct moe_weights* next;
} moe_weights;

/* (host struct of device pointers) Routing produced by moe_route/moe_forward.
 *  idx     [T, k] int32   selected experts, largest s+b first, ties -> lower e
 *  gate    [T, k] float   s_idx / sum of selected s (exactly 1 when k = 1)
 *  counts  [E]    int32   load of each expert: number of (t, j) picking it
 *  offsets [E+1]  int32   exclusive prefix sum of counts
 *  perm    [T*k]  int32   slot -> t*k + j; slots of expert e are
 *                         offsets[e] .. offsets[e+1]-1, ascending in t*k + j
 *  pos     [T, k] int32   (t, j) -> slot, the inverse of perm */
typedef struct {
  int32_t* idx;
  float* gate;
  int32_t* counts;
  int32_t* offsets;
  int32_t* perm;
  int32_t* pos;
} moe_routing;

/* (host struct of device pointers) Weight gradients, float32, same shapes as
 * the weights (act layouts).  Overwritten, not accumulated. */
typedef struct {
  float* dw_router;
  float* dw_gate_up;
  float* dw_down;
  float* dw_sh_gate_up;
  float* dw_sh_down;
} moe_grads;

/* Bytes of device workspace that moe_route / moe_forward / moe_backward need
 * for these dims (training = 1 adds the activations moe_backward reads).
 * Returns 0 when the dims are invalid or unsupported. */
size_t moe_workspace_bytes(const moe_dims* dims, int training);

/* Router only: logits x.W_r, s = sigmoid, top-k on s + bias, normalised gates,
 * per-expert loads, offsets and the dispatch order (architecture paragraph:
 * sigmoid-plus-bias router, top-2).  For callers that must know the selected
 * experts before computing them (the streaming engine of the proof-of-loop
 * paragraph).  ws: at least moe_workspace_bytes(dims, 0). */
moe_status moe_route(const moe_dims* dims, const void* x, const void* w_router, const float* bias,
                     const moe_routing* out, void* ws, size_t ws_bytes, void* stream);

/* The layer: y_t = Shared(x_t) + sum_j gate_tj * Expert_{idx_tj}(x_t), with
 * Expert(x) = W_d (silu(W_g x) * (W_u x)) and the shared expert ungated
 * (architecture and proof-of-loop paragraphs; the top-2 paragraph of the
 * "Relay training" section names the routing weight).  x, y: [T, d] act.
 * bias: [E] float32, read only (moe_bias_update changes it).  routing: filled
 * as by moe_route.  training = 1 stores in ws what moe_backward needs.
 * With w_routed = MOE_INT4_G128 this is the top-1 serving path (k = 1,
 * gate = 1; F % 128 == 0, else MOE_E_UNSUPPORTED).  Up to 64 tokens at the
 * NanoColibri shape (d = 1024, F = 512, Fs = 2048) the int4 experts are
 * dequantised inside the decode kernels; every other batch (the prefill,
 * and small batches of other shapes) runs the grouped GEMMs, which expand
 * each int4 operand fragment to bf16(q * scale) in registers (one rounding
 * of an exact product; d and F up to 3072, above that the experts that
 * received tokens are first dequantised to bf16 in the workspace). */
moe_status moe_forward(const moe_dims* dims, const void* x, const moe_weights* w, const float* bias,
                       void* y, const moe_routing* routing, int training,
                       void* ws, size_t ws_bytes, void* stream);

/* One training step's forward and bias step in one call (architecture
 * paragraph: the expert bias is nudged after each batch; the "Relay
 * training" section's top-2 paragraph watches the dead-expert fraction):
 * moe_forward with the current bias, then
 *   bias[e] <- fl32(bias[e] + gamma * sign(T*k - E * counts[e]))
 * and, when stats is not NULL, stats[0..3] = the balance figures of
 * moe_bias_update_stats.  The same results, bit for bit, as moe_forward
 * followed by moe_bias_update_stats (moe_bias_update when stats is NULL),
 * with one launch fewer (the launch that knows the loads takes the step).
 *  bias   [E] float32 (device), read by the router, then updated in place;
 *         must not be NULL (MOE_E_ARG)
 *  stats  [4] float32 (device, written) or NULL
 * bias and stats may overlap no other argument (MOE_E_ALIAS).  The other
 * arguments, shapes and statuses are moe_forward's. */
moe_status moe_forward_bias_step(const moe_dims* dims, const void* x, const moe_weights* w, float* bias,
                                 float gamma, float* stats, void* y, const moe_routing* routing, int training,
                                 void* ws, size_t ws_bytes, void* stream);

/* moe_forward for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc.  There
 * is no workspace argument; the workspace is a static device array of
 * MOE_NOALLOC_SCRATCH_BYTES (8 MiB) that the library holds on every GPU it
 * runs on until the process ends.  No hipMalloc, hipFree or other allocating
 * call is made.  Inference only (training = 0).  Dims whose
 * moe_workspace_bytes(dims, 0) exceeds the array return MOE_E_WORKSPACE
 * before anything is enqueued (at the NanoColibri shape: the bf16 layer up to
 * 512 tokens, the int4 top-1 serving path up to 64 tokens).  Every call on a
 * GPU uses that GPU's one array: calls that overlap on one GPU (two streams,
 * two threads) race and give wrong results, so serialise them.  Nothing the
 * forward reads from the array is left over from an earlier call.  The other
 * arguments, outputs and statuses are moe_forward's. */
#define MOE_NOALLOC_SCRATCH_BYTES (8u << 20)
moe_status moe_forward_noalloc(const moe_dims* dims, const void* x, const moe_weights* w, const float* bias,
                               void* y, const moe_routing* routing, void* stream);

/* Expert streaming (the opening section's proof-of-loop paragraph: a token
 * touches the resident shared expert plus a couple of small routed experts
 * streamed from larger storage).  moe_forward on the int4 top-1 decode path
 * (w_routed = MOE_INT4_G128, T <= 64 at the decode kernels' shape; else
 * MOE_E_UNSUPPORTED) with the routed
 * weights held in n_slots slots: w->w_gate_up, s_gate_up, w_down, s_down are
 * [n_slots, ...] arrays in the moe_weights int4 layout, and expert e's
 * weights are in slot slot[e].
 *  slot     [E] int32 (device, read): every expert the batch routes to must
 *           have its weights in the slot named (moe_cache_prepare arranges
 *           it); entries are clamped to [0, n_slots), so a stale table gives
 *           wrong rows, never an out-of-range read
 *  n_slots  1 .. E (else MOE_E_ARG)
 * Everything else is moe_forward's (no training). */
moe_status moe_forward_cached(const moe_dims* dims, const void* x, const moe_weights* w, const int32_t* slot,
                              int32_t n_slots, const float* bias, void* y, const moe_routing* routing,
                              void* ws, size_t ws_bytes, void* stream);

/* (host) The expert cache that fills those slots: least-recently-used
 * replacement over n_slots slots, filled from a pinned host copy of all E
 * experts.  Per step: moe_route, copy counts to the host, moe_cache_prepare,
 * then moe_forward_cached on the same stream.
 *  moe_cache_create: dims of the layer (int4 routed, E <= 64, d and F
 *    multiples of 128); host: the int4 fields (w_gate_up, s_gate_up, w_down,
 *    s_down) point to pinned host arrays of all E experts; dev: the same
 *    fields point to device arrays of n_slots slots; dev_slot: [E] int32
 *    device.  The caller owns all of them and keeps them alive.  flags: 0, or
 *    MOE_CACHE_DRY_RUN (bookkeeping only: no copies, no launches; pointers
 *    may be NULL), or MOE_CACHE_COPY_FILLS (fill misses with hipMemcpyAsync
 *    even where one launch could read the host copy in place); other bits
 *    are MOE_E_ARG.  Starts empty.
 *  moe_cache_prepare: host_counts [E] (host) = the batch's loads.  Experts
 *    with a load that are resident are kept; each other one (in ascending
 *    order) takes a free slot, else the slot whose last use is oldest among
 *    those the batch does not need (lowest slot first among equals); its four
 *    arrays are copied host -> slot on stream (one launch for all misses, or
 *    hipMemcpyAsync calls: moe_cache_state), then the slot table is rewritten
 *    by one small launch.  *misses (may be NULL) =
 *    this step's misses.  More experts with a load than slots:
 *    MOE_E_UNSUPPORTED, nothing changed.
 *  moe_cache_state: slot_of [E] (host, may be NULL) = each expert's slot or
 *    -1; hits_misses [3] (host, may be NULL) = hits and misses since
 *    creation, then 1 if misses are filled by one launch that reads the host
 *    copy in place (the runtime maps it at the same address on the device),
 *    0 if by hipMemcpyAsync calls.
 *  moe_cache_destroy: frees the bookkeeping (not the caller's buffers). */
typedef struct moe_expert_cache moe_expert_cache;
enum { MOE_CACHE_DRY_RUN = 1, MOE_CACHE_COPY_FILLS = 2 };
moe_status moe_cache_create(const moe_dims* dims, int32_t n_slots, const moe_weights* host, const moe_weights* dev,
                            int32_t* dev_slot, int32_t flags, moe_expert_cache** out);
moe_status moe_cache_prepare(moe_expert_cache* cache, const int32_t* host_counts, void* stream, int32_t* misses);
moe_status moe_cache_state(const moe_expert_cache* cache, int32_t* slot_of, int64_t* hits_misses);
void moe_cache_destroy(moe_expert_cache* cache);

/* The MoE block around the layer, as the architecture paragraph places the
 * layer in 23 of the model's 24 transformer layers (pre-norm and residual:
 * this library's reading):
 *   x     = bf16(h / sqrt(mean_i h_i^2 + eps) * norm_weight)   (RMSNorm, per token row)
 *   h_out = h + MoE(x), summed in fp32 with the layer's combine and rounded once.
 * h, h_out: [T, d] bf16 (device), must not overlap (MOE_E_ALIAS); norm_weight:
 * [d] float32 (device); eps >= 0.  bf16 activations only, d <= 8192
 * (MOE_E_UNSUPPORTED otherwise); no training mode.  x is kept in the
 * workspace (moe_workspace_bytes(dims, 0) bytes); routing and bias as in
 * moe_forward (the routing of x).  With w_routed = MOE_INT4_G128 this is the
 * top-1 serving path of moe_forward with the same norm and residual. */
moe_status moe_forward_block(const moe_dims* dims, const void* h, const float* norm_weight, float eps,
                             const moe_weights* w, const float* bias, void* h_out, const moe_routing* routing,
                             void* ws, size_t ws_bytes, void* stream);

/* Aux-loss-free balancing step (architecture paragraph, DeepSeek-V3 recipe):
 * bias[e] <- fl32(bias[e] + gamma * sign(total_assignments - E * counts[e])),
 * i.e. the target load total_assignments/E compared exactly in integers,
 * sign(0) = 0, one float32 addition.  counts: [E] int32 (device, e.g. the
 * routing of the forward that used the old bias); bias: [E] float32 in/out.
 * total_assignments = T*k of that forward. */
moe_status moe_bias_update(int32_t E, int64_t total_assignments, const int32_t* counts, float gamma,
                           float* bias, void* stream);

/* The same bias step in the same launch, plus the batch's expert-balance
 * figures, which the article's "Relay training" section watches (the top-2
 * paragraph: a low dead-expert fraction under aux-loss-free balancing; the
 * baton paragraph: expert balance on the training dashboard).  stats: [4]
 * float32 (device, caller-owned; e.g. row `step` of a [steps, 4] buffer, so a
 * loop of steps needs no host synchronisation), written as
 *   stats[0] = (experts with counts[e] == 0) / E,
 *   stats[1] = max_e counts[e] * E / total_assignments   (max over mean load),
 *   stats[2] = -sum_e p_e ln p_e, p_e = counts[e] / total_assignments
 *              (0 ln 0 = 0; nats),
 *   stats[3] = stats[2] / ln E (1 when E = 1);
 * total_assignments = 0 gives (1, 0, 0, 0).  fp32, reductions in a fixed
 * order (run-to-run identical).  Errors as moe_bias_update; stats may not
 * overlap counts or bias (MOE_E_ALIAS), a null stats is MOE_E_ARG. */
moe_status moe_bias_update_stats(int32_t E, int64_t total_assignments, const int32_t* counts, float gamma,
                                 float* bias, float* stats, void* stream);

/* Backward of a training moe_forward with the selection held fixed: dx [T, d]
 * act, and the float32 weight gradients.  The router gradient flows only
 * through the normalised gates (top-2 paragraph of the "Relay training"
 * section: with k = 1 it is zero).  x, w, routing: those of the forward; ws:
 * the workspace that forward filled (training = 1), unchanged since. */
moe_status moe_backward(const moe_dims* dims, const void* x, const moe_weights* w,
                        const moe_routing* routing, const void* dy, void* dx, const moe_grads* dw,
                        void* ws, size_t ws_bytes, void* stream);

/* int4 export of expert weights into the container that MOE_INT4_G128 reads
 * (the article's opening section, proof-of-loop paragraph, says the
 * containers are int4; the format is this library's reading, as described at
 * moe_weights): per group of 128 consecutive elements of a row,
 *   scale = absmax / 7 rounded once to bf16 (ties to even), 0 for an all-zero group,
 *   q     = clamp(round-half-even(w / scale), -8, 7), a two's-complement nibble,
 * with both decisions taken in float64 from the exact inputs.
 *  dtype   MOE_BF16 or MOE_F32 (else MOE_E_UNSUPPORTED)
 *  w       [rows, K] dtype, row-major (device, read only); K % 128 == 0 (else
 *          MOE_E_UNSUPPORTED); for a layer: rows = E * 2F, K = d (gate/up) or
 *          rows = E * d, K = F (down)
 *  packed  [rows, K/2] uint8 (device, written): element 2i in the low nibble
 *  scales  [rows, K/128] bf16 (device, written)
 * rows = 0 does nothing.  Outputs may not overlap w or each other
 * (MOE_E_ALIAS).  Inputs are finite with absmax / 7 in bf16's normal range
 * (or zero); other values are not checked. */
moe_status moe_quantize_int4(int32_t dtype, const void* w, int64_t rows, int32_t K, uint8_t* packed,
                             void* scales, void* stream);

/* Routed bf16 expert weights into the stage-major layout that w_routed =
 * MOE_BF16_STAGED reads (a storage order of the same matrices, for the
 * routed experts of the article's layer; the values are copied unchanged).
 * The grouped GEMM streams each 256-row weight tile in contraction chunks of
 * 32 elements; in row-major order such a chunk is 64 bytes from each of 256
 * rows 2 KiB or 1 KiB apart, which HBM serves less efficiently than one
 * contiguous 16 KiB block.  The packed arrays hold, per expert, per 256-row
 * tile, per chunk, the tile's 256 row pieces in the order the kernel places
 * them in LDS.  Pack once when the weights are loaded.
 *  dims         act = MOE_BF16, d % 256 == 0, F % 128 == 0 (else
 *               MOE_E_UNSUPPORTED); T and w_routed are ignored
 *  w_gate_up    [E, 2F, d] bf16 row-major, as moe_weights (device, read only)
 *  w_down       [E, d, F]  bf16 row-major (device, read only)
 *  out_gate_up  E * 2F * d bf16 (device, written): pass it as w_gate_up
 *  out_down     E * d * F  bf16 (device, written): pass it as w_down
 * Outputs may not overlap the inputs or each other (MOE_E_ALIAS). */
moe_status moe_pack_routed_bf16(const moe_dims* dims, const void* w_gate_up, const void* w_down, void* out_gate_up,
                                void* out_down, void* stream);

/* Instrumentation, not part of the layer.  moe_forward (bias_step = 0; gamma
 * and stats ignored) or moe_forward_bias_step (bias_step = 1) that also
 * records the caller's hipEvent_t handles events[0 .. n_events-1] (passed
 * as void*, n_events 0..8) on `stream` at its phase boundaries:
 *   0 before the router, 1 after routing and dispatch bookkeeping (the int4
 *   decode: after the whole forward and its bias step),
 *   2 after the gate/up launch (routed and shared experts together),
 *   3 after the down launch (routed and shared together), 4 after the combine.
 * Boundaries beyond n_events are not recorded.  Nothing is kept after the
 * call returns (no process-wide state); the caller owns the events.  A null
 * entry among the first n_events, n_events outside 0..8, or bias_step not 0
 * or 1 is MOE_E_ARG; otherwise the statuses of the call it instruments. */
moe_status moe_forward_events(const moe_dims* dims, const void* x, const moe_weights* w, float* bias,
                              int32_t bias_step, float gamma, float* stats, void* y, const moe_routing* routing,
                              int training, void* ws, size_t ws_bytes, void* stream, void* const* events,
                              int32_t n_events);

/* Static, NUL-terminated description of a status code. */
const char* moe_status_str(moe_status s);

#ifdef __cplusplus
}
#endif

#endif /* FGMOE_MOE_H */
