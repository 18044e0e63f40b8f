/*
 * moe.h -- C interface of the capacity-limited Mixture-of-Experts layer forward pass,
 * hand-written HIP for AMD Instinct MI355X (gfx950, CDNA4).
 *
 * The layer (one token row x of width d_model, E experts, top-k routing, capacity factor C):
 *   1. route     : router logits L = W_r x + b_r, softmax over all E experts, the k largest
 *                  gates, unrenormalised.
 *   2. dispatch  : each expert owns a fixed buffer of `capacity` = floor(C*T*k/E) slots; the
 *                  assignments of an expert fill it in the order (gate descending, token
 *                  index ascending, choice rank ascending); the rest are dropped.
 *   3. expert FFN: y = W2 SiLU(W1 x + b1) + b2 for every kept assignment, as a grouped
 *                  GEMM over the routed rows.
 *   4. combine   : out[t] = x[t] + sum over kept choices of gate * y; a token with no kept
 *                  choice leaves the layer bit for bit as it entered.
 * Sources: "Expert Networks > Worked Example: Expert Specialization" (the whole worked
 * example: configuration, capacity paragraph, trace of token 0, trace of token 4);
 * "Some Tokens Do Not Get In", sections "Why there is a buffer" and "Past the edge";
 * "Dynamic Token Routing AI", section "How it works" (the gating network).
 *
 * Conventions for every call below:
 *   - All array arguments are DEVICE pointers (hipMalloc'd or from a caching allocator),
 *     row-major and contiguous.  In the bf16 dtype, x, weights, biases, y_rows and out
 *     must be 16-byte aligned.  The library never allocates device memory and never
 *     frees a caller's pointer; the caller owns every buffer, including the workspace.
 *   - Calls only enqueue work on `stream` (a hipStream_t; NULL is the null stream) and
 *     return; there is no host synchronisation and no device-to-host copy inside, so a
 *     device fault shows up at the caller's next synchronisation.
 *   - Arguments are checked on the host before anything is enqueued; on any non-OK status
 *     no output has been touched.  moe_last_error() then gives a one-line reason.
 *   - T == 0 is valid and enqueues nothing.
 *   - Calls that share a workspace must not overlap (same stream, or ordered by events).
 *   - Layouts: W_r [E, d_model]; W1 [E, d_ff, d_model]; b1 [E, d_ff]; W2 [E, d_model, d_ff];
 *     b2 [E, d_model]; x and out [T, d_model]; per-assignment arrays [T, top_k], with
 *     choice 0 the largest gate.  Biases have the weight dtype; the router bias is fp32.
 *   - Limits: 1 <= top_k <= n_experts <= 256 (MOE_ERR_INVALID_ARGUMENT otherwise: the slot
 *     keys pack the expert id in 8 bits); capacity >= 0; T * top_k < 2^31; bf16 needs d_model
 *     and d_ff multiples of 8; x must be smaller than 2 GiB (MOE_ERR_UNSUPPORTED otherwise).
 *   - shape->weight_layout says how w1 (w13) and w2 are stored (row-major as above, or packed
 *     by moe_pack_weights); every call that reads them honours it.
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ihipStream_t* moe_stream_t; /* hipStream_t */
typedef struct ihipEvent_t* moe_event_t;   /* hipEvent_t  */

typedef enum {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARGUMENT = 1, /* NULL required pointer, bad sizes, k > E, E > 256,
                                   capacity < 0 */
  MOE_ERR_UNSUPPORTED = 2,      /* misaligned pointer, d not a multiple of 8 for bf16, 32-bit
                                   size limits */
  MOE_ERR_WORKSPACE = 3,        /* ws_bytes < moe_workspace_bytes(shape) */
  MOE_ERR_DEVICE = 4            /* a HIP call failed; moe_last_error() has its text */
} moe_status;

typedef enum { MOE_F32 = 0, MOE_BF16 = 1 } moe_dtype;

/* Storage of the expert weight matrices W1 (or W13) and W2.
 *   MOE_WEIGHTS_ROW_MAJOR: [E, rows, cols] as in the layouts below.
 *   MOE_WEIGHTS_PACKED:    [E, ceil(cols / 32), rows, 32], made once by moe_pack_weights: the
 *                          32-column slices of consecutive rows that the expert GEMMs read
 *                          together are contiguous.  bf16 only; results are bit-identical to
 *                          the row-major layout's (same products, same summation order). */
typedef enum { MOE_WEIGHTS_ROW_MAJOR = 0, MOE_WEIGHTS_PACKED = 1 } moe_weight_layout;

/* Problem shape.  `capacity` is the per-expert slot count, normally moe_capacity(...). */
typedef struct {
  int64_t T;         /* tokens */
  int32_t d_model;
  int32_t d_ff;
  int32_t n_experts; /* E */
  int32_t top_k;     /* k */
  int32_t capacity;  /* slots per expert */
  int32_t dtype;     /* moe_dtype of x, weights, biases, y_rows, out */
  int32_t weight_layout; /* moe_weight_layout of w1 / w13 and w2 */
} moe_shape;

/* floor(C * T * k / E), evaluated exactly on the binary value of C (no rounding of the
 * product).  Worked Example, capacity paragraph: 1.25 * 8 * 1 / 4 = 2.5, rounded down to 2.
 * Returns -1 if T < 0, k < 1, E < 1, C < 0 or not finite, or the result exceeds INT32_MAX. */
int32_t moe_capacity(int64_t T, int32_t top_k, int32_t n_experts, double capacity_factor);

/* Bytes of device workspace every call below needs for this shape (one buffer serves all
 * of them).  0 for an invalid shape.  The workspace holds no state between calls. */
size_t moe_workspace_bytes(const moe_shape* shape);

/* Upper bound on the number of kept rows: min(T * k, E * capacity).  y_rows needs this
 * many rows.  -1 for an invalid shape. */
int64_t moe_max_kept_rows(const moe_shape* shape);

/* Bytes of one packed weight array: E experts of rows x cols, cols rounded up to 32.  0 for an
 * invalid shape. */
size_t moe_packed_weights_bytes(const moe_shape* shape, int32_t rows, int32_t cols);

/* Pack an expert weight array for MOE_WEIGHTS_PACKED (a one-time preparation of the weights).
 *   w        [E, rows, cols] bf16 row-major in (E = shape->n_experts); W1: rows = d_ff, cols =
 *            d_model; W13 of the gated expert: rows = 2 d_ff; W2: rows = d_model, cols = d_ff
 *   w_packed [moe_packed_weights_bytes] out: element (e, r, c) at ((e * ceil(cols / 32) + c / 32)
 *            * rows + r) * 32 + c % 32; columns past cols are zero
 * bf16 only (shape->dtype); cols a multiple of 8; w_packed must not overlap w. */
moe_status moe_pack_weights(const moe_shape* shape, const void* w, int32_t rows, int32_t cols,
                            void* w_packed, moe_stream_t stream);

const char* moe_status_string(int32_t status);
/* Reason for the last non-OK status returned on the calling thread ("" if none). */
const char* moe_last_error(void);

/* Step 1, router.  "Dynamic Token Routing AI", "How it works": a gating network scores each
 * token and selects its experts; Worked Example, trace of token 0: the chosen expert's
 * output is scaled by the router's confidence.
 *   x          [T, d_model]  dtype
 *   w_router   [E, d_model]  dtype
 *   b_router   [E] fp32, or NULL for no bias
 *   topk_ids   [T, k] int32  out: expert of choice c, c = 0 the largest gate
 *   topk_gates [T, k] fp32   out: softmax probability over all E experts (not renormalised)
 *   logits     [T, E] fp32 or NULL   out (diagnostic): the logits rounded to fp32
 * Logits are accumulated in fp64 from exact products, the softmax is evaluated in fp64 and
 * rounded once to fp32; top-k compares the fp32 gates, ties going to the lower expert. */
moe_status moe_route(const moe_shape* shape, const void* x, const void* w_router,
                     const float* b_router, int32_t* topk_ids, float* topk_gates,
                     float* logits, void* ws, size_t ws_bytes, moe_stream_t stream);

/* Step 2, capacity and slot assignment.  Worked Example, capacity paragraph: an expert that
 * receives more tokens than its capacity keeps the most confident ones and drops the rest;
 * "Some Tokens Do Not Get In", "Past the edge": tokens are placed in some order until the
 * buffer is full.  Order used: gate descending, then token ascending, then choice ascending.
 *   topk_ids, topk_gates [T, k]  in (from moe_route, or any caller-made routing; gates must
 *                                not be NaN; an id outside [0, E) is dropped and not counted)
 *   expert_counts  [E]    int32 out: assignments per expert before the capacity cut
 *   expert_offsets [E+1]  int32 out: expert e owns slots [off[e], off[e+1]),
 *                         off[e+1] - off[e] = min(count[e], capacity); off[E] = N_kept
 *   slot_of        [T, k] int32 out: slot of the assignment, or -1 if dropped
 *   row_token      [moe_max_kept_rows] int32 out: token of each slot (first N_kept valid)
 *   drop_mask      [T, k] uint8 out: 1 if dropped
 *   x              [T, d_model] dtype in, or NULL
 *   x_routed       [moe_max_kept_rows, d_model] dtype out, or NULL: row s = x[row_token[s]] for
 *                  s < N_kept (the token rows in slot order, as the first expert GEMM reads
 *                  them: fused-MoE flow diagram, GEMM 1 box); rows past N_kept unspecified.
 *                  x and x_routed are given together or both NULL; they must not overlap.
 * Within an expert, slot off[e] + r holds the assignment of rank r in the fill order. */
moe_status moe_dispatch(const moe_shape* shape, const int32_t* topk_ids, const float* topk_gates,
                        int32_t* expert_counts, int32_t* expert_offsets, int32_t* slot_of,
                        int32_t* row_token, uint8_t* drop_mask, const void* x, void* x_routed,
                        void* ws, size_t ws_bytes, moe_stream_t stream);

/* Step 3, expert FFN over the routed rows.  Worked Example, trace of token 0: h = W1 x + b1,
 * a = SiLU(h), y = W2 a + b2.  Fused-MoE flow diagram (moe-vllm flow), GEMM 1 box: the first
 * GEMM gathers its token rows itself; here through row_token.
 *   x [T, d_model]; row_token, expert_offsets from moe_dispatch (device)
 *   w1 [E, d_ff, d_model], b1 [E, d_ff], w2 [E, d_model, d_ff], b2 [E, d_model]
 *   y_rows [moe_max_kept_rows, d_model] out: y of slot s in row s (first N_kept rows valid)
 * bf16: products accumulate in fp32 on the matrix cores; the activation between the two
 * GEMMs is stored as bf16; y_rows is bf16.  f32: fp32 throughout. */
moe_status moe_expert_ffn(const moe_shape* shape, const void* x, const int32_t* row_token,
                          const int32_t* expert_offsets, const void* w1, const void* b1,
                          const void* w2, const void* b2, void* y_rows, void* ws,
                          size_t ws_bytes, moe_stream_t stream);

/* Step 4, combine with the residual.  Worked Example, traces of tokens 0 and 4: a kept token
 * leaves as x + gate * y, a dropped one as x unchanged.  With k > 1 the kept choices are
 * summed (fp32, one rounding to the dtype); the gates of the kept choices are not
 * renormalised when another choice dropped.  A token with no kept choice gets a bit copy of
 * x ("Past the edge": it reaches the next layer exactly as it entered).
 *   x [T, d_model]; topk_gates, slot_of [T, k]; y_rows from moe_expert_ffn; out [T, d_model]
 * out must not alias x. */
moe_status moe_combine(const moe_shape* shape, const void* x, const float* topk_gates,
                       const int32_t* slot_of, const void* y_rows, void* out,
                       moe_stream_t stream);

/* The whole layer: moe_route, moe_dispatch, moe_expert_ffn, moe_combine on one stream.
 * topk_ids, topk_gates, slot_of, drop_mask, expert_counts are optional outputs (NULL keeps
 * them in the workspace).  Same kernels as the four calls above. */
moe_status moe_layer_forward(const moe_shape* shape, const void* x, const void* w_router,
                             const float* b_router, const void* w1, const void* b1,
                             const void* w2, const void* b2, void* out, int32_t* topk_ids,
                             float* topk_gates, int32_t* slot_of, uint8_t* drop_mask,
                             int32_t* expert_counts, void* ws, size_t ws_bytes,
                             moe_stream_t stream);

/* Bytes of the fixed device scratch that moe_layer_forward_noalloc uses as its workspace. */
#define MOE_NOALLOC_SCRATCH_BYTES (64u << 20)

/* moe_layer_forward without a workspace argument, for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc).  The workspace is a fixed array of MOE_NOALLOC_SCRATCH_BYTES (64 MiB) inside the
 * library, one per device, held from the first use on a device until the process ends; its
 * address is looked up once per device (hipGetSymbolAddress).  The call makes no allocation
 * (no hipMalloc, hipFree or allocating library routine) and needs nothing in the scratch to
 * start at zero.  Same kernels and results as moe_layer_forward.
 * Errors: as moe_layer_forward; MOE_ERR_WORKSPACE when moe_workspace_bytes(shape) exceeds
 * MOE_NOALLOC_SCRATCH_BYTES (decode-sized batches fit: T = 64, d_model 2048, d_ff 8192, top-2
 * needs under 3 MiB).  Every call on one device shares that device's scratch: calls that
 * overlap on a device (other streams or threads without ordering) race and give undefined
 * results; calls ordered on one stream are safe. */
moe_status moe_layer_forward_noalloc(const moe_shape* shape, const void* x, const void* w_router,
                                     const float* b_router, const void* w1, const void* b1,
                                     const void* w2, const void* b2, void* out,
                                     int32_t* topk_ids, float* topk_gates, int32_t* slot_of,
                                     uint8_t* drop_mask, int32_t* expert_counts,
                                     moe_stream_t stream);

/* moe_layer_forward, also recording caller-created events on the stream at the stage
 * boundaries, so the cost of each stage can be read back (the pages ask for the routing
 * decision's own overhead to be watched):
 *   events[0] before routing, [1] after routing, [2] after dispatch, [3] after the first
 *   expert GEMM (up-projection + SiLU), [4] after the second (down-projection), [5] after
 *   the combine.  `events` must hold 6 valid hipEvent_t. */
moe_status moe_layer_forward_profiled(const moe_shape* shape, const void* x,
                                      const void* w_router, const float* b_router,
                                      const void* w1, const void* b1, const void* w2,
                                      const void* b2, void* out, int32_t* topk_ids,
                                      float* topk_gates, int32_t* slot_of, uint8_t* drop_mask,
                                      int32_t* expert_counts, void* ws, size_t ws_bytes,
                                      moe_stream_t stream, moe_event_t const* events);

/* Kernel timing of the two expert GEMMs (the layer's expert-FFN stage, Worked Example: the
 * expert computations whose slowest expert sets the wall-clock time), with nothing inserted
 * between launches.  Arms the NEXT call on this thread of moe_layer_forward (or its _profiled,
 * _padded or _gated form), moe_layer_forward_dropless(_gated), moe_expert_ffn or
 * moe_expert_ffn_pairs:
 *   events[0], [1]  start and end of the up-projection's kernel
 *   events[2], [3]  start and end of the down-projection's kernel
 * recorded by the kernel launches themselves (hipExtLaunchKernel).  The events are the
 * caller's (hipEventCreate, timing enabled); a pair may be NULL (both handles) to time one GEMM
 * only, which halves the markers the timing puts on the stream.  A GEMM that launches nothing
 * (T = 0, no kept rows) gets its two events recorded back to back on the stream.  That next
 * call consumes the arm even if it fails; other calls leave it armed.  events == NULL
 * disarms.  Errors: MOE_ERR_INVALID_ARGUMENT for a half-NULL pair or four NULL handles. */
moe_status moe_set_gemm_timing(const moe_event_t* events);

/* Router and combine kernel timing, for measurement: the kernel time of step 1 (router logits,
 * softmax and top-k: "Dynamic Token Routing AI", "How it works") and of step 4 (the
 * gate-weighted combine and residual: Worked Example, trace of token 0), without the launch
 * gaps that events recorded between stages include.  Arms the NEXT call on this thread of
 * moe_layer_forward (or its _profiled, _padded, _gated or _noalloc form):
 *   events[0], [1]  start and end of the router's kernel
 *   events[2], [3]  start and end of the combine's kernel
 * recorded by those launches themselves (hipExtLaunchKernel).  The events are the caller's
 * (hipEventCreate, timing enabled); a pair may be NULL (both handles).  An empty batch (T = 0)
 * gets the events recorded back to back on the stream.  That next call consumes the arm even
 * if it fails; other calls leave it armed.  events == NULL disarms.  Errors:
 * MOE_ERR_INVALID_ARGUMENT for a half-NULL pair or four NULL handles. */
moe_status moe_set_stage_timing(const moe_event_t* events);

/* ---- Padded fixed-buffer layout.  "Some Tokens Do Not Get In", "Why there is a buffer": each
 * expert gets a buffer of `capacity` slots whether it fills it or not, and the empty slots are
 * computed anyway.  Same layer and same result as moe_layer_forward; only the layout of the
 * expert rows differs: expert e owns rows [e * capacity, (e + 1) * capacity), row e * capacity
 * + r holds its kept assignment of rank r in the fill order, and an unused row is a zero input
 * row, so its expert output is W2 SiLU(b1) + b2 of that expert.  The expert FFN runs over all
 * n_experts * capacity rows (the cost of the fixed buffers), against min(T * k, E * capacity)
 * kept rows at most in the compact layout. */

/* Workspace bytes for moe_layer_forward_padded; 0 for an invalid shape or when
 * n_experts * capacity >= 2^31. */
size_t moe_workspace_bytes_padded(const moe_shape* shape);

/* moe_layer_forward in the padded layout.
 *   slot_of [T, k] out (optional): e * capacity + rank, or -1 if dropped
 *   y_rows  [n_experts * capacity, d_model] out (optional, dtype): every buffer row's expert
 *           output, unused rows included; NULL keeps them in the workspace
 *   events  NULL, or 6 hipEvent_t recorded as in moe_layer_forward_profiled (the padded
 *           remap belongs to the dispatch stage)
 * Other arguments, rules and errors as moe_layer_forward; MOE_ERR_UNSUPPORTED when
 * n_experts * capacity >= 2^31. */
moe_status moe_layer_forward_padded(const moe_shape* shape, const void* x, const void* w_router,
                                    const float* b_router, const void* w1, const void* b1,
                                    const void* w2, const void* b2, void* out, int32_t* topk_ids,
                                    float* topk_gates, int32_t* slot_of, uint8_t* drop_mask,
                                    int32_t* expert_counts, void* y_rows, void* ws,
                                    size_t ws_bytes, moe_stream_t stream,
                                    moe_event_t const* events);

/* ---- Gated expert.  Fused-MoE flow diagram (moe-vllm flow): GEMM 1 writes two halves per
 * row, the SiLU x mul box turns them into one, GEMM 2 follows; the diagram shows no biases.
 * Reading taken: the first half is the gate, the second the up projection, so each expert is
 *   y = W2 (SiLU(W_gate x) * (W_up x))       (element-wise product, no biases)
 * with SiLU(gate) * up fused into GEMM 1's epilogue.
 *   w13 [E, 2 * d_ff, d_model] dtype: rows 0 .. d_ff - 1 of expert e are W_gate, rows d_ff ..
 *       2 d_ff - 1 are W_up;  w2 [E, d_model, d_ff].
 * Routing, capacity, dispatch and combine (with the residual) as moe_layer_forward; shape.d_ff
 * is the width of the product (the activation), the workspace is moe_workspace_bytes(shape);
 * events NULL or 6 hipEvent_t as in moe_layer_forward_profiled.  bf16 only:
 * MOE_ERR_UNSUPPORTED for fp32 and when 2 * d_ff * d_model weights per expert reach 2 GiB. */
moe_status moe_layer_forward_gated(const moe_shape* shape, const void* x, const void* w_router,
                                   const float* b_router, const void* w13, const void* w2,
                                   void* out, int32_t* topk_ids, float* topk_gates,
                                   int32_t* slot_of, uint8_t* drop_mask, int32_t* expert_counts,
                                   void* ws, size_t ws_bytes, moe_stream_t stream,
                                   moe_event_t const* events);

/* ---- Dropless pair-order flow.  Fused-MoE flow diagram (moe-vllm flow): no capacity and no
 * combine gather.  Pair p = t * top_k + c is choice c of token t.  GEMM 1 reads token row
 * p / top_k and writes activation row p; everything up to moe_sum stays in pair order; GEMM 2
 * writes pair row p multiplied by topk_weights[p] (here the unrenormalised gates); moe_sum adds
 * the top_k consecutive rows of each token.  Both GEMMs walk the pairs grouped by expert, so
 * each tile uses one expert's weights.  Reading taken for the output: the residual is added as
 * in the Worked Example's traces, so with a capacity that holds every pair this is
 * moe_layer_forward's result.  shape.capacity is ignored.  bf16 only (moe_sum also takes fp32);
 * MOE_ERR_UNSUPPORTED for fp32 and when the T * top_k * d_ff activation reaches 2 GiB. */

/* Workspace bytes for the dropless calls; 0 for an invalid shape. */
size_t moe_workspace_bytes_dropless(const moe_shape* shape);

/* Group the pairs by expert (the diagram's sorted ids).  A stable counting sort: expert e's
 * pairs, in ascending p, at sorted_pairs[offsets[e] .. offsets[e+1] - 1].
 *   topk_ids       [T, k] int32 in; an id outside [0, E) is not counted and its pair is placed
 *                  after offsets[E]
 *   expert_counts  [E] int32 out;  expert_offsets [E+1] int32 out (exclusive prefix of counts)
 *   sorted_pairs   [T * k] int32 out;  row_token [T * k] int32 out: sorted_pairs[i] / top_k */
moe_status moe_dispatch_pairs(const moe_shape* shape, const int32_t* topk_ids,
                              int32_t* expert_counts, int32_t* expert_offsets,
                              int32_t* sorted_pairs, int32_t* row_token, void* ws,
                              size_t ws_bytes, moe_stream_t stream);

/* The two expert GEMMs in pair order (diagram boxes GEMM 1, SiLU x mul, GEMM 2):
 *   pair_rows[p] = topk_weights[p] * (W2[e] act(W1[e] x[p / top_k] + b1[e]) + b2[e])
 * for every pair p of expert e listed by moe_dispatch_pairs.  gated = 0: act = SiLU, w1
 * [E, d_ff, d_model], biases b1, b2 required.  gated != 0: w1 is w13 [E, 2 d_ff, d_model] of
 * moe_layer_forward_gated, act(.) = SiLU(gate) * up, no biases (b1, b2 ignored).
 *   topk_weights [T, k] fp32 in; pair_rows [T * k, d_model] bf16 out (rows of pairs with an id
 *   outside [0, E) are not written).  fp32 accumulation on the matrix cores, the activation
 *   stored as bf16, the weight applied before the bf16 rounding of pair_rows. */
moe_status moe_expert_ffn_pairs(const moe_shape* shape, const void* x,
                                const int32_t* sorted_pairs, const int32_t* row_token,
                                const int32_t* expert_offsets, const void* w1, const void* b1,
                                const void* w2, const void* b2, const float* topk_weights,
                                int32_t gated, void* pair_rows, void* ws, size_t ws_bytes,
                                moe_stream_t stream);

/* moe_sum box: out[t] = x[t] + sum over c of pair_rows[t * k + c], in choice order, fp32
 * with one rounding to the dtype.
 *   x [T, d_model] or NULL (no residual: the sum alone)
 *   topk_ids [T, k] or NULL: when given, pairs whose id is outside [0, E) are skipped
 *   pair_rows [T * k, d_model];  out [T, d_model], aliasing neither x nor pair_rows
 * A token with no pair row left leaves as x[t] bit for bit (zeros without x). */
moe_status moe_sum(const moe_shape* shape, const void* x, const int32_t* topk_ids,
                   const void* pair_rows, void* out, moe_stream_t stream);

/* The whole dropless layer: moe_route, moe_dispatch_pairs, moe_expert_ffn_pairs (gated = 0),
 * moe_sum with the residual.  topk_ids, topk_gates, expert_counts and pair_rows [T * k,
 * d_model] are optional outputs (NULL keeps them in the workspace); events NULL or 6
 * hipEvent_t recorded before routing, after routing, after the pair dispatch, after GEMM 1,
 * after GEMM 2 and after moe_sum. */
moe_status moe_layer_forward_dropless(const moe_shape* shape, const void* x,
                                      const void* w_router, const float* b_router,
                                      const void* w1, const void* b1, const void* w2,
                                      const void* b2, void* out, int32_t* topk_ids,
                                      float* topk_gates, int32_t* expert_counts, void* pair_rows,
                                      void* ws, size_t ws_bytes, moe_stream_t stream,
                                      moe_event_t const* events);

/* moe_layer_forward_dropless with the gated expert (w13 as in moe_layer_forward_gated): the
 * flow diagram end to end. */
moe_status moe_layer_forward_dropless_gated(const moe_shape* shape, const void* x,
                                            const void* w_router, const float* b_router,
                                            const void* w13, const void* w2, void* out,
                                            int32_t* topk_ids, float* topk_gates,
                                            int32_t* expert_counts, void* pair_rows, void* ws,
                                            size_t ws_bytes, moe_stream_t stream,
                                            moe_event_t const* events);

/* ---- Batch consolidation.  "Token Routing Optimization in Batch Processing" (subtext diagram):
 * token-level routing stays as it is, and a Token Scheduler regroups the tokens of several
 * batches so that each new batch activates fewer experts with more tokens per expert (from
 * every expert active with one token each, to half the experts with two each).  For
 * decode-sized batches the expert GEMMs stream every active expert's weights once per batch,
 * so fewer active experts per batch means fewer weight bytes per batch.
 * Reading taken (the pages give no algorithm): tokens are ordered by their expert set (the k
 * ids sorted ascending, compared as a tuple), ties by token index, and the ordered pool is cut
 * into consecutive batches of the original size.
 * A pool is n_batches batches of batch_shape->T tokens each, stored batch after batch
 * (pool token i is token i % T of batch i / T). */

/* Workspace bytes for moe_layer_forward_batches; 0 for an invalid shape. */
size_t moe_workspace_bytes_batches(const moe_shape* batch_shape, int32_t n_batches);

/* The Token Scheduler on a routed pool.
 *   topk_ids [n_batches * T, k] int32 in (an id outside [0, E) sorts as E and is not counted)
 *   order    [n_batches * T] int32 out: order[i] = the pool token at position i; new batch b is
 *            positions b * T .. b * T + T - 1
 *   batch_experts      [n_batches] int32 out or NULL: distinct experts of each new batch
 *   orig_batch_experts [n_batches] int32 out or NULL: the same for the original batches
 * One workgroup sorts the pool: MOE_ERR_UNSUPPORTED for more than 8192 pool tokens, top_k > 8,
 * or top_k * (bits of E) + 13 > 64.  No workspace. */
moe_status moe_schedule_batches(const moe_shape* batch_shape, int32_t n_batches,
                                const int32_t* topk_ids, int32_t* order,
                                int32_t* batch_experts, int32_t* orig_batch_experts,
                                moe_stream_t stream);

/* A pool of batches through the capacity layer, one batch after another on the stream, as a
 * serving loop runs them: the router once over the pool (routing is per token); with
 * consolidate != 0 the Token Scheduler regroups the pool and the batches run in the new
 * grouping; each batch then runs dispatch (batch_shape->capacity slots per expert), the expert
 * FFN and the combine.  out [n_batches * T, d_model] is in the pool's token order either way.
 * With a capacity of at least T nothing can drop and out does not depend on the grouping.
 *   topk_ids, topk_gates [n_batches * T, k] optional outputs (pool order)
 *   order [n_batches * T] optional output, written when consolidating
 *   batch_experts [n_batches] optional output: distinct experts of each batch as run
 *   events NULL, or 5 hipEvent_t recorded before routing, after routing, after scheduling and
 *          regrouping, after the last batch, and after the outputs are back in pool order.
 * Limits as moe_layer_forward for the pool, and moe_schedule_batches' when consolidating. */
moe_status moe_layer_forward_batches(const moe_shape* batch_shape, int32_t n_batches,
                                     int32_t consolidate, const void* x, const void* w_router,
                                     const float* b_router, const void* w1, const void* b1,
                                     const void* w2, const void* b2, void* out,
                                     int32_t* topk_ids, float* topk_gates, int32_t* order,
                                     int32_t* batch_experts, void* ws, size_t ws_bytes,
                                     moe_stream_t stream, moe_event_t const* events);

#ifdef __cplusplus
}
#endif

#endif /* MOE_H */
