/*
 * moe.h - C ABI of libmoe, a local Mixture-of-Experts forward pass for
 * AMD Instinct MI355X (gfx950).
 *
 * The operation follows the ruDNN user guide (RUDA docs, German edition),
 * sections 3-6 ("MoE workflow", "routing contract", "expert weights and
 * dispatch", "calling MoE"), and the expert stage of the docs.rs page
 * "ruDNN 0.1.25 source, src/moe/experts.rs" (SwiGluExperts::new,
 * forward_dispatched_with_strategy, forward):
 *
 *   logits [T,E] -> FP32 softmax over all E + top-k -> compact dispatch
 *   -> SwiGLU experts -> weighted combine -> out [T,H]
 *
 * and the same pass with the group-limited sigmoid routing of section 10
 * in place of the softmax (experts page, forward_sigmoid_grouped).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Every pointer argument is a DEVICE pointer on the current HIP device,
 *   to a dense row-major array (the shapes below list the dimensions
 *   outermost first).  The caller allocates and owns all memory; the library
 *   borrows pointers for the duration of the call and allocates nothing.
 * - All work is enqueued on `stream` (a hipStream_t; NULL means the default
 *   stream).  No call synchronises the stream or reads device memory on the
 *   host: results are ready when the stream reaches them.
 * - Every argument check runs on the host BEFORE anything is enqueued.  A
 *   failed check returns a nonzero moe_status and enqueues nothing;
 *   moe_last_error() then describes it.  A failed kernel launch returns
 *   MOE_ERR_HIP.  There is no fallback to another path on any error.
 * - NaN and infinity in the data are not errors: they propagate as the
 *   routing contract describes (guide, section 4).
 * - T == 0 (or N == 0) is valid and enqueues nothing.
 * - Outputs must not overlap inputs or each other.
 * - Sizes are int64_t; T*top_k must be below 2^32 (row ids are uint32) and
 *   every array size in bytes must fit in int64_t.
 * - Element types: moe_dtype.  Activations, expert weights and expert
 *   outputs share one dtype `dt`; logits and routing weights share `ldt`
 *   (the guide admits F32, F16 and BF16 for both).
 * - Where a declaration below says "No passage of the pages", the call is
 *   this library's own (host arithmetic or instrumentation) and the pages
 *   define nothing it computes.  Size limits beyond those the guide states
 *   (the E limits of routing, dispatch and the experts, top_k <= 8192 in
 *   combine) are this library's, not the pages'.
 */
#ifndef MOE_MI355X_MOE_H
#define MOE_MI355X_MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum moe_dtype {
    MOE_F32 = 0,
    MOE_F16 = 1,
    MOE_BF16 = 2
} moe_dtype;

typedef enum moe_index_type {
    MOE_IDX_U32 = 0,
    MOE_IDX_I32 = 1,
    MOE_IDX_I64 = 2
} moe_index_type;

typedef enum moe_scoring {
    MOE_SCORE_SOFTMAX = 0,
    MOE_SCORE_SIGMOID = 1
} moe_scoring;

typedef enum moe_status {
    MOE_OK = 0,
    MOE_ERR_INVALID_ARG = 1, /* null pointer, top_k out of range, ...   */
    MOE_ERR_SHAPE = 2,       /* a size is zero/negative or overflows     */
    MOE_ERR_DTYPE = 3,       /* unknown dtype code                        */
    MOE_ERR_UNSUPPORTED = 4, /* valid but beyond this library's limits    */
    MOE_ERR_HIP = 5          /* a HIP launch failed                        */
} moe_status;

/*
 * moe_route - softmax/top-k routing (guide, section 4 "routing contract").
 *
 *   logits  [T,E]      ldt     input
 *   idx     [T,top_k]  uint32  output: selected experts, best first
 *   weights [T,top_k]  ldt     output: routing weights
 *
 * Per row: the softmax is taken over all E experts in FP32; experts are
 * ranked by logit (descending) with ties going to the lower expert id, and
 * the first top_k are taken in that order.  With renormalize != 0 the
 * selected probabilities are divided by their FP32 sum.  The weights are
 * then rounded (nearest even) to ldt.  A row holding a NaN, a +inf, or only
 * -inf gets weights NaN and indices 0..top_k-1.
 * Requires 1 <= top_k <= E (guide, section 4).  E <= 65536 is this
 * library's limit, not the pages' (MOE_ERR_UNSUPPORTED beyond).
 */
int moe_route(const void* logits, int ldt, int64_t T, int64_t E,
              int64_t top_k, int renormalize, uint32_t* idx, void* weights,
              void* stream);

/*
 * moe_dispatch_workspace_size - bytes of scratch moe_dispatch needs for
 * (T, E, top_k): the per-chunk expert count table.  No passage of the
 * pages: pure host arithmetic of this library's dispatch layout; never
 * touches the device.  Returns 0 for invalid sizes.
 */
size_t moe_dispatch_workspace_size(int64_t T, int64_t E, int64_t top_k);

/*
 * moe_dispatch - compact expert-contiguous dispatch (guide, section 5).
 *
 *   x          [T,H]      dt      input token rows
 *   idx        [T,top_k]  uint32  input: expert of each (token, slot)
 *   xd         [N,H]      dt      output: dispatched rows, N = T*top_k
 *   offsets    [E+1]      uint32  output: expert e owns rows
 *                                 [offsets[e], offsets[e+1])
 *   row_expert [N]        uint32  output: expert of each dispatched row
 *   row_token  [N]        uint32  output: source token of each row
 *   token_row  [T,top_k]  uint32  output: the dispatched row of each
 *                                 (token, slot): the stored mapping that
 *                                 restores token order
 *   workspace  moe_dispatch_workspace_size(T,E,top_k) bytes of scratch
 *
 * No token is dropped: offsets[E] == N and every row is a bit copy of its
 * token.  Inside an expert, rows follow (token, slot) order (the guide
 * leaves that order open; this library keeps it stable and deterministic).
 * idx values must be < E.  An out-of-range value is not read as an expert:
 * its rows are placed after offsets[E] with row_expert 0xFFFFFFFF (so
 * offsets[E] < N signals it), every access stays in bounds, and
 * moe_experts_forward writes zeros for those rows.
 * E <= 16383 is this library's limit, not the pages' (the per-chunk count
 * table must fit in LDS; MOE_ERR_UNSUPPORTED beyond).
 */
int moe_dispatch(const void* x, int dt, int64_t T, int64_t H, int64_t E,
                 int64_t top_k, const uint32_t* idx, void* xd,
                 uint32_t* offsets, uint32_t* row_expert, uint32_t* row_token,
                 uint32_t* token_row, void* workspace, size_t workspace_bytes,
                 void* stream);

/*
 * moe_dispatch_noalloc - moe_dispatch for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc): the same arguments, outputs and
 * results without the workspace.  The count table lives in a static
 * device array of 4 MiB (2^20 uint32 entries) that each device the
 * library runs on holds until the process ends; no call allocates or frees
 * anything.  Sizes whose table would need more than that (very large E
 * times many chunks; never below E = 16383 with T*top_k <= 2^26) return
 * MOE_ERR_UNSUPPORTED before anything is enqueued.  All calls on one device
 * share the array, so calls that overlap on one device (concurrent
 * streams, or threads) race: serialise them.  Every table entry a call
 * reads is written by that call first, so nothing needs clearing.
 */
int moe_dispatch_noalloc(const void* x, int dt, int64_t T, int64_t H,
                         int64_t E, int64_t top_k, const uint32_t* idx,
                         void* xd, uint32_t* offsets, uint32_t* row_expert,
                         uint32_t* row_token, uint32_t* token_row,
                         void* stream);

/*
 * moe_experts_forward - SwiGLU experts over expert segments (experts page,
 * forward_dispatched_with_strategy; weight layouts from SwiGluExperts::new).
 *
 *   xd      [N,H]    dt      dispatched rows
 *   w_gate  [E,I,H]  dt      gate weights (no bias)
 *   w_up    [E,I,H]  dt      up weights (no bias)
 *   w_down  [E,H,I]  dt      down weights (no bias)
 *   offsets [E+1]    uint32  segments as written by moe_dispatch
 *   act     [N,I]    dt      output/scratch: SiLU(gate) * up
 *   y       [N,H]    dt      output: expert output rows
 *
 * For a row r of segment e:  g = xd[r] . w_gate[e]^T,  u = xd[r] . w_up[e]^T
 * (FP32 accumulation, each rounded to dt), act = SiLU(g) * u (FP32, rounded
 * to dt), y[r] = act . w_down[e]^T (FP32 accumulation, rounded to dt).
 * Segments must be monotone with offsets[0] == 0 and offsets[E] <= N; rows
 * in [offsets[E], N) get y = 0 and their act rows are not written.
 * E <= 16383 is this library's limit, not the pages'.
 */
int moe_experts_forward(const void* xd, int dt, int64_t N, int64_t H,
                        int64_t I, int64_t E, const void* w_gate,
                        const void* w_up, const void* w_down,
                        const uint32_t* offsets, void* act, void* y,
                        void* stream);

/*
 * moe_experts_forward_clipped - moe_experts_forward with the clipped SwiGLU
 * activation (MindSpeed-Ops page, clipped_swiglu: swiglu_alpha, default
 * 1.702, and swiglu_limit, default 7).  Arguments as moe_experts_forward
 * plus alpha (finite) and limit (finite, >= 0); act becomes
 *   gc * sigmoid(alpha * gc) * uc,  gc = min(g, limit),
 *   uc = min(max(u, -limit), limit)
 * in FP32 from the rounded g and u, rounded to dt (NaN stays NaN through
 * the clamps).  Violations: MOE_ERR_INVALID_ARG.
 */
int moe_experts_forward_clipped(const void* xd, int dt, int64_t N, int64_t H,
                                int64_t I, int64_t E, const void* w_gate,
                                const void* w_up, const void* w_down,
                                const uint32_t* offsets, float alpha,
                                float limit, void* act, void* y, void* stream);

/*
 * moe_combine - weighted merge back into token order (guide, section 6).
 *
 *   y         [N,H]      dt      expert output rows
 *   weights   [T,top_k]  wdt     routing weights
 *   token_row [T,top_k]  uint32  mapping written by moe_dispatch
 *   out       [T,H]      dt      output
 *
 * out[t] = sum over slots j = 0..top_k-1, in slot order and in FP32, of
 * weights[t,j] * y[token_row[t,j]], rounded once to dt.  The routing
 * weights are applied here and nowhere else.  A token_row value >= N makes
 * that token's output NaN instead of being read.  top_k <= 8192
 * (MOE_ERR_UNSUPPORTED beyond).
 */
int moe_combine(const void* y, int dt, int64_t N, int64_t T, int64_t H,
                int64_t top_k, const void* weights, int wdt,
                const uint32_t* token_row, void* out, void* stream);

/*
 * moe_forward_workspace_size - bytes of scratch moe_forward needs.  No
 * passage of the pages: pure host arithmetic of this library's workspace
 * layout (routing result, dispatch mapping and rows, count table, act, y);
 * never touches the device.  Returns 0 for invalid arguments.
 */
size_t moe_forward_workspace_size(int64_t T, int64_t H, int64_t I, int64_t E,
                                  int64_t top_k, int dt, int ldt);

/*
 * moe_forward - the whole local MoE forward (experts page,
 * SwiGluExperts::forward): moe_route -> moe_dispatch ->
 * moe_experts_forward -> moe_combine on one stream.
 *
 *   x      [T,H]   dt    input tokens
 *   logits [T,E]   ldt   router logits, computed by the caller
 *   w_gate, w_up [E,I,H], w_down [E,H,I]   dt
 *   out    [T,H]   dt    output
 *   workspace  moe_forward_workspace_size(...) bytes, 256-byte aligned
 *
 * Limits are those of the four stages: 1 <= top_k <= E (guide, section 4);
 * E <= 16383, top_k <= 8192 and T*top_k < 2^32 are this library's.  The workspace holds the routing result,
 * the dispatch mapping and rows, the dispatch count table, act and y.
 */
int moe_forward(const void* x, int dt, const void* logits, int ldt,
                int64_t T, int64_t H, int64_t I, int64_t E, int64_t top_k,
                int renormalize, const void* w_gate, const void* w_up,
                const void* w_down, void* out, void* workspace,
                size_t workspace_bytes, void* stream);

/*
 * moe_forward_clipped - moe_forward with the clipped SwiGLU activation of
 * moe_experts_forward_clipped (MindSpeed-Ops page, clipped_swiglu parameter
 * table; alpha finite, limit finite and >= 0, MOE_ERR_INVALID_ARG
 * otherwise).  Workspace and limits as moe_forward.
 */
int moe_forward_clipped(const void* x, int dt, const void* logits, int ldt,
                        int64_t T, int64_t H, int64_t I, int64_t E,
                        int64_t top_k, int renormalize, float alpha,
                        float limit, const void* w_gate, const void* w_up,
                        const void* w_down, void* out, void* workspace,
                        size_t workspace_bytes, void* stream);

/*
 * moe_route_sigmoid_grouped - group-limited sigmoid routing (guide,
 * section 10 "group-limited sigmoid MoE routing": route_sigmoid_grouped
 * with GroupRoutingOptions).
 *
 *   logits  [T,E]      ldt      input
 *   bias    [E]        float32  input, optional correction bias (NULL: none)
 *   idx     [T,top_k]  uint32   output: chosen experts, best first
 *   weights [T,top_k]  ldt      output: routing weights
 *
 * Per row: s_e is the FP32 sigmoid of logit e (evaluated in float64 and
 * rounded once, so it is the correctly rounded value in all but ~1e-9 of
 * cases) and c_e = s_e + bias[e] in FP32.  The experts form `groups` groups
 * of E/groups consecutive ids.  A group's score is its largest c, or with
 * group_top_two != 0 the FP32 sum of its two largest.  The selected_groups
 * best groups are kept, then the top_k kept experts with the largest c are
 * chosen and listed best first; ties, between groups and between experts,
 * go to the smaller id.  The weight of a chosen expert is s_e (the bias only
 * changes the choice), divided by the FP32 sum of the chosen s in slot
 * order if renormalize != 0, then multiplied by scale and rounded (nearest
 * even) to ldt.  A row whose c or group scores hold a NaN gets indices
 * 0..top_k-1 and NaN weights; +inf and -inf logits are ordinary scores
 * (1 and 0).  With renormalisation, a row whose chosen s are all 0 gets
 * NaN weights (0/0).
 * Limits of the guide, MOE_ERR_INVALID_ARG when violated: 1 <= E <= 1024;
 * 1 <= groups <= 128 with E % groups == 0; 1 <= selected_groups <= groups;
 * 1 <= top_k <= 64 and top_k <= selected_groups * E / groups;
 * group_top_two needs E / groups >= 2; scale finite and > 0.
 */
int moe_route_sigmoid_grouped(const void* logits, int ldt, int64_t T,
                              int64_t E, const float* bias, int64_t top_k,
                              int64_t groups, int64_t selected_groups,
                              int group_top_two, int renormalize, float scale,
                              uint32_t* idx, void* weights, void* stream);

/*
 * moe_forward_sigmoid_grouped - the whole local MoE forward with
 * group-limited sigmoid routing (experts page,
 * SwiGluExperts::forward_sigmoid_grouped): moe_route_sigmoid_grouped ->
 * moe_dispatch -> moe_experts_forward -> moe_combine on one stream.
 *
 * Arguments are those of moe_forward plus the routing options and the
 * optional bias of moe_route_sigmoid_grouped; the workspace size is
 * moe_forward_workspace_size(T, H, I, E, top_k, dt, ldt) (the same layout).
 * Limits are those of moe_route_sigmoid_grouped and moe_forward.
 */
int moe_forward_sigmoid_grouped(const void* x, int dt, const void* logits,
                                int ldt, const float* bias, int64_t T,
                                int64_t H, int64_t I, int64_t E,
                                int64_t top_k, int64_t groups,
                                int64_t selected_groups, int group_top_two,
                                int renormalize, float scale,
                                const void* w_gate, const void* w_up,
                                const void* w_down, void* out,
                                void* workspace, size_t workspace_bytes,
                                void* stream);

/*
 * moe_selected_router_weights - FP32 router weights of a fixed selection
 * (guide, section 12 "first-order MoE training": selected_router_weights
 * with RouterWeightOptions).
 *
 *   logits  [T,E]      ldt         input
 *   indices [T,top_k]  index_type  input: experts of each row (moe_index_type)
 *   weights [T,top_k]  float32     output
 *
 * Scores: scoring MOE_SCORE_SOFTMAX takes the softmax over all E experts of
 * the row, MOE_SCORE_SIGMOID the sigmoid of each logit (FP32).  Slot j's
 * weight is the score of expert indices[t,j] (a repeated index gathers the
 * same score again); with renormalize != 0 divided by the sum of the row's
 * selected scores; then multiplied by scale.  An invalid index (negative,
 * or >= E) makes the whole row NaN, without an out-of-bounds access; NaN
 * also follows from the scores (softmax: a row holding a NaN, a +inf or
 * only -inf; sigmoid: a NaN logit, or a zero sum when renormalising).
 * Limits, MOE_ERR_INVALID_ARG when violated: 1 <= top_k <= min(E, 64),
 * E < 2^31, scale finite and > 0, scoring and index_type known.
 */
int moe_selected_router_weights(const void* logits, int ldt, int64_t T,
                                int64_t E, const void* indices,
                                int index_type, int64_t top_k, int scoring,
                                int renormalize, float scale, float* weights,
                                void* stream);

/*
 * moe_selected_router_backward - the logits gradient of
 * moe_selected_router_weights (guide, section 12: selected_router_backward).
 *
 *   logits       [T,E]      ldt         input (the same as for the weights)
 *   indices      [T,top_k]  index_type  input
 *   grad_weights [T,top_k]  float32     input: dL/dweights
 *   grad_logits  [T,E]      ldt         output: dL/dlogits
 *
 * The exact vector-Jacobian product of the weights for the fixed selection
 * (the choice itself is not differentiated), computed in FP32 and rounded
 * to ldt.  With u_j the selected scores, g_j = grad_weights, S = sum_l u_l,
 * v_j = u_j/S, gbar = sum_l g_l v_l, and A_e the sum over the slots
 * selecting e of a_j:
 *   softmax:        grad_e = p_e * (A_e - sum_j u_j a_j), a_j = scale*g_j;
 *   softmax, renormalised: grad_e = A_e with a_j = scale*v_j*(g_j - gbar)
 *                   for a selected e, 0 for the others (the renormalised
 *                   weights are the softmax over the selected logits);
 *   sigmoid:        grad_e = s_e*(1-s_e)*A_e for a selected e, exactly 0 for
 *                   the others, a_j = scale*g_j, or (scale/S)*(g_j - gbar)
 *                   renormalised.
 * NaN scores give NaN gradients as the arithmetic carries them.  An invalid
 * index makes the whole gradient row NaN.  Limits as
 * moe_selected_router_weights.
 */
int moe_selected_router_backward(const void* logits, int ldt, int64_t T,
                                 int64_t E, const void* indices,
                                 int index_type, int64_t top_k,
                                 const float* grad_weights, int scoring,
                                 int renormalize, float scale,
                                 void* grad_logits, void* stream);

/*
 * First-order training (guide, section 12; experts page,
 * forward_dispatched_training and ExpertTrainingCache::backward).  The
 * backward chain, after a forward that used moe_dispatch and
 * moe_experts_forward_training (and FP32 routing weights, e.g. from
 * moe_selected_router_weights):
 *   moe_combine_backward -> moe_experts_backward -> moe_dispatch_backward
 *   -> moe_selected_router_backward (logits gradient from the weight
 *   gradient).
 * Tensors the chain materialises are rounded to their dtype once; weight
 * gradients are FP32.
 */

/*
 * moe_experts_forward_training - moe_experts_forward that keeps what the
 * expert backward needs (experts page, forward_dispatched_training).
 *
 *   xd, w_gate, w_up, w_down, offsets   as moe_experts_forward
 *   gate [N,I] dt   output: xd . w_gate[e]^T, FP32 accumulation, rounded
 *   up   [N,I] dt   output: xd . w_up[e]^T, rounded
 *   act  [N,I] dt   output: SiLU(gate) * up (FP32 from the stored gate and
 *                   up), rounded
 *   y    [N,H] dt   output: act . w_down[e]^T, rounded
 * Rows in [offsets[E], N) get zeros.  Limits as moe_experts_forward.
 */
int moe_experts_forward_training(const void* xd, int dt, int64_t N,
                                 int64_t H, int64_t I, int64_t E,
                                 const void* w_gate, const void* w_up,
                                 const void* w_down, const uint32_t* offsets,
                                 void* gate, void* up, void* act, void* y,
                                 void* stream);

/*
 * moe_combine_backward - gradients of moe_combine (guide, section 12,
 * step 1).
 *
 *   y            [N,H]      dt      expert output rows (forward input)
 *   weights      [T,top_k]  wdt     routing weights (forward input)
 *   token_row    [T,top_k]  uint32  the dispatch mapping
 *   grad_out     [T,H]      dt      dL/dout
 *   grad_expert  [N,H]      dt      output: row token_row[t,j] gets
 *                                   weights[t,j] * grad_out[t] (FP32,
 *                                   rounded); rows no slot maps are not
 *                                   written (moe_dispatch maps every row)
 *   grad_weights [T,top_k]  float32 output: grad_out[t] . y[token_row[t,j]]
 *                                   in FP32
 * A token_row value >= N gets a NaN weight gradient and writes no row.
 * top_k <= 8192.
 */
int moe_combine_backward(const void* y, int dt, int64_t N, int64_t T,
                         int64_t H, int64_t top_k, const void* weights,
                         int wdt, const uint32_t* token_row,
                         const void* grad_out, void* grad_expert,
                         float* grad_weights, void* stream);

/*
 * moe_experts_backward_workspace_size - bytes of scratch
 * moe_experts_backward needs (one transposed weight tensor, three [N,I] and
 * two [N,H] intermediates).  No passage of the pages: pure host arithmetic of this
 * library's workspace layout; never touches the device.
 * Returns 0 for invalid arguments.
 */
size_t moe_experts_backward_workspace_size(int64_t N, int64_t H, int64_t I,
                                           int64_t E, int dt);

/*
 * moe_experts_backward - the expert backward (guide, section 12, step 2;
 * experts page, ExpertTrainingCache::backward_with_strategy).
 *
 *   xd, w_gate, w_up, w_down, offsets   the forward's inputs
 *   gate, up, act [N,I] dt   the training forward's cache
 *   grad_y      [N,H]   dt       dL/dy (from moe_combine_backward)
 *   grad_xd     [N,H]   dt       output: dL/dxd
 *   grad_w_gate [E,I,H] float32  output
 *   grad_w_up   [E,I,H] float32  output
 *   grad_w_down [E,H,I] float32  output
 *   workspace   moe_experts_backward_workspace_size(N,H,I,E,dt) bytes,
 *               256-byte aligned.  It holds, in this order, each part at
 *               the next 256-byte aligned offset: one transposed weight
 *               tensor (E*H*I elements of dt; written only for shapes the
 *               K-major weight read does not take), then dact, dgate_raw,
 *               dup_raw [N,I] and the two input-gradient halves
 *               round(dgate_raw . w_gate[e]), round(dup_raw . w_up[e])
 *               [N,H], all dt; after the call dact .. the second half
 *               hold the intermediates named below.
 *
 * In the experts page's order, each intermediate rounded to dt:
 * dact = grad_y . w_down[e]; dgate_raw = dact * up * s * (1 + gate*(1-s)),
 * dup_raw = dact * gate * s with s = sigmoid(gate); grad_xd =
 * round(round(dgate_raw . w_gate[e]) + round(dup_raw . w_up[e])).  Weight
 * gradients, FP32 sums over each expert's rows: grad_w_down[e] =
 * grad_y^T . act, grad_w_gate[e] = dgate_raw^T . xd, grad_w_up[e] =
 * dup_raw^T . xd; an expert with no rows gets zeros.  Rows in
 * [offsets[E], N) get grad_xd = 0.  Limits as moe_experts_forward.
 */
int moe_experts_backward(const void* xd, int dt, int64_t N, int64_t H,
                         int64_t I, int64_t E, const void* w_gate,
                         const void* w_up, const void* w_down,
                         const uint32_t* offsets, const void* gate,
                         const void* up, const void* act, const void* grad_y,
                         void* grad_xd, float* grad_w_gate, float* grad_w_up,
                         float* grad_w_down, void* workspace,
                         size_t workspace_bytes, void* stream);

/*
 * moe_dispatch_backward - the gradient of moe_dispatch (guide, section 12,
 * step 3): grad_x[t] = sum over slots j, in slot order and in FP32, of
 * grad_xd[token_row[t,j]], rounded once to dt; the routing weights are not
 * applied again.
 *
 *   grad_xd   [N,H]      dt      dL/dxd
 *   token_row [T,top_k]  uint32  the dispatch mapping
 *   grad_x    [T,H]      dt      output
 * A token_row value >= N makes that token's gradient NaN.  top_k <= 8192.
 */
int moe_dispatch_backward(const void* grad_xd, int dt, int64_t N, int64_t T,
                          int64_t H, int64_t top_k,
                          const uint32_t* token_row, void* grad_x,
                          void* stream);

/*
 * moe_set_timing_events - instrumentation for measuring each kernel.  No
 * passage of the pages: this library's own timing hook; it changes no
 * result.
 *
 * events: `count` hipEvent_t handles created by the caller (hipEventCreate),
 * or NULL with count 0 to switch recording off.  While set, every
 * moe_forward, moe_forward_clipped and moe_forward_sigmoid_grouped call
 * on this thread records
 * events[0] on its stream before its first kernel and events[i] right
 * after its i-th kernel, so the elapsed time between events[i-1] and
 * events[i] is kernel i.  The kernels of the forwards, in order: 1 route
 * (softmax or group-limited sigmoid), 2 dispatch count, 3 dispatch scan,
 * 4 dispatch (the mapping alone where the gate+up GEMM reads the token
 * rows in place, else the row scatter), 5 gate+up GEMM with SwiGLU,
 * 6 down GEMM, 7 combine.  Where the softmax forwards route and count in
 * one launch, that launch is kernel 1 and events[1] and events[2] are
 * recorded back to back (interval 2 holds no kernel).  A NULL entry
 * skips that mark (each recorded event costs a few microseconds of GPU
 * time; a caller timing one kernel sets only its two events).  count must
 * be 0 or MOE_TIMING_EVENTS.  The library does not own the events; the
 * caller keeps them alive while recording is on.
 */
#define MOE_TIMING_EVENTS 8
int moe_set_timing_events(void* const* events, int count);

/*
 * moe_status_string - static text for a status code ("unknown status" for
 * codes outside moe_status).  The status codes stand for the pages'
 * MoeError results: the guide's MoE calls return a Result with MoeError
 * (guide, section 3 "MoE workflow" and section 6 "calling MoE"), and the
 * experts page's SwiGluExperts::new and forward_dispatched_with_strategy
 * reject mismatched ranks, shapes and dtypes with static messages.
 */
const char* moe_status_string(int status);

/*
 * moe_last_error - detail of the last failed call on this thread ("" if
 * the last call succeeded): the static-message text of the pages' MoeError
 * (guide, sections 3 and 6; experts page, SwiGluExperts::new), plus the
 * offending values.  The string stays valid until the next call on this
 * thread.
 */
const char* moe_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* MOE_MI355X_MOE_H */
