/*
 * switch_moe.h -- C ABI of the Switch FFN layer forward pass on one AMD
 * MI355X GPU (gfx950), library libswitchmoe.so.
 *
 * The operation is the Switch layer of the Switch Transformer, as defined in
 * the engineering write-up "Switch Transformers: Scaling to Trillion Parameter
 * Models" (sections "Switch Routing: From Top-k to k = 1", "Expert Capacity
 * and the Capacity Factor", "The Load-Balancing Loss", "The Architecture in
 * Place", "Making Sparse Training Stable"):
 *
 *   h(x) = W_r x (+ b)                     router logits, fp32
 *   p_i(x) = exp(h_i) / sum_j exp(h_j)     softmax gate, fp32
 *   e(x) = argmax_i p_i(x)                 top-1 ("Switch") routing, k = 1
 *   capacity = T / N * capacity_factor     per-expert buffer, overflow dropped
 *   E_i(x) = W_out,i ReLU(W_in,i x)        N independent expert FFNs
 *   y(x) = p_e(x) E_e(x)                   gate-scaled combine (0 if dropped)
 *   aux = N sum_i f_i P_i                  load-balancing loss (no alpha)
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Array arguments are DEVICE pointers owned by the caller; the library
 *   allocates and frees nothing, keeps no state between calls and never
 *   blocks the host (but see debug mode below).  All work is enqueued on
 *   `stream` (a hipStream_t passed as void*; NULL = null stream).
 * - Layouts are dense row-major, except the weights W_r, W_in and W_out
 *   when s->weight_layout is SWITCH_WEIGHTS_TILED (see below).  T tokens are
 *   the caller's [batch][seq] flattened in row-major order; that order is
 *   the "token order" that decides which tokens overflow an expert.
 * - Activation dtype (s->dtype) applies to x, W_in, W_out, dispatched,
 *   expert_out and y: SWITCH_F32 (float) or SWITCH_BF16 (bfloat16, stored as
 *   16-bit words).  The router (W_r, bias, logits, softmax, gate) is always
 *   fp32, whatever the activation dtype.
 * - Every call validates all of its arguments on the host before it enqueues
 *   anything: a call that returns an error has enqueued nothing and left
 *   every output untouched.  Device faults are asynchronous and surface at
 *   the caller's next synchronisation of the stream.
 * - Debug mode: when the environment variable SMX_DEBUG_SYNC is set to a
 *   value other than "" and "0" (read once per process), every entry point
 *   waits for `stream` after each kernel it launches; when a wait reports an
 *   error, the call launches nothing more and returns SWITCH_E_HIP with the
 *   failing kernel's name in switch_last_error().  Kernels launched before
 *   the failure stay enqueued; the outputs are then undefined.
 * - Outputs must not alias inputs or each other.  Calls on different streams
 *   with different buffers are independent; the library is reentrant.
 * - Alignment: x, W_in, W_out, dispatched, expert_out, y, x_residual, W_r
 *   must be 16-byte aligned; workspace 256-byte aligned; other arrays 4-byte
 *   aligned (dropped: any).
 * - Supported shapes: d_model and d_ff multiples of 64; 0 <= tokens <= 2^31-1;
 *   num_experts >= 1; capacity >= 0.  Shapes outside that give
 *   SWITCH_E_UNSUPPORTED, and so does SWITCH_WEIGHTS_TILED with fp32; a
 *   weight_layout other than the two values below gives SWITCH_E_INVALID.
 *   Every call that reads W_r, W_in or W_out reads them in s->weight_layout.
 */
#ifndef SWITCH_MOE_H
#define SWITCH_MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SWITCH_OK 0
#define SWITCH_E_INVALID (-1)     /* NULL / misaligned pointer, negative or zero dimension, bad dtype */
#define SWITCH_E_UNSUPPORTED (-2) /* shape outside the kernels' contract (see above) */
#define SWITCH_E_WORKSPACE (-3)   /* workspace smaller than switch_workspace_bytes() */
#define SWITCH_E_HIP (-4)         /* a HIP runtime / launch call failed; see switch_last_error() */

enum { SWITCH_F32 = 0, SWITCH_BF16 = 1 };

/* Storage of the weights.  The expert weights W_in [N][d_ff][d_model] and
 * W_out [N][d_model][d_ff]: each expert matrix has R rows and K columns, K
 * being the contraction dimension (d_model for W_in, d_ff for W_out).
 *   SWITCH_WEIGHTS_ROWS   row-major: element (r, k) of matrix m at
 *                         (m R + r) K + k.
 *   SWITCH_WEIGHTS_TILED  bf16 only: 16-row x 32-column blocks in row-major
 *                         block order, each block as 64 groups of 8
 *                         consecutive columns, group g = 16 (k % 32 / 8) +
 *                         r % 16; element (r, k) of matrix m at
 *                           ((m R/16 + r/16) K/32 + k/32) 512 + g 8 + k % 8.
 *                         This is the operand order of the matrix cores'
 *                         16x16x32 bf16 product, so a wave reads a block of
 *                         weights as one contiguous 1 KB piece; the layer is
 *                         faster and its results are bit-identical to those of
 *                         the row-major layout.  switch_tile_weights converts.
 *                         The same byte count either way.
 * The router weights W_r: fp32 [N][d_model] row-major with SWITCH_WEIGHTS_ROWS;
 * with SWITCH_WEIGHTS_TILED the argument w_router instead points at W_r's
 * exact three-way bf16 split in the router's matrix-core operand order, as
 * switch_tile_router writes it (switch_tiled_router_bytes bytes).  That is
 * the form the router's products read: with row-major W_r a bf16 layer call
 * first writes it into its workspace, a pass the tiled form skips.  The
 * router computes the same fp32 logits either way.
 * The layout is not checked: weights in the other layout than the one
 * declared give wrong results, not an error. */
enum { SWITCH_WEIGHTS_ROWS = 0, SWITCH_WEIGHTS_TILED = 1 };

typedef struct switch_shape {
  int64_t tokens;        /* T: tokens per batch (capacity equation)                      */
  int32_t d_model;       /* d: token width                                               */
  int32_t d_ff;          /* expert hidden width                                          */
  int32_t num_experts;   /* N                                                            */
  int32_t capacity;      /* C: per-expert buffer rows, normally from switch_capacity()   */
  int32_t dtype;         /* SWITCH_F32 or SWITCH_BF16 (activations and expert weights)   */
  int32_t weight_layout; /* SWITCH_WEIGHTS_ROWS (0) or SWITCH_WEIGHTS_TILED: W_r, W_in, W_out */
} switch_shape;

/* Expert capacity, "Expert Capacity and the Capacity Factor" (capacity
 * equation): tokens per batch / number of experts x capacity factor, rounded
 * up, computed exactly on the binary64 value of capacity_factor.  Host only.
 * Errors: SWITCH_E_INVALID (tokens < 0, num_experts < 1, factor not finite
 * and > 0, NULL out), SWITCH_E_UNSUPPORTED (result above 2^31-1). */
int switch_capacity(int64_t tokens, int32_t num_experts, double capacity_factor, int32_t *capacity_out);

/* Bytes of device workspace that every entry point below accepts for this
 * shape (the largest need, which is switch_layer_forward's).  Host only.
 * Smaller needs: switch_route needs the value reported for the same shape
 * with capacity 0; switch_expert_ffn needs num_experts * capacity * d_ff *
 * sizeof(activation) rounded up to 256 bytes. */
int switch_workspace_bytes(const switch_shape *s, size_t *bytes_out);

/* Text of the last error on the calling thread ("" if none). */
const char *switch_last_error(void);

/* Routing: router logits, fp32 softmax, top-1 choice, gate, capacity
 * assignment and the load-balancing loss ("Switch Routing", "Expert
 * Capacity", "The Load-Balancing Loss").
 *   x            [T][d]    activation dtype
 *   w_router     [N][d]    fp32 (tiled layout: switch_tile_router's planes)
 *   router_bias  [N] fp32 or NULL (added to the logits)
 * Outputs:
 *   expert_idx   [T] int32  argmax of the logits; ties go to the lowest index
 *   gate         [T] fp32   p_e(x) = 1 / sum_j exp(h_j - max_j h_j)
 *   slot         [T] int32  number of earlier tokens routed to the same
 *                           expert (also for dropped tokens)
 *   dropped      [T] uint8  1 if slot >= capacity (overflow), else 0
 *   expert_count [N] int32  tokens routed to each expert before capacity
 *   aux_loss     [1] fp32   N * sum_i f_i P_i; f_i = expert_count_i / T,
 *                           P_i = mean over all T tokens of p_i; 0 when T = 0
 * Results are deterministic: integer slots, fixed-order float reductions. */
int switch_route(const switch_shape *s, const void *x, const float *w_router, const float *router_bias,
                 int32_t *expert_idx, float *gate, int32_t *slot, uint8_t *dropped, int32_t *expert_count,
                 float *aux_loss, void *workspace, size_t workspace_bytes, void *stream);

/* Dispatch: copy every kept token's row into its expert's buffer,
 * dispatched[expert_idx[t]][slot[t]][:] = x[t][:] ("Expert Capacity" figure:
 * dispatch to the single top expert).  dispatched is [N][C][d]; rows at or
 * past an expert's kept count are padding and left untouched. */
int switch_dispatch(const switch_shape *s, const void *x, const int32_t *expert_idx, const int32_t *slot,
                    const uint8_t *dropped, void *dispatched, void *stream);

/* Routing and dispatch in one pass over x (the router, "Expert Capacity and
 * the Capacity Factor" and "The Load-Balancing Loss" of the Switch
 * Transformers write-up): the outputs of switch_route followed by
 * switch_dispatch, from a single kernel that reads each row of x once.  Every
 * router block assigns its own tokens' slots after adding the expert counts of
 * the blocks before it in token order, which it finds by a look-back over
 * their published partial results in the workspace (a small clearing kernel
 * runs first), and copies each kept row to dispatched[expert_idx[t]][slot[t]]
 * while the row is still in cache.  expert_idx, gate, slot, dropped,
 * expert_count and dispatched equal those of switch_route + switch_dispatch
 * bit for bit; aux_loss sums P_i in 2^-31 fixed point (deterministic, within
 * 1e-6 relative of switch_route's value; NaN would report a failed internal
 * wait, which a correct launch never reaches).  dispatched is [N][C][d] of
 * s->dtype (may be NULL when C = 0); padding rows are left untouched.
 * Workspace: switch_workspace_bytes(s).  SWITCH_E_UNSUPPORTED for more than
 * 2048 experts or N x C above 2^31-1.  Two calls must not share a workspace
 * concurrently (the same holds for every call here). */
int switch_route_dispatch(const switch_shape *s, const void *x, const float *w_router, const float *router_bias,
                          int32_t *expert_idx, float *gate, int32_t *slot, uint8_t *dropped,
                          int32_t *expert_count, float *aux_loss, void *dispatched, void *workspace,
                          size_t workspace_bytes, void *stream);

/* Expert FFNs ("The Core Idea": N independent FFNs; the expert form
 * E(x) = W_out ReLU(W_in x) has no biases):
 *   expert_out[i][r] = W_out,i ReLU(W_in,i dispatched[i][r])
 * for r < min(expert_count[i], C).  w_in is [N][d_ff][d], w_out is
 * [N][d][d_ff]; expert_out is [N][C][d].  In bf16 the hidden ReLU output is
 * rounded to bf16; accumulation is fp32.  Padding rows are neither read nor
 * written. */
int switch_expert_ffn(const switch_shape *s, const void *dispatched, const int32_t *expert_count,
                      const void *w_in, const void *w_out, void *expert_out, void *workspace,
                      size_t workspace_bytes, void *stream);

/* Combine ("Switch Routing" combine equation with k = 1; "Expert Capacity":
 * dropped tokens skip the expert):
 *   y[t] = gate[t] * expert_out[expert_idx[t]][slot[t]]   (kept t)
 *   y[t] = 0                                              (dropped t)
 * plus x_residual[t] for every t when x_residual is not NULL.  fp32
 * arithmetic, one rounding to the activation dtype. */
int switch_combine(const switch_shape *s, const void *expert_out, const int32_t *expert_idx,
                   const int32_t *slot, const uint8_t *dropped, const float *gate, const void *x_residual,
                   void *y, void *stream);

/* The whole Switch FFN layer ("The Architecture in Place": the Switch layer
 * that takes the place of the dense FFN; its steps are those of "Switch
 * Routing: From Top-k to k = 1" and "Expert Capacity and the Capacity
 * Factor") in one stream-ordered call: the results of switch_route,
 * switch_dispatch, switch_expert_ffn and switch_combine, fused.  The expert
 * FFN reads each kept token's row of x directly (no dispatch copy) and
 * writes y[t] = gate[t] * E_e(x_t) (+ x_t) straight from its fp32
 * accumulators, so every output element is rounded once.  In bf16 with
 * d_model 128 or 256, d_ff a multiple of 128 and capacity <= 160 (shapes
 * where it was measured faster), the whole expert FFN is one kernel and the hidden activations
 * ReLU(W_in x) never leave the chip (rounded to bf16 between the two
 * products, as in switch_expert_ffn); other shapes run the up-projection
 * into a workspace buffer, then the down-projection.  The workspace holds
 * the router's partial results and the slot -> token map; it is NOT a valid
 * forward workspace for switch_layer_backward, which needs the hidden
 * activations that switch_layer_forward_train saves.  add_residual != 0 returns y = x + layer output
 * (dropped tokens then pass x through unchanged); 0 returns the bare layer
 * output (0 for dropped tokens).  Outputs as for switch_route plus y [T][d]. */
int switch_layer_forward(const switch_shape *s, const void *x, const float *w_router, const float *router_bias,
                         const void *w_in, const void *w_out, int32_t add_residual, void *y,
                         int32_t *expert_idx, float *gate, int32_t *slot, uint8_t *dropped,
                         int32_t *expert_count, float *aux_loss, void *workspace, size_t workspace_bytes,
                         void *stream);

/* The Switch layer followed by the block's Add + Normalize ("The
 * Architecture in Place": the Switch FFN layer's output is added to its
 * input x and normalized), in the layer call:
 *   out[t] = (v - mean(v)) / sqrt(var(v) + eps) * gamma + beta,
 *   v = x[t] + y_bare[t]   (y_bare = 0 for dropped tokens),
 * mean and population variance over the d_model features of the row; gamma,
 * beta [d_model] fp32 (device); eps host scalar, finite and >= 0.  fp32
 * arithmetic from the layer's fp32 accumulators (y_bare is not rounded
 * before the sum), one rounding of each output.  out [T][d] replaces y; the
 * routing outputs and the workspace are those of switch_layer_forward.  Where
 * switch_layer_forward runs one fused expert kernel the normalization is its
 * epilogue (dropped rows: the assignment kernel); elsewhere the bare layer
 * writes out, then switch_add_norm's kernel normalizes it in place.  Errors:
 * as switch_layer_forward; SWITCH_E_INVALID for NULL / misaligned gamma or
 * beta or a bad eps; SWITCH_E_UNSUPPORTED for d_model above switch_add_norm's
 * limit. */
int switch_layer_forward_add_norm(const switch_shape *s, const void *x, const float *w_router,
                                  const float *router_bias, const void *w_in, const void *w_out, const float *gamma,
                                  const float *beta, float eps, void *out, int32_t *expert_idx, float *gate,
                                  int32_t *slot, uint8_t *dropped, int32_t *expert_count, float *aux_loss,
                                  void *workspace, size_t workspace_bytes, void *stream);

/* The layer forward of a training step: the same results as
 * switch_layer_forward (bit for bit where both take the two-product path;
 * elsewhere the same arithmetic in a different kernel, so y may differ in the
 * last bf16 place), and the workspace then also holds what
 * switch_layer_backward reads: the hidden activations H [N][C][d_ff] of the
 * kept rows besides the slot maps ("The Core Idea": E(x) = W_out ReLU(W_in
 * x); its gradient needs ReLU(W_in x)).  Same arguments, workspace size and
 * errors as switch_layer_forward. */
int switch_layer_forward_train(const switch_shape *s, const void *x, const float *w_router,
                               const float *router_bias, const void *w_in, const void *w_out, int32_t add_residual,
                               void *y, int32_t *expert_idx, float *gate, int32_t *slot, uint8_t *dropped,
                               int32_t *expert_count, float *aux_loss, void *workspace, size_t workspace_bytes,
                               void *stream);

/* switch_layer_forward for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same kernels and results, with the workspace in a static
 * device array of switch_noalloc_scratch_bytes (128 MiB) that the library
 * holds on every GPU it runs on until the process ends.  Nothing is allocated
 * or freed by the call.  Arguments as switch_layer_forward without the
 * workspace; SWITCH_E_WORKSPACE (nothing launched) when the shape needs more
 * workspace than the array holds (switch_workspace_bytes tells; the base and
 * large layers fit).  The array keeps the last call's contents, and no kernel
 * of the layer reads workspace it has not written in the same call.  Every
 * call on one GPU uses that GPU's one array: calls whose work overlaps on the
 * GPU (on different streams, or from several threads) race and give
 * undefined results; serialise them.  The first call on each device looks up
 * the array's device address (hipGetSymbolAddress) with that device current;
 * SWITCH_E_HIP if that fails. */
int switch_layer_forward_noalloc(const switch_shape *s, const void *x, const float *w_router,
                                 const float *router_bias, const void *w_in, const void *w_out,
                                 int32_t add_residual, void *y, int32_t *expert_idx, float *gate, int32_t *slot,
                                 uint8_t *dropped, int32_t *expert_count, float *aux_loss, void *stream);

/* Bytes of the static workspace switch_layer_forward_noalloc uses.  Host only. */
int switch_noalloc_scratch_bytes(size_t *bytes_out);

/* The block's "Add + Normalize" after the layer (Switch Transformers
 * write-up, "The Architecture in Place", the block figure): for every token t,
 * out[t] = (v - mean v) / sqrt(var v + eps) * gamma + beta with v = x[t] +
 * y[t] (layer normalisation over d_model: mean and population variance of the
 * row; x may be NULL, then v = y[t]).  Typical use: y = the bare output of
 * switch_layer_forward (add_residual = 0) and x its input, so the residual add
 * happens in fp32 inside the normalisation.  Uses s->tokens, s->d_model,
 * s->dtype: x, y, out [T][d] of that dtype (16-byte aligned); gamma, beta [d]
 * fp32; eps finite and >= 0.  out may be y itself (in place); it must not
 * overlap x or y otherwise.  Arithmetic in fp32, one rounding to the output
 * dtype; deterministic.  SWITCH_E_UNSUPPORTED for d_model above 4096 (bf16) /
 * 2048 (fp32). */
int switch_add_norm(const switch_shape *s, const void *x, const void *y, const float *gamma, const float *beta,
                    float eps, void *out, void *stream);

/* Classic top-k MoE layer, the variant the Switch layer simplifies
 * ("Switch Routing: From Top-k to k = 1": each token goes to its top-k
 * experts and the output is the gate-weighted sum y = sum over the selected
 * set of p_i(x) E_i(x)), for top_k = 1 or 2.  top_k = 1 gives exactly
 * switch_layer_forward.  Readings of what the write-up leaves open:
 *   - route r (0-based) of a token goes to its expert with the (r+1)-th
 *     largest logit; equal logits rank the lower index first;
 *   - gate[r][t] = p_i(x) of that expert (the full softmax, not renormalised
 *     over the chosen experts);
 *   - capacity is claimed route-major: all first routes in token order, then
 *     all second routes; slot[r][t] = number of earlier routes in that order to
 *     the same expert; dropped[r][t] = slot >= capacity (a dropped route adds
 *     nothing; the token keeps its other routes).  s->capacity is the caller's
 *     (switch_capacity(top_k * tokens, ...) gives k T / N x cf, room for k
 *     routes' worth of tokens);
 *   - expert_count[i] = routes to expert i before capacity; aux_loss = N sum_i
 *     f_i P_i with f_i = expert_count[i] / (top_k T).
 * Arguments as switch_layer_forward, except: expert_idx, gate, slot, dropped
 * are [top_k][T] (route-major); workspace of switch_topk_workspace_bytes
 * (for top_k = 2 it holds a [2][T][d_model] buffer of gate-scaled expert
 * outputs that a last kernel sums per token, in route order, in fp32, with one
 * rounding to y's dtype).  Errors: SWITCH_E_INVALID for top_k < 1 or above
 * num_experts; SWITCH_E_UNSUPPORTED for top_k > 2 or top_k x tokens above
 * 2^31-1. */
int switch_topk_workspace_bytes(const switch_shape *s, int32_t top_k, size_t *bytes_out);
int switch_topk_layer_forward(const switch_shape *s, int32_t top_k, const void *x, const float *w_router,
                              const float *router_bias, const void *w_in, const void *w_out, int32_t add_residual,
                              void *y, int32_t *expert_idx, float *gate, int32_t *slot, uint8_t *dropped,
                              int32_t *expert_count, float *aux_loss, void *workspace, size_t workspace_bytes,
                              void *stream);

/* Backward pass of the Switch layer (k = 1): the gradients of a loss
 * L = <dy, y> + d_aux * aux_loss with respect to the layer's inputs, for the
 * routing of the preceding switch_layer_forward call ("Switch Routing: From
 * Top-k to k = 1": the gate multiplies the expert output, which keeps the
 * router differentiable; "The Load-Balancing Loss": f_i is a hard count with
 * no gradient, P_i is differentiable; "Making Sparse Training Stable": the
 * router's arithmetic stays in fp32).  The routing is held fixed: expert
 * choices, drops and f_i are the forward's.  For a kept token t with expert
 * e, gate g, u = W_in,e x, h = ReLU(u) and z = W_out,e^T dy_t:
 *   dL/dg = <z, h>,  du = g z [h > 0],
 *   dW_out,e += (g dy_t) h^T,  dW_in,e += du x_t^T,  dx_t += W_in,e^T du;
 * router, every token: dL/dp_i = d_aux N f_i / T + [i = e, t kept] dL/dg,
 *   dL/dh = p (dL/dp - <dL/dp, p>),  dW_r += dL/dh x_t^T,
 *   dbias += dL/dh,  dx_t += W_r^T dL/dh;  with add_residual, dx_t += dy_t.
 * Inputs: the forward's shape, x, w_router, router_bias, w_in, w_out and
 * add_residual; its outputs expert_idx [T], dropped [T], expert_count [N];
 * fwd_workspace: the workspace of a switch_layer_forward_train call on the
 * same inputs, unmodified since (it holds the hidden activations H and the
 * slot maps; a switch_layer_forward workspace lacks H); dy [T][d] (activation
 * dtype); d_aux (host scalar, finite: the weight of aux_loss in L, e.g. the
 * alpha of the write-up).
 * Outputs (device, caller-owned, overwritten): dx [T][d] and dw_in
 * [N][d_ff][d], dw_out [N][d][d_ff] in the activation dtype; dw_router [N][d]
 * and d_router_bias [N] (may be NULL) in fp32.  An expert that received no
 * kept token gets exact zeros.  Arithmetic: bf16 MFMA with fp32 accumulation
 * for the expert products (du and g dy rounded to bf16 as operands), fp32 for
 * the router (in bf16 layers the router's matrix products run on bf16 MFMA
 * from exact three-way bf16 splits of their fp32 operands: dW_r with all
 * products exact, W_r^T dL/dh with the six plane products above 2^-24 of the
 * result); dx summed in fp32 and rounded once.  Deterministic.
 * workspace: switch_backward_workspace_bytes bytes (256-byte aligned).
 * Errors: as switch_layer_forward; SWITCH_E_WORKSPACE if fwd_workspace_bytes
 * is below the forward's workspace size; SWITCH_E_UNSUPPORTED for
 * s->weight_layout = SWITCH_WEIGHTS_TILED (the backward reads, and writes
 * dw_in / dw_out, row-major: keep a row-major copy of the weights for
 * training, or convert with switch_untile_weights). */
int switch_backward_workspace_bytes(const switch_shape *s, size_t *bytes_out);
int switch_layer_backward(const switch_shape *s, const void *x, const float *w_router, const float *router_bias,
                          const void *w_in, const void *w_out, int32_t add_residual, const int32_t *expert_idx,
                          const uint8_t *dropped, const int32_t *expert_count, const void *fwd_workspace,
                          size_t fwd_workspace_bytes, const void *dy, float d_aux, void *dx, float *dw_router,
                          float *d_router_bias, void *dw_in, void *dw_out, void *workspace, size_t workspace_bytes,
                          void *stream);
/* Measurement variant of switch_layer_backward, with the contract of
 * switch_layer_forward_profiled: kernels first_kernel..last_kernel only, each
 * `times` times.  The backward's launch steps, in order: "bwd_dz",
 * "bwd_dw_out", "bwd_dx", "bwd_dw_in", "bwd_router", "bwd_router_dx" (bf16
 * layers: the router's part of dx on matrix cores, two launches; fp32 layers:
 * none, dx is formed in "bwd_router"), "bwd_router_w", "bwd_router_w_sum";
 * none modifies its own inputs. */
int switch_layer_backward_profiled(const switch_shape *s, const void *x, const float *w_router,
                                   const float *router_bias, const void *w_in, const void *w_out,
                                   int32_t add_residual, const int32_t *expert_idx, const uint8_t *dropped,
                                   const int32_t *expert_count, const void *fwd_workspace,
                                   size_t fwd_workspace_bytes, const void *dy, float d_aux, void *dx,
                                   float *dw_router, float *d_router_bias, void *dw_in, void *dw_out,
                                   void *workspace, size_t workspace_bytes, void *stream, int32_t first_kernel,
                                   int32_t last_kernel, int32_t times);

/* Combine and the block's Add + Normalize in one pass (stage API; the
 * write-up's block figure puts "Add + Normalize" right after the combine):
 *   out[t] = LayerNorm(x[t] + y[t]),  y[t] = gate[t] * expert_out[expert_idx[t]][slot[t]]
 * (y[t] = 0 for a dropped token), with the statistics and the
 * definitions of switch_add_norm.  The sum is formed in fp32 from the expert
 * output and rounded once (switch_combine followed by switch_add_norm
 * rounds y first).  Arguments as switch_combine (expert_out [N][C][d], the
 * routing arrays [T]) plus x [T][d] (required), gamma, beta [d] fp32, eps;
 * out [T][d] must not overlap the inputs.  SWITCH_E_UNSUPPORTED for d_model
 * above 4096 (bf16) / 2048 (fp32). */
int switch_combine_add_norm(const switch_shape *s, const void *expert_out, const int32_t *expert_idx,
                            const int32_t *slot, const uint8_t *dropped, const float *gate, const void *x,
                            const float *gamma, const float *beta, float eps, void *out, void *stream);

/* Measurement variant of switch_layer_forward: same arguments and
 * asynchrony, but it launches only the kernels numbered first_kernel ..
 * last_kernel of the call (0-based, in the order switch_launch_names gives),
 * each `times` (>= 1) times back to back.  Every kernel of the layer reads
 * only the inputs and what earlier kernels of the call left in the
 * workspace, and never its own outputs: after one full call, calls covering
 * 0..i-1, then i..i, then i+1..n-1 reproduce the full call exactly, so a
 * caller can bracket kernel i with its own events inside an otherwise
 * ordinary step.  SWITCH_E_INVALID if the range is empty or past the last
 * kernel of this shape. */
int switch_layer_forward_profiled(const switch_shape *s, const void *x, const float *w_router,
                                  const float *router_bias, const void *w_in, const void *w_out,
                                  int32_t add_residual, void *y, int32_t *expert_idx, float *gate,
                                  int32_t *slot, uint8_t *dropped, int32_t *expert_count, float *aux_loss,
                                  void *workspace, size_t workspace_bytes, void *stream, int32_t first_kernel,
                                  int32_t last_kernel, int32_t times);

/* Names of the kernels switch_layer_forward launches for this shape, in
 * launch order (static strings: "router", then "assign" or "assign_scan" +
 * "assign_apply", then "ffn_up", "ffn_down").  Up to max_names are stored in
 * names[]; *num_names receives their number (at most 5).  Host only. */
int switch_launch_names(const switch_shape *s, const char **names, int32_t max_names, int32_t *num_names);

/* Expert weights between the two layouts of SWITCH_WEIGHTS_ROWS and
 * SWITCH_WEIGHTS_TILED (defined at switch_shape): count bf16 matrices of
 * rows x cols (W_in: count = N, rows = d_ff, cols = d_model; W_out: rows =
 * d_model, cols = d_ff), src -> dst, device pointers, 16-byte aligned, not
 * overlapping, count * rows * cols * 2 bytes each.  A pure permutation of
 * 16-byte pieces: untile(tile(w)) == w bit for bit.  A conversion of the
 * parameters (after loading or updating them), not part of a layer call:
 * the layer with tiled weights computes the same products in the same order
 * as with row-major ones ("The Core Idea: Sparse Activation via Routing":
 * each expert is an ordinary FFN; only its storage changes).  Enqueued on
 * `stream`.
 * Errors: SWITCH_E_INVALID (negative sizes, NULL / misaligned / overlapping
 * pointers when there is anything to move), SWITCH_E_UNSUPPORTED (rows not a
 * multiple of 16 or cols of 32, sizes overflowing), SWITCH_E_HIP. */
int switch_tile_weights(int32_t count, int32_t rows, int32_t cols, const void *src, void *dst, void *stream);
int switch_untile_weights(int32_t count, int32_t rows, int32_t cols, const void *src, void *dst, void *stream);

/* Router weights in the form SWITCH_WEIGHTS_TILED reads (defined at
 * switch_shape).  w_router: W_r [num_experts][d_model] fp32, row-major.
 * planes: switch_tiled_router_bytes(num_experts, d_model) bytes =
 * ceil(num_experts / 16) x d_model / 32 x 3 KB: for each tile of 16 experts
 * and 32 columns, three 1 KB pieces (the hi, mid and lo bf16 planes, each
 * taking the next 8 significant bits of every value, so hi + mid + lo is the
 * fp32 value exactly), each piece 64 lanes x 8 bf16 with lane l holding
 * expert 16 tile + l % 16 (zeros past num_experts) at columns 8 (l / 16) ..
 * + 7 of the 32.  The router stays fp32 ("Making Sparse Training Stable",
 * selective precision): every product of a bf16 token value with a plane is
 * exact in fp32.  A conversion of the parameters, like
 * switch_tile_weights; device pointers, 16-byte aligned, not overlapping;
 * enqueued on `stream`.  Errors: SWITCH_E_INVALID (num_experts or d_model
 * below 1, NULL / misaligned / overlapping pointers, NULL bytes_out),
 * SWITCH_E_UNSUPPORTED (d_model not a multiple of 64, sizes overflowing),
 * SWITCH_E_HIP. */
int switch_tiled_router_bytes(int32_t num_experts, int32_t d_model, size_t *bytes_out);
int switch_tile_router(int32_t num_experts, int32_t d_model, const float *w_router, void *planes, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* SWITCH_MOE_H */
