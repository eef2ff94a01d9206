/*
 * switch_layer.h -- C ABI of the Switch FFN layer forward pass on MI355X (gfx950).
 *
 * One call computes, for T tokens x[T, d] (flattened batch x sequence, row-major):
 *   h[t, i]     = sum_k x[t, k] W_r[i, k] + b_r[i]              router logits, fp32
 *   p_i(t)      = softmax_i(h[t, :]);  e_t = argmax_i h[t, i] (lowest i on ties)
 *   gate[t]     = p_{e_t}(t)
 *   C           = ceil(c * T / N)   (or the configured override)
 *   position[t] = #{ t' < t : e_t' = e_t }                      token-order rank
 *   drop[t]     = position[t] >= C
 *   out[t]      = x[t] + gate[t] * W_out[e_t] relu(W_in[e_t] x[t])   if !drop[t]
 *               = x[t] (bit for bit)                                  if  drop[t]
 *   aux_loss    = alpha N sum_i f_i P_i,  f_i = load_i / T,  P_i = mean_t p_i(t)
 *
 * With top_k = 2 (classic top-2 MoE routing, the routing the Switch layer
 * simplifies: llm-papers-study section 3.1, where the output is the sum over
 * the K best experts of p_i(x) E_i(x), and the MoELayer code of the Incredible.AI
 * blog, section "Mixture of Experts Routing") every per-token output is [T, 2],
 * choice 0 the best expert and choice 1 the best of the rest (lowest index on
 * ties), gate[t, j] = p_{e_tj}(t) (not renormalised); assignments (t, j) take
 * positions in (token, choice) order against C = ceil(2 c T / N), each dropped
 * on its own; out[t] = x[t] + sum over kept j of gate[t, j] E_{e_tj}(x[t]); and
 * f_i = load_i / (2 T) with load_i counting assignments.
 *
 * Sources (the Switch Transformers paper as described on these pages):
 *   router logits and softmax -- "精读 06 | Switch Transformers" (llm-papers-study
 *     close reading), section 3.1; top-1 choice and the gate-scaled output --
 *     same page, section 3.2, and kasblo "Switch Transformerとは？", section
 *     "Top-1 Routingを数式で追う";
 *   capacity and overflow -- llm-papers-study section 3.4; kasblo sections
 *     "Expert Capacityはtokenの受付上限" and "16 token、4 Expertで考える";
 *     "Switch Transformer by Hand" (byhand.ai) steps 7 and 13;
 *   token-order truncation -- Incredible.AI blog "Switch Transformer - Scaling to
 *     Trillion Parameter Models...", section "MoE Layer";
 *   load-balancing loss -- llm-papers-study section 3.3; kasblo section
 *     "補助負荷分散lossは何を均等にするのか";
 *   fp32 router, bf16 dispatch/combine -- kasblo section "Routerだけfloat32で
 *     計算するSelective Precision";
 *   dispatch / expert matmul / combine -- kasblo section
 *     "tokenをExpertへ送って戻すforward pass".
 *
 * Conventions for every entry point:
 *   - Tensor pointers are DEVICE pointers (the caller owns them), contiguous,
 *     row-major, 16-byte aligned.  Scalars are host values.
 *   - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *     Calls only enqueue work on it and return; SWITCH_OK means "enqueued".
 *     Results are valid once the stream has reached that point.
 *   - Nothing is launched when a call returns an error status.  No call
 *     aborts the process, and no call allocates device memory: all scratch
 *     lives in the caller's workspace (switch_forward_noalloc: in a fixed
 *     array of the library).
 *   - Calls do not synchronise the stream; one handle may be used on several
 *     streams concurrently only with distinct workspaces and outputs.
 *   - Inputs must be finite.
 */
#ifndef SWITCH_LAYER_H
#define SWITCH_LAYER_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  SWITCH_OK = 0,
  SWITCH_E_INVALID = 1,      /* bad size, NULL required pointer, misalignment, T > t_max,
                                workspace too small */
  SWITCH_E_UNSUPPORTED = 2,  /* dtype combination or shape the kernels do not handle */
  SWITCH_E_HIP = 3,          /* a HIP runtime call or kernel launch failed */
  SWITCH_E_TOO_LARGE = 4     /* switch_forward_noalloc: the call needs more scratch than the
                                library's fixed array holds */
} switch_status;

typedef enum { SWITCH_F32 = 0, SWITCH_BF16 = 1 } switch_dtype;

/* How the expert FFN runs (switch_set_ffn_mode). */
typedef enum {
  SWITCH_FFN_AUTO = 0,     /* the library's choice (the default): the faster form measured
                              for the shape, at present the two-launch form */
  SWITCH_FFN_UNFUSED = 1,  /* two matmul launches, H [rows, F] through the workspace */
  SWITCH_FFN_FUSED = 2     /* one launch, H kept on chip (bf16, top-1, d a multiple of 256
                              up to 1024, F a multiple of 256) */
} switch_ffn_mode;

typedef struct {
  int64_t t_max;            /* largest T any call on this handle may pass (>= 0) */
  int32_t d_model;          /* d; a multiple of 8 (of 128 for bf16 layers) */
  int32_t d_ff;             /* F; a multiple of 8 (of 128 for bf16 layers) */
  int32_t n_experts;        /* 1 <= N <= 8192 */
  double capacity_factor;   /* c >= 0; C = ceil(c * T / N) evaluated in double */
  int32_t capacity_override;/* > 0: use this C instead of the formula */
  float alpha;              /* load-balancing loss coefficient (the paper uses 0.01) */
  int32_t act_dtype;        /* switch_dtype of x, out and the expert activations */
  int32_t expert_dtype;     /* switch_dtype of W_in / W_out; must equal act_dtype */
  int32_t top_k;            /* experts per token: 1 (the Switch layer; 0 also means 1)
                               or 2 (top-2 routing); k <= n_experts.  Per-token
                               outputs (expert_idx, gate, position, drop_mask) are
                               [T, k] row-major, and C = ceil(k c T / N) */
} switch_config;

typedef struct switch_layer switch_layer;

/*
 * Create a layer handle over caller-owned device weights: the router W_r (one
 * row per expert, llm-papers-study section 3.1, h(x) = W_r x) and N experts,
 * each the dense FFN it replaces (kasblo explainer, section
 * "TransformerのどこへSwitch layerが入るのか"), relu(x W_in^T) W_out^T with no
 * biases.  The capacity factor and alpha are those of llm-papers-study sections
 * 3.4 and 3.3.  Nothing is copied:
 * the weights are BORROWED and must stay valid and unchanged for the life of
 * the handle.
 *   W_r   [N, d] fp32 router weights (one row per expert)
 *   b_r   [N] fp32 router bias, or NULL for none
 *   W_in  [N, F, d] expert first-layer weights, expert_dtype
 *   W_out [N, d, F] expert second-layer weights, expert_dtype
 * On success *out receives the handle (host memory owned by the library;
 * release with switch_layer_destroy).  Returns SWITCH_E_INVALID for bad sizes
 * or NULL weights, SWITCH_E_UNSUPPORTED for other dtype mixes, SWITCH_E_HIP if
 * the current device cannot be queried.
 */
switch_status switch_layer_create(const switch_config* cfg, const float* W_r, const float* b_r,
                                  const void* W_in, const void* W_out, switch_layer** out);

/* Release a handle (NULL is allowed).  Does not touch the borrowed weights. */
void switch_layer_destroy(switch_layer* layer);

/* Capacity C used for a call with T tokens (-1 on a NULL handle or T < 0). */
int64_t switch_capacity(const switch_layer* layer, int64_t T);

/* Bytes of device workspace a switch_forward / switch_route call with T tokens needs
 * (0 on a NULL handle or T outside [0, t_max]). */
size_t switch_workspace_bytes(const switch_layer* layer, int64_t T);

/*
 * Routing stage only: router logits, softmax, top-1, capacity positions,
 * drops, per-expert loads and the load-balancing loss (llm-papers-study
 * sections 3.1 to 3.4: logits and softmax, the top-1 choice and its gate, the
 * auxiliary loss, capacity and overflow; positions in token order as the
 * Incredible.AI blog's MoE layer assigns them, section "MoE Layer").
 *   x          [T, d]  act_dtype input tokens
 *   logits     [T, N]  fp32 router logits, or NULL if not wanted
 *   expert_idx [T]     int32 chosen expert
 *   gate       [T]     fp32 softmax probability of the chosen expert (also for
 *                      dropped tokens)
 *   position   [T]     int32 token-order rank within the chosen expert (may be >= C)
 *   drop_mask  [T]     uint8 1 if position >= C
 *   aux_loss   [1]     fp32 load-balancing loss (device scalar)
 *   load       [N]     int32 tokens per expert before the capacity cut, or NULL
 *   ws, ws_bytes       device workspace of at least switch_workspace_bytes(T)
 * T = 0 is allowed (aux_loss = 0).
 */
switch_status switch_route(switch_layer* layer, const void* x, int64_t T, float* logits,
                           int32_t* expert_idx, float* gate, int32_t* position,
                           uint8_t* drop_mask, float* aux_loss, int32_t* load, void* ws,
                           size_t ws_bytes, void* stream);

/*
 * The whole layer (kasblo explainer, section "tokenをExpertへ送って戻す
 * forward pass": route, send each token to its expert, run the expert, bring
 * the result back scaled by the gate; llm-papers-study section 3.2 for
 * y = p_{i*} E_{i*}(x), section 3.4 and "Switch Transformer by Hand" step 13
 * for dropped tokens leaving on the residual): everything switch_route
 * returns, plus
 *   out [T, d] act_dtype layer output x + gate * E(x) (dropped tokens: x
 *   unchanged).  `out` must not overlap `x`.
 * Expert activations are rounded to bf16 between the two expert matmuls and
 * after the second (bf16 layers); accumulation is fp32 throughout.
 */
switch_status switch_forward(switch_layer* layer, const void* x, int64_t T, void* out,
                             int32_t* expert_idx, float* gate, int32_t* position,
                             uint8_t* drop_mask, float* aux_loss, float* logits, int32_t* load,
                             void* ws, size_t ws_bytes, void* stream);

/*
 * Backward pass of the layer (bf16 layers, top_k 1 or 2): gradients of a loss L given
 * grad_out = dL/dout and grad_aux = dL/daux_loss, at the routing of a forward
 * call on the same x.  The expert choice and the capacity cut carry no
 * gradient; the router learns through the gate p_{i*}(x) that scales the
 * chosen expert's output (kasblo "Switch Transformerとは？", section
 * "argmaxは離散なのに、Routerはなぜ学習できるのか") and through P_i of the
 * load-balancing loss (llm-papers-study section 3.3: f_i is a count, P_i is
 * differentiable):
 *   kept t:  dE = gate_t grad_out_t,  dgate_t = grad_out_t . E_t,
 *            dW_out[e] += dE relu(u)^T,  du = (W_out[e]^T dE) * [u > 0],
 *            dW_in[e] += du x_t^T,  dx_t += W_in[e]^T du;
 *   all t:   dp_i = [i = e_t, kept] dgate_t + grad_aux alpha N load_i / T^2,
 *            dh = p * (dp - p . dp),  dW_r += dh x_t^T,  db += dh,
 *            dx_t += grad_out_t + W_r^T dh.
 * With top_k = 2 every kept choice (t, j) is a "kept t" above with its own
 * gate, dp_i sums the dgate of the kept choices with e = i, and the loss term
 * is grad_aux alpha N load_i / (2 T^2) (load counts assignments).
 *   x, grad_out   [T, d] bf16 (grad_x must overlap neither)
 *   logits [T, N] fp32, expert_idx, gate, position, drop_mask [T] ([T, top_k]),
 *                 load [N]: the outputs of switch_forward / switch_route for this x
 *   grad_x        [T, d] bf16 out
 *   grad_W_r      [N, d] fp32 out;  grad_b_r [N] fp32 out, or NULL
 *   grad_W_in     [N, F, d] bf16 out;  grad_W_out [N, d, F] bf16 out
 *   ws, ws_bytes  device workspace of at least switch_backward_workspace_bytes(T)
 *   fwd_ws, fwd_ws_bytes  the workspace of that forward call (switch_forward,
 *                 unchanged since; at least switch_workspace_bytes(T)), whose
 *                 expert activations H are then read instead of recomputed
 *                 (the same values), or NULL.  A forward that ran the fused
 *                 expert FFN left no H there (a flag word in the workspace says
 *                 so): the backward then recomputes H into that workspace
 * Weight gradients are fp32 sums over the expert's tokens rounded once to bf16;
 * grad_x is summed in fp32 and rounded once.  Every output is written (zeros
 * where nothing contributes).  SWITCH_E_UNSUPPORTED for fp32 layers.  The
 * expert outputs Y are read from fwd_ws when that forward call kept them (see
 * switch_set_keep_expert_out; the call's second matmul writes a flag word into
 * its workspace, which the backward's kernels read on the device), else
 * recomputed; H is recomputed when fwd_ws is NULL.
 */
switch_status switch_backward(switch_layer* layer, const void* x, int64_t T, const void* grad_out,
                              float grad_aux, const float* logits, const int32_t* expert_idx,
                              const float* gate, const int32_t* position,
                              const uint8_t* drop_mask, const int32_t* load, void* grad_x,
                              float* grad_W_r, float* grad_b_r, void* grad_W_in,
                              void* grad_W_out, void* ws, size_t ws_bytes, void* fwd_ws,
                              size_t fwd_ws_bytes, void* stream);

/* Bytes of device workspace a switch_backward call with T tokens needs (0 on a
 * NULL handle or T outside [0, t_max]). */
size_t switch_backward_workspace_bytes(const switch_layer* layer, int64_t T);

/*
 * Expert FFN variant of the following forward calls of this layer.  Both compute
 * relu(x W_in[e]^T) rounded to bf16, its product with W_out[e]^T rounded to
 * bf16, and the combine, in fp32 sums; the fused variant keeps H on chip
 * instead of writing it to the workspace between two launches (the single-
 * device forward pass of the kasblo explainer, section
 * "tokenをExpertへ送って戻すforward pass", done in one pass over each expert's
 * tokens), and its sums run in another order, so the two agree within
 * rounding, not bit for bit.  Calls that must return or keep the expert outputs
 * (switch_forward_debug, switch_set_keep_expert_out(1)) and top-2 layers always
 * run the two-launch form.  SWITCH_E_UNSUPPORTED for SWITCH_FFN_FUSED on a
 * layer whose shape or type the fused kernel does not take; SWITCH_E_INVALID for
 * a NULL handle or another mode.
 */
switch_status switch_set_ffn_mode(switch_layer* layer, int mode);

/*
 * Training forward.  The gate's gradient needs the chosen expert's output Y
 * (dL/dgate = dL/dout . Y: the gradient reaches the router through the gate
 * that scales that output; kasblo explainer, section
 * "argmaxは離散なのに、Routerはなぜ学習できるのか").  keep = 1 makes the
 * following switch_forward calls of this layer also store Y in their workspace
 * (a few MB of extra writes from the combine epilogue), so that a
 * switch_backward given that workspace reads it instead of recomputing it;
 * keep = 0 (the default) stores nothing extra.  Outputs are the same either
 * way.  SWITCH_E_INVALID for a NULL handle or keep other than 0 or 1.
 */
switch_status switch_set_keep_expert_out(switch_layer* layer, int keep);

/*
 * Test hook: the routing stage from given fp32 logits [T, N] (device), with the
 * same outputs as switch_route minus the logits.  -inf logits are allowed
 * (probability 0); NaN is not.
 */
switch_status switch_route_from_logits(switch_layer* layer, const float* logits, int64_t T,
                                       int32_t* expert_idx, float* gate, int32_t* position,
                                       uint8_t* drop_mask, float* aux_loss, int32_t* load,
                                       void* ws, size_t ws_bytes, void* stream);

/*
 * Test hook: switch_forward that also copies the expert outputs E(x) of the
 * kept tokens into expert_out [N, Cb, d], Cb = min(C, T) (act_dtype, row p of
 * expert e holds the token with position p; rows p >= n_e are left untouched).
 * expert_out may be NULL only when Cb = 0.
 */
switch_status switch_forward_debug(switch_layer* layer, const void* x, int64_t T, void* out,
                                   int32_t* expert_idx, float* gate, int32_t* position,
                                   uint8_t* drop_mask, float* aux_loss, float* logits,
                                   int32_t* load, void* ws, size_t ws_bytes, void* expert_out,
                                   void* stream);

/*
 * Per-kernel timing for measurement.  switch_profile_enable(layer, n) makes the
 * next n switch_forward / switch_route / switch_backward calls time each stage
 * (a kernel, or a few kernels in a row) with HIP events that the kernel
 * dispatches themselves record (hipExtLaunchKernel: the start of the stage's
 * first kernel, the end of its last), on the call's stream, without
 * synchronising (n = 0 turns recording off and frees the events; calls past
 * the n-th are not recorded).  switch_profile_read waits for the last
 * recorded call to finish and writes, for each stage in launch order, the mean
 * time in milliseconds over the recorded calls and its name (a static string);
 * all recorded calls must have launched the same stages.  Returns the number of
 * stages (at most `cap` are written), 0 if nothing was recorded, -1 on error.
 * Enabling allocates host memory and HIP events (SWITCH_E_HIP on failure).
 */
switch_status switch_profile_enable(switch_layer* layer, int max_calls);
int switch_profile_read(switch_layer* layer, float* ms, const char** names, int cap);

/*
 * For callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc): switch_forward with the
 * same arguments and results minus the workspace.  Its scratch is a fixed device
 * array inside the library, SWITCH_NOALLOC_SCRATCH_BYTES (64 MiB), one copy per
 * GPU: it is resolved when the first handle is created on that GPU and held until
 * the process ends.  The call itself allocates nothing.
 *   - Returns SWITCH_E_TOO_LARGE, launching nothing, when the call would need more
 *     than the array holds (switch_workspace_bytes(layer, T) > the maximum; the
 *     Switch-Base shape, 4096 tokens of d = 768, F = 3072 over 8 experts, needs
 *     about 40 MB).  SWITCH_E_HIP if the array's address could not be resolved.
 *   - Every call on one GPU, from any handle, stream or thread, uses that GPU's one
 *     array: calls that overlap on one GPU race, and the caller must order them
 *     (one stream, or events).  The array keeps the last call's contents; the
 *     forward writes everything it reads there, so nothing must start at zero.
 *   - The array is not a forward workspace for switch_backward (its address is not
 *     exported).
 */
#define SWITCH_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
switch_status switch_forward_noalloc(switch_layer* layer, const void* x, int64_t T, void* out,
                                     int32_t* expert_idx, float* gate, int32_t* position,
                                     uint8_t* drop_mask, float* aux_loss, float* logits,
                                     int32_t* load, void* stream);

/* Human-readable name of a status code (static string). */
const char* switch_status_string(switch_status s);

/*
 * Error state of the work this library enqueued for `layer` on `stream`, without
 * waiting: SWITCH_E_HIP if a launch on this thread failed since the last check
 * (hipGetLastError, which also clears it) or the stream reports a failed kernel
 * (hipStreamQuery); SWITCH_OK otherwise, also while the work is still running.
 * SWITCH_E_INVALID for a NULL layer or when the current device is not the
 * layer's.
 */
switch_status switch_last_async_error(switch_layer* layer, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* SWITCH_LAYER_H */
