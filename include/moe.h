/*
 * moe.h -- C ABI of libmoe, the forward pass of a Mixture-of-Experts FFN layer
 * on AMD Instinct MI355X (gfx950).
 *
 * The layer (Vector Institute, "Mixture-of-Experts: From sparse routing to
 * multimodal deployment", router paragraphs and Eq. (moe-output); "Fine-Tuning
 * Mixture of Experts (MoE) Models: Router Optimization Techniques", What Is It?):
 *
 *   y[t] = sum over the k experts e selected for token t of  g_e(t) * FFN_e(x[t])
 *          (+ FFN_shared(x[t]) when a shared expert is configured)
 *
 * computed as five stages, each a call below, all enqueued on one HIP stream:
 *   moe_route       router logits, scores, top-k, gates, counts, balance statistics
 *   moe_permute     expert histogram, exclusive scan, stable expert-contiguous gather
 *   moe_grouped_ffn every expert's FFN as one grouped GEMM over variable-size segments
 *                   (= moe_expert_up then moe_expert_down)
 *   moe_shared_ffn  the always-on shared SwiGLU expert (dense)
 *   moe_combine     gate-weighted sum back to token order (+ shared output)
 * and moe_forward, which chains them; moe_backward differentiates the layer.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Memory:    every pointer argument is caller-owned DEVICE memory of the current
 *            HIP device (except `shape`, which is host memory). The library never
 *            allocates, frees or synchronises and keeps no state between calls;
 *            scratch comes only from the caller's workspace `ws` of `ws_bytes`
 *            bytes, sized by moe_workspace_bytes(), which needs no initialisation.
 *            The one exception is moe_permute_noalloc, whose scratch is a fixed
 *            array inside the library.
 * Layout:    row-major everywhere. Weights use the Linear [out, in] layout, so
 *            both operands of every product are contiguous along the reduced
 *            dimension. Expert weights are stacked along a leading expert axis.
 *            bf16 tensors hold IEEE bfloat16 bit patterns (uint16_t storage).
 * dtype:     `dtype` (MOE_F32 or MOE_BF16) is the type of x, expert weights and
 *            biases, x_perm, y_perm, y_shared and y. The router weights, the
 *            selection bias, logits, gates and statistics are always fp32
 *            ("Mixture of Experts" tutorial, Selective precision; "Fine-tuning and
 *            serving MoE models", the router softmax runs in FP32).
 * Alignment: every device pointer must be 16-byte aligned.
 * Streams:   `stream` is a hipStream_t passed as moe_stream_t; NULL is the null
 *            stream. Every call only enqueues work, so results are ready when the
 *            stream reaches that point. Calls are graph-capturable (no host
 *            synchronisation, no device-to-host reads).
 * Aliasing:  outputs must not overlap inputs or each other.
 * Errors:    every call returns MOE_OK (0) or a negative moe_status. All argument
 *            checks run on the host before any HIP call; a rejected call enqueues
 *            nothing. MOE_ERR_HIP reports a failed launch. T = 0 is a successful
 *            no-op. Non-finite inputs are outside the contract (not checked).
 * Threads:   re-entrant; concurrent calls on different streams with different
 *            workspaces are independent.
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    MOE_OK = 0,
    MOE_ERR_INVALID_ARG = -1, /* null required pointer, bad enum, inconsistent sizes, misalignment */
    MOE_ERR_UNSUPPORTED = -2, /* valid request the library does not implement (e.g. a bf16 backward
                                 with d_model % 64 != 0) */
    MOE_ERR_WORKSPACE = -3,   /* ws_bytes below moe_workspace_bytes() for the call */
    MOE_ERR_HIP = -4          /* a kernel launch failed (hipGetLastError) */
} moe_status;

/* dtype */
enum { MOE_F32 = 0, MOE_BF16 = 1 };
/* act: expert FFN form */
enum {
    MOE_GELU_MLP = 0, /* Linear(d->F, bias) + exact erf GELU + Linear(F->d, bias)
                         ("Fine-tuning and serving MoE models", How an MoE layer actually works) */
    MOE_SWIGLU = 1    /* (SiLU(x Wg^T) * (x Wu^T)) Wd^T, no biases
                         ("Router Optimization Techniques", What Is It?: W_gate, W_up, W_down) */
};
/* score: router scoring */
enum {
    MOE_SOFTMAX = 0, /* softmax over the E logits; selection on the logit (+ bias) */
    MOE_SIGMOID = 1  /* per-expert sigmoid; selection on sigmoid + bias; gates = s / sum_selected s */
};
/* stage argument of moe_workspace_bytes */
enum {
    MOE_STAGE_ROUTE = 0,
    MOE_STAGE_PERMUTE = 1,
    MOE_STAGE_FFN = 2,
    MOE_STAGE_SHARED = 3,
    MOE_STAGE_FORWARD = 4,
    MOE_STAGE_EXPERT = 5,      /* moe_expert_up / moe_expert_down */
    MOE_STAGE_ROUTE_NOISY = 6, /* moe_route_noisy */
    MOE_STAGE_BACKWARD = 7     /* moe_backward */
};

/* Layer description (host memory). Limits: T >= 0; 1 <= E <= 1024; 1 <= k <= min(E, 32); capacity >= 0;
 * T*k <= 2^31-1; d_model, d_ff and d_ff_shared multiples of 8 (bf16) or 4 (f32), so every row is
 * whole 16-byte vectors (MOE_ERR_INVALID_ARG otherwise); d_model, d_ff and d_ff_shared at most
 * MOE_MAX_WIDTH (MOE_ERR_UNSUPPORTED otherwise: the matrix kernels address a tile's operand rows
 * with 32-bit byte offsets); MOE_SIGMOID requires renorm = 1 (MOE_ERR_UNSUPPORTED). moe_backward on
 * bf16 layers further needs multiples of 64 (MOE_ERR_UNSUPPORTED). */
#define MOE_MAX_WIDTH (1 << 18)
typedef struct {
    int64_t T;           /* tokens */
    int32_t d_model;     /* hidden size d */
    int32_t d_ff;        /* routed expert intermediate size F */
    int32_t E;           /* routed experts */
    int32_t k;           /* experts per token */
    int32_t dtype;       /* MOE_F32 | MOE_BF16 */
    int32_t act;         /* MOE_GELU_MLP | MOE_SWIGLU */
    int32_t score;       /* MOE_SOFTMAX | MOE_SIGMOID */
    int32_t renorm;      /* 1: gates renormalised over the selected k; 0: raw softmax probabilities */
    int32_t d_ff_shared; /* shared SwiGLU expert intermediate size; 0 = no shared expert */
    int32_t capacity;    /* rows each expert may take (moe_permute); 0 = unlimited (dropless) */
} moe_shape;

typedef void* moe_stream_t; /* a hipStream_t */

/* Scratch bytes a call needs. stage: MOE_STAGE_*. Writes the size to *bytes (a status and an
 * out-parameter rather than a bare size_t, so an invalid shape or stage is reported, not sized).
 * Returns MOE_ERR_INVALID_ARG for an invalid shape or stage, else MOE_OK. */
int moe_workspace_bytes(const moe_shape* shape, int stage, size_t* bytes);

/* moe_route -- the router: logits, scores, per-token top-k, gates, counts, statistics.
 *
 * Defined by: Vector Institute post, router score W_r x and softmax, top-k, gate
 * renormalisation paragraph; "Router Optimization Techniques", What Is It? (h(x) = x W_g,
 * TopK, Softmax(TopK(h))), How It Works 1 (f_i, P_i, L_aux), How It Works 2 (bias used only
 * to pick the top-k, gates from the unbiased scores); "Fine-tuning and serving MoE models",
 * load_balancing_loss and the utilisation tally.
 *
 *   x        [T, d_model]  dtype          token activations
 *   w_router [E, d_model]  fp32           router weights (no router bias)
 *   sel_bias [E]           fp32 or NULL   selection-only bias: enters the top-k key, never a gate
 *   logits   [T, E]        fp32 or NULL   out: l[t,e] = sum_i x[t,i] w_router[e,i]
 *   topk_idx [T, k]        int32          out: selected experts, slot order = descending key,
 *                                         equal keys -> lower expert index first
 *   topk_w   [T, k]        fp32           out: gates of the selected experts, same slot order
 *   counts   [E]           int32          out: assignments per expert (sums to T*k)
 *   stats    [2E + 2]      fp32 or NULL   out: f[0..E) = counts/T, P[E..2E) = mean over tokens of
 *                                         the softmax probability (sigmoid: s / sum_e s),
 *                                         stats[2E] = aux = E * sum_e f_e P_e (alpha not applied),
 *                                         stats[2E+1] = mean token entropy -sum_e p ln p (nats)
 * Key: softmax -> logit (+ sel_bias); sigmoid -> sigmoid(logit) + sel_bias.
 * Gates: softmax & renorm -> softmax over the selected logits; softmax & !renorm -> full-softmax
 * probability; sigmoid -> selected sigmoid scores over their sum.
 * All reductions are deterministic (fixed order, no float atomics): repeated calls give
 * identical bits. Workspace: MOE_STAGE_ROUTE. */
int moe_route(const moe_shape* shape, const void* x, const float* w_router, const float* sel_bias,
              float* logits, int32_t* topk_idx, float* topk_w, int32_t* counts, float* stats,
              void* ws, size_t ws_bytes, moe_stream_t stream);

/* moe_route_noisy -- moe_route with noisy top-k gating.
 *
 * Defined by: "Mixture of Experts" tutorial, Noisy top-k gating: Gaussian noise is added to the
 * gating logits before the top-k, scaled per token by a second learned linear projection of x:
 *   H = x W_router^T + noise * softplus(x W_noise^T)
 * (the page's formula was lost; the scale is kept positive with softplus as in the published
 * recipe). H then replaces the logits everywhere: key, top-k, gates and statistics, exactly as in
 * moe_route. The noise is an input (the caller draws it), so the call is deterministic.
 *   w_noise [E, d_model] fp32  in: noise-scale projection
 *   noise   [T, E]       fp32  in: standard normal draws
 *   logits  [T, E] fp32 or NULL out: H
 * Other arguments as moe_route. Workspace: MOE_STAGE_ROUTE_NOISY. */
int moe_route_noisy(const moe_shape* shape, const void* x, const float* w_router, const float* w_noise,
                    const float* noise, const float* sel_bias, float* logits, int32_t* topk_idx,
                    float* topk_w, int32_t* counts, float* stats, void* ws, size_t ws_bytes,
                    moe_stream_t stream);

/* moe_permute -- expert-contiguous, stable order of the T*k assignments.
 *
 * Defined by: "Fine-tuning and serving MoE models", the loop over experts (nonzero(idx == e)
 * gathers each expert's tokens in ascending token order); "Router Optimization Techniques",
 * What Most Articles Miss 2 (all assigned tokens packed into one contiguous workspace).
 *
 *   topk_idx     [T, k]        int32  in: experts per token (each in [0, E); a token's k experts
 *                                     distinct, as moe_route produces; other values: undefined)
 *   x            [T, d_model]  dtype  in: token activations
 *   offsets      [E + 1]       int32  out: exclusive prefix sum of the rows each expert keeps;
 *                                     offsets[E] = T*k when dropless
 *   sorted_token [T*k]         int32  out: row p < offsets[E] of x_perm holds token sorted_token[p]
 *   inv_pos      [T*k]         int32  out: assignment (t, j) sits at row inv_pos[t*k + j], or -1
 *                                     when it was dropped
 *   x_perm       [T*k, d_model] dtype out: x_perm[p] = x[sorted_token[p]] for p < offsets[E];
 *                                     or NULL: positions only (offsets, sorted_token, inv_pos), the
 *                                     form moe_forward uses, whose up projection reads x's rows
 *                                     through sorted_token itself
 * Within an expert's segment rows are ordered by ascending t*k + j. Expert capacity
 * (shape->capacity = C > 0; "Router Optimization Techniques", Why It Matters 3 and FAQ 6, with
 * C = ceil(capacity factor * T * k / E); "Mixture of Experts" tutorial, The capacity factor
 * formula): an expert keeps only the first C of its assignments in that order; the others get
 * inv_pos = -1 and no row, and contribute nothing to the layer output (they reach the next layer
 * through the residual connection, outside this layer). Rows p >= offsets[E] are untouched.
 * Integer outputs are exact and deterministic. Workspace: MOE_STAGE_PERMUTE. */
int moe_permute(const moe_shape* shape, const int32_t* topk_idx, const void* x, int32_t* offsets,
                int32_t* sorted_token, int32_t* inv_pos, void* x_perm, void* ws, size_t ws_bytes,
                moe_stream_t stream);

/* moe_permute_noalloc -- moe_permute with no workspace argument and no allocation.
 *
 * For callers that cannot allocate device memory: code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc. Same arguments, outputs and errors as moe_permute,
 * without ws / ws_bytes; the outputs are bit-identical to moe_permute's.
 * Scratch: a fixed device array of MOE_NOALLOC_SCRATCH_BYTES (4 MiB) inside the library, one per
 * device, held until the process ends (its device address is looked up on the first call on each
 * device). A shape whose MOE_STAGE_PERMUTE workspace exceeds it returns MOE_ERR_WORKSPACE, before
 * any HIP call (the permute needs 8 * E * ceil(T*k / 1024) bytes, rounded up to 256 per region).
 * Every call on one device shares that array: calls that overlap on one device (other streams,
 * other host threads) race and must be serialised by the caller. Allocates nothing (no hipMalloc,
 * hipFree or allocating library call). */
#define MOE_NOALLOC_SCRATCH_BYTES (4u << 20)
int moe_permute_noalloc(const moe_shape* shape, const int32_t* topk_idx, const void* x, int32_t* offsets,
                        int32_t* sorted_token, int32_t* inv_pos, void* x_perm, moe_stream_t stream);

/* moe_grouped_ffn -- every expert's FFN on its contiguous rows, as one grouped GEMM pair.
 *
 * Defined by: "Router Optimization Techniques", What Is It? (expert = SwiGLU FFN with W_gate,
 * W_up, W_down) and Production Deployment 1 / What Most Articles Miss 2 (one grouped-GEMM launch
 * instead of one kernel per expert); "Fine-tuning and serving MoE models", the expert
 * Linear + GELU + Linear and grouped GEMM in one launch.
 *
 *   e_begin, e_end  experts [e_begin, e_end) are computed (0 <= e_begin <= e_end <= E); only rows
 *                   [offsets[e_begin], offsets[e_end]) of y_perm are written (the share of one
 *                   expert-parallel rank)
 *   x_perm  [T*k, d_model]      dtype  in: rows grouped by expert (moe_permute)
 *   offsets [E + 1]             int32  in: segment starts (device memory; never read by the host)
 *   w_in    [E, n_in, d_model]  dtype  in: GELU: n_in = d_ff (W1); SwiGLU: n_in = 2*d_ff,
 *                                      rows [0, d_ff) = W_gate, rows [d_ff, 2 d_ff) = W_up
 *   b_in    [E, d_ff]           dtype or NULL  GELU only (must be NULL for SwiGLU)
 *   w_out   [E, d_model, d_ff]  dtype  in: W2 / W_down
 *   b_out   [E, d_model]        dtype or NULL  GELU only
 *   y_perm  [T*k, d_model]      dtype  out: FFN_e(x_perm[p]) for each row p of expert e
 * Accumulation is fp32; bf16 layers round the intermediate activation once to bf16 (RNE) and
 * the output once. Empty experts cost nothing: the tile schedule is built on the device from
 * offsets. Workspace: MOE_STAGE_FFN (holds the intermediate activation h). */
int moe_grouped_ffn(const moe_shape* shape, int32_t e_begin, int32_t e_end, const void* x_perm,
                    const int32_t* offsets, const void* w_in, const void* b_in, const void* w_out,
                    const void* b_out, void* y_perm, void* ws, size_t ws_bytes, moe_stream_t stream);

/* moe_expert_up -- the first projection and activation of every expert (one grouped-GEMM launch,
 * plus a short second launch when the last round of tiles is split along K).
 *
 * The first half of moe_grouped_ffn, exposed on its own (same definitions and arguments):
 *   h [T*k, d_ff] dtype  out: GELU: gelu(x_perm[p] W1_e^T + b1_e); SwiGLU: SiLU(x_perm[p] Wg_e^T) *
 *                        (x_perm[p] Wu_e^T), for each row p of an expert e in [e_begin, e_end);
 *                        other rows untouched. bf16 layers round h once to bf16.
 * Workspace: MOE_STAGE_EXPERT (bf16 layers: fp32 partial tiles of the split last round, summed in a
 * fixed order, so results are deterministic; fp32 layers need none). */
int moe_expert_up(const moe_shape* shape, int32_t e_begin, int32_t e_end, const void* x_perm,
                  const int32_t* offsets, const void* w_in, const void* b_in, void* h, void* ws,
                  size_t ws_bytes, moe_stream_t stream);

/* moe_expert_down -- the second projection of every expert (launches as moe_expert_up).
 *
 * The second half of moe_grouped_ffn (same definitions and arguments):
 *   h      [T*k, d_ff]    dtype  in: moe_expert_up's output
 *   y_perm [T*k, d_model] dtype  out: h[p] W2_e^T (+ b2_e) for each row p of an expert in range.
 * Workspace: MOE_STAGE_EXPERT (as for moe_expert_up). */
int moe_expert_down(const moe_shape* shape, int32_t e_begin, int32_t e_end, const void* h,
                    const int32_t* offsets, const void* w_out, const void* b_out, void* y_perm, void* ws,
                    size_t ws_bytes, moe_stream_t stream);

/* moe_shared_ffn -- the always-on shared SwiGLU expert on every token (gate 1).
 *
 * Defined by: Vector Institute post, shared experts that run for every token (DeepSeekMoE);
 * "Router Optimization Techniques", lesson 2 (1 shared + 256 routed experts).
 *
 *   x        [T, d_model]             dtype  in
 *   ws_in    [2*d_ff_shared, d_model] dtype  in: rows [0, Fs) gate, [Fs, 2 Fs) up
 *   ws_out   [d_model, d_ff_shared]   dtype  in
 *   y_shared [T, d_model]             dtype  out
 * Requires shape->d_ff_shared > 0. Workspace: MOE_STAGE_SHARED. */
int moe_shared_ffn(const moe_shape* shape, const void* x, const void* ws_in, const void* ws_out,
                   void* y_shared, void* ws, size_t ws_bytes, moe_stream_t stream);

/* moe_combine -- gate-weighted sum of each token's k expert outputs, back in token order.
 *
 * Defined by: Vector Institute post, Eq. (moe-output); "Router Optimization Techniques",
 * MoE Layer Output = sum_{i in TopK} P_i(x) E_i(x); "Fine-tuning and serving MoE models",
 * index_add of gate-scaled expert outputs.
 *
 *   y_perm   [T*k, d_model] dtype        in
 *   inv_pos  [T*k]          int32        in: moe_permute's inverse permutation (-1: dropped by
 *                                        capacity; that slot contributes nothing)
 *   topk_w   [T, k]         fp32         in: gates
 *   y_shared [T, d_model]   dtype or NULL in: shared-expert output, added with gate 1
 *   y        [T, d_model]   dtype        out: y[t] = sum_j topk_w[t,j] y_perm[inv_pos[t*k+j]]
 *                                        (+ y_shared[t]), fp32 accumulation in slot order
 *                                        j = 0..k-1, shared last, one final rounding
 * Needs no workspace. */
int moe_combine(const moe_shape* shape, const void* y_perm, const int32_t* inv_pos, const float* topk_w,
                const void* y_shared, void* y, moe_stream_t stream);

/* moe_update_bias -- one step of auxiliary-loss-free load balancing on the selection bias.
 *
 * Defined by: "Router Optimization Techniques", How It Works 2 and Fine-Tuning Strategies 1 (the
 * dynamic-bias router): the uniform load is T*k/E assignments per expert; an expert above it
 * lowers its bias by gamma, one below raises it by gamma, one exactly at it keeps it:
 *   sel_bias[e] <- sel_bias[e] - gamma * sign(counts[e] - T*k/E)
 * The comparison is exact (counts[e] * E against T * k in 64-bit integers); the step is one fp32
 * subtraction.
 *   counts   [E]  int32  in: assignments per expert (moe_route's counts)
 *   sel_bias [E]  fp32   in/out: the bias moe_route adds to the selection key
 *   gamma         fp32   step (the pages use 0.001); must be finite
 * Needs no workspace. */
int moe_update_bias(const moe_shape* shape, const int32_t* counts, float gamma, float* sel_bias,
                    moe_stream_t stream);

/* moe_forward -- route, permute, grouped FFN, shared expert and combine on one stream.
 *
 * Same definitions as the stage calls. Inputs as in moe_route / moe_grouped_ffn /
 * moe_shared_ffn (ws_in and ws_out required iff d_ff_shared > 0). y [T, d_model] dtype is the
 * layer output. The optional outputs topk_idx_out [T,k] int32, topk_w_out [T,k] fp32,
 * counts_out [E] int32 and stats_out [2E+2] fp32 receive the routing results when non-NULL.
 * Workspace: MOE_STAGE_FORWARD. */
int moe_forward(const moe_shape* shape, const void* x, const float* w_router, const float* sel_bias,
                const void* w_in, const void* b_in, const void* w_out, const void* b_out,
                const void* ws_in, const void* ws_out, void* y, int32_t* topk_idx_out,
                float* topk_w_out, int32_t* counts_out, float* stats_out, void* ws, size_t ws_bytes,
                moe_stream_t stream);

/* moe_backward -- gradients of the layer for an output gradient dy (fine-tuning).
 *
 * Defined by: the chain rule through the forward above, for the fine-tuning the pages describe
 * ("Fine-tuning and serving MoE models", Why MoE breaks naive fine-tuning: task loss plus the
 * balancing loss, backpropagated; "Router Optimization Techniques", How It Works 1: L_aux puts
 * gradients on the router weights). The routing
 * choice is piecewise constant, so gradients reach the router only through the gates of the
 * selected experts ("Mixture of Experts" tutorial, Noisy top-k gating: entries outside the top-k are
 * -inf before the softmax); the selection bias gets none (it moves by moe_update_bias); assignments
 * dropped by capacity get none. Per piece (row vectors, Linear [out, in] weights):
 *   combine:  dg[t,j] = <dy[t], y_perm[row]>,  dY[row] = g[t,j] dy[t]
 *   expert:   GELU   dh = dY W2, dz = dh gelu'(z), dW1 = dz^T X, db1 = sum dz, dX = dz W1,
 *                    dW2 = dY^T h, db2 = sum dY;
 *             SwiGLU dh = dY Wd, da = dh u silu'(a), du = dh silu(a), dWg = da^T X, dWu = du^T X,
 *                    dX = da Wg + du Wu, dWd = dY^T h
 *   gates:    softmax & renorm: dl_S = g (dg - <g, dg>); softmax & !renorm: dl = p (dp - <p, dp>)
 *             with dp = dg on the selection; sigmoid: dl_S = (dg - <g, dg>) / sum_S s * s (1 - s)
 *   balance:  + gradient of aux_coef * E * sum_e f_e P_e with f = counts / T held constant
 *   router:   dW_router = dl^T x,  dx = sum of the kept slots' dX rows + shared dX + dl W_router
 * The expert pre-activations and h are recomputed from x_perm (one grouped GEMM), not stored by the
 * forward: the selective recomputation of the intra-expert activations that "Router Optimization
 * Techniques", Lessons From Production Deployments, Lesson 3 describes.
 *
 * Inputs: the forward's arguments (shape, x, w_router, w_in, b_in, w_out, b_out, ws_in, ws_out) and
 * its saved results:
 *   logits   [T, E]        fp32   moe_route's logits (moe_route_noisy: H)
 *   topk_idx [T, k], topk_w [T, k], counts [E] (NULL allowed when aux_coef == 0)   moe_route
 *   offsets [E + 1], inv_pos [T*k], x_perm [T*k, d_model]                          moe_permute
 *   y_perm   [T*k, d_model] dtype  moe_grouped_ffn's output
 *   dy       [T, d_model]   dtype  gradient of the loss with respect to y
 *   aux_coef                       weight of the balancing term (0: none); must be finite
 * Outputs (fp32 except dx):
 *   dx        [T, d_model]        dtype  one rounding of the fp32 sum
 *   dw_router [E, d_model]
 *   dw_in     [E, n_in, d_model], dw_out [E, d_model, d_ff]   zero for an expert without rows
 *   db_in [E, d_ff], db_out [E, d_model]   exactly when b_in / b_out are given (else NULL)
 *   dws_in [2 d_ff_shared, d_model], dws_out [d_model, d_ff_shared]   exactly when d_ff_shared > 0
 *   dlogits   [T, E] or NULL      the router logit gradient dl
 * Products accumulate in fp32 (bf16 layers: bf16 operands on the matrix cores; the recomputed
 * pre-activation, h, dY and the activation gradient are rounded once to bf16 as operands); every sum
 * runs in a fixed order, so results are deterministic. Gradients are written, not accumulated.
 * Workspace: MOE_STAGE_BACKWARD. */
int moe_backward(const moe_shape* shape, const void* x, const float* w_router, const void* w_in, const void* b_in,
                 const void* w_out, const void* b_out, const void* ws_in, const void* ws_out, const float* logits,
                 const int32_t* topk_idx, const float* topk_w, const int32_t* counts, const int32_t* offsets,
                 const int32_t* inv_pos, const void* x_perm, const void* y_perm, const void* dy, float aux_coef,
                 void* dx, float* dw_router, float* dw_in, float* db_in, float* dw_out, float* db_out,
                 float* dws_in, float* dws_out, float* dlogits, void* ws, size_t ws_bytes, moe_stream_t stream);

/* Human-readable name of a moe_status value (static string; never NULL). */
const char* moe_status_str(int status);

#ifdef __cplusplus
}
#endif

#endif /* MOE_H */
