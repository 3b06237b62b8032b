/*
 * ttt.h -- C ABI of libttt, the MI355X (gfx950) hot path of TTT layers.
 *
 * A TTT layer keeps, per (batch, head), a hidden state that is itself a small
 * model and trains it on the sequence while reading it: tokens are grouped in
 * mini-batches of K; inside a mini-batch every token contributes the loss
 *     l_j = 1/2 || LN(f(k_j)) - (v_j - k_j) ||^2
 * at the mini-batch-start parameters, the output of token i is
 *     out_i = q_i + LN(f_i(q_i)),
 * where f_i is the state after one gradient step on the losses of tokens
 * j <= i of the mini-batch, each weighted by the token's learning rate eta_j,
 * and the step over the whole mini-batch is carried to the next one.
 * TTT-Linear: f(x) = x W + b.  TTT-MLP: f(x) = GELU(x W1 + b1) W2 + b2.
 *
 * Sources (web pages, by title and listing/section):
 *  - "代码连连看——TTT" (jiafeimiao.top): listings TTTBase.forward (layout,
 *    rotary at position mod mini_batch_size, remainder handling),
 *    TTTLinear.ttt (state tiling, dual/primal choice, cache update) and
 *    compute_mini_batch (dual branch: Z1, Attn1, b1_bar, Z1_bar, W1_last,
 *    b1_last; primal branch: grad_W1, W1_bar, the carried gradients);
 *    closing remark that TTT-MLP is TTT-Linear stacked twice.
 *  - "测试时学习（TTT）原理解析" (nanhubrain.csdn.net): TTTLinear parameter
 *    init (section "TTT的核心创新"), TTTCache with seqlen_offset and
 *    mini_batch_size (section "TTT缓存机制").
 *  - ttt-lm-pytorch README (downcodes.com): TTT-Linear and TTT-MLP hidden
 *    states; quick start with prefill and decoding.
 *
 * Readings where the pages leave a step open (the bodies of ln_fwd,
 * ln_fused_l2_bwd, the rotary helpers, get_ttt_inputs and TTTCache.update are
 * not printed):
 *  - LN uses the population variance with eps inside the square root;
 *    gamma/beta are per head ("ttt_norm_weight/bias" reshaped per head);
 *  - the loss is half the squared error;
 *  - eta_ij = token_eta_i * lr_j: lr_j is the learning rate of key token j,
 *    token_eta_i scales the step seen by output row i of the mini-batch and
 *    the step carried at the boundary is that of the last row (token_eta is
 *    optional, all ones by default); the causal mask includes the diagonal;
 *  - rotary embedding pairs dimension i with i + D/2, angle
 *    p * base^(-2i/D), p = absolute position mod K; applied to q and k only,
 *    before everything else (target and residual use the rotated values);
 *  - between mini-batch boundaries the state holds the mini-batch-start W, b
 *    plus the accumulated eta-weighted gradients (the pages' W1_grad,
 *    b1_grad); they are committed and cleared at every boundary;
 *  - TTT-MLP uses the erf form of GELU, x * Phi(x) (the kernel evaluates erf
 *    to within 1.5e-7, Abramowitz & Stegun 7.1.26).
 *
 * Conventions for every entry point:
 *  - Memory: the caller allocates every buffer (device memory unless stated)
 *    and keeps ownership.  libttt allocates no device memory and keeps no
 *    per-call state; its only global is the per-thread error message.
 *  - Streams: ``stream`` is a hipStream_t passed as void* (NULL = the null
 *    stream).  Calls only enqueue work; results are valid once the stream has
 *    been synchronised.  There is no host/device synchronisation inside.
 *  - Activations use ttt_tensor: element strides for batch, head and token,
 *    the D values of one (b, h, t) contiguous.  The pages' [B, L, H*D] layout
 *    is sB = L*H*D, sH = D, sL = H*D; [B, H, L, D] is sB = H*L*D, sH = L*D,
 *    sL = D.  Data pointers and every stride in bytes must be multiples of
 *    16 bytes.
 *  - Errors: on any status other than TTT_OK nothing has been enqueued and
 *    the state (including ``offset``) is unchanged, with one exception: a
 *    call is split into up to three launches (below), and if the runtime
 *    refuses a later launch after an earlier one was enqueued, the call
 *    returns TTT_ERR_HIP with ``offset`` advanced by the tokens of the
 *    enqueued launches (their work completes; the state is consistent with
 *    the new offset).  An error left by an earlier HIP call on the thread is
 *    reported (and cleared) as TTT_ERR_HIP before anything is enqueued.
 *    ttt_last_error() returns a per-thread message describing the last
 *    failure.
 *  - Inputs (XQ, XK, XV, eta, ln_w, ln_b, token_eta) and out must not
 *    overlap the state buffers, and out must not overlap an input
 *    (TTT_ERR_ALIAS).
 *  - NaN/Inf in the inputs propagate to the outputs; they are not checked.
 *  - Range of bf16 inputs.  With bf16 inputs, whole mini-batches (K = 16) run
 *    their products on fp16 MFMA operands with fp32 accumulation (fp16's 11
 *    significant bits keep the 2e-2 output bar that bf16's 8 would not).
 *    The gradients are carried scaled by 2^8 and the 16x16 matrices they
 *    multiply by 2^-8, which leaves every product unchanged; the values must
 *    then stay within fp16's range: |q|, |k| (after rotary) and |W| (TTT-MLP:
 *    |W1|, |W2|, |GELU(x W1 + b1)|) at most 65504; dot products of two
 *    q/k rows of a mini-batch, of k rows of neighbouring mini-batches and
 *    (TTT-MLP) of two hidden-activation rows below 2^8 * 65504 = 1.7e7; and
 *    |eta_j g_j| elementwise below 256.  Outside these bounds the results
 *    are undefined (typically inf or NaN).  fp32 inputs have no such bounds
 *    (fp32 MFMA for TTT-Linear, fp32 arithmetic for TTT-MLP).
 *  - Calls on one state must be ordered (same stream, or synchronised);
 *    calls on distinct states and buffers may run concurrently.
 */
#ifndef TTT_H
#define TTT_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum ttt_status {
    TTT_OK = 0,
    TTT_ERR_NULL = 1,        /* a required pointer is NULL */
    TTT_ERR_SHAPE = 2,       /* D != 64, K outside 1..16, B/H/L < 1, F != 256 */
    TTT_ERR_DTYPE = 3,       /* unknown in/out dtype */
    TTT_ERR_ALIGN = 4,       /* pointer or stride not a multiple of 16 bytes */
    TTT_ERR_ALIAS = 5,       /* out overlaps an input or the state, or an input overlaps the state */
    TTT_ERR_STATE = 6,       /* negative offset, or state incompatible with the call */
    TTT_ERR_UNSUPPORTED = 7, /* valid request outside what is implemented */
    TTT_ERR_HIP = 8          /* the HIP runtime reported an error at launch */
} ttt_status;

typedef enum ttt_dtype {
    TTT_F32 = 0,
    TTT_BF16 = 1
} ttt_dtype;

/* Strided activation tensor [B, H, L, D]; D contiguous; strides in elements. */
typedef struct ttt_tensor {
    void *data;
    int64_t sB, sH, sL;
} ttt_tensor;

/* Learning rates.
 *  data:      eta[b, h, t] (fp32, token stride 1); sB = 0 shares them over
 *             the batch.  The rate of key token t ("ttt_lr_eta" in
 *             compute_mini_batch).
 *  token_eta: NULL, or K fp32 values (device, 16-byte aligned): the scale of
 *             the step seen by the token at position i (mod K) of its
 *             mini-batch ("token_eta" in compute_mini_batch: the primal
 *             branch's W1_bar = W1_init - grad_W1 * token_eta, the dual
 *             branch's eta_ij = token_eta_i * lr_j).  The step committed at
 *             a mini-batch boundary is that of the last position,
 *             token_eta[K-1] * sum_j lr_j k_j^T g_j.  NULL means all ones.
 *             The same values for every batch and head. */
typedef struct ttt_eta {
    const float *data;
    int64_t sB, sH;
    const float *token_eta;
} ttt_eta;

typedef struct ttt_linear_cfg {
    int32_t B, H;        /* batch, heads */
    int32_t D;           /* head_dim, must be 64 */
    int32_t K;           /* mini_batch_size, 1..16 (the MFMA dual-form path needs 16) */
    int32_t in_dtype;    /* ttt_dtype of XQ, XK, XV */
    int32_t out_dtype;   /* ttt_dtype of out */
    int32_t rope;        /* 1: rotary embedding at position mod K on q and k */
    float rope_base;     /* rotary base, e.g. 10000 */
    float ln_eps;        /* LayerNorm eps, e.g. 1e-6 */
    int32_t grad_layout; /* ttt_grad_layout of state->W_grad (0: dense) */
} ttt_linear_cfg;

/* How state->W_grad holds the open mini-batch's gradient sum
 * G = sum_j eta_j k_j^T g_j (j = 0 .. offset % K - 1, k_j after rotary):
 *   TTT_GRAD_DENSE : G itself, [D, D] per chain (the pages' cache key).
 *   TTT_GRAD_ROWS  : the rows that make it up.  Per chain the [D, D] buffer is
 *                    read as [D/2, 2D]: row j = [k_j (D values), eta_j g_j
 *                    (D values)] for j < offset % K; rows past that are
 *                    undefined.  A call reads offset % K rows and writes the
 *                    ones it adds, instead of reading and writing all of G:
 *                    ~22 KB instead of ~50 KB of state traffic per chain and
 *                    decoded token.  Outputs, W, b and b_grad are the same
 *                    function of the inputs in both layouts (up to rounding
 *                    order); G is the sum of the rows' outer products.
 * The layout is a property of the state: use one layout for all calls on a
 * state (state_init writes zeros, valid in both). */
typedef enum ttt_grad_layout {
    TTT_GRAD_DENSE = 0,
    TTT_GRAD_ROWS = 1
} ttt_grad_layout;

/* TTTCache-style carried state of TTT-Linear (all fp32, device, contiguous):
 *   W      [B, H, D, D]  mini-batch-start weights, row r = input dim
 *   b      [B, H, D]     mini-batch-start bias
 *   W_grad [B, H, D, D]  the open mini-batch's sum of eta_j k_j^T g_j, in
 *                        cfg->grad_layout
 *   b_grad [B, H, D]     sum over the open mini-batch of eta_j g_j
 *   offset (host)        tokens consumed so far (the cache's seqlen_offset);
 *                        W_grad and b_grad are zero whenever offset % K == 0
 *                        (in the rows layout no row is open then). */
typedef struct ttt_linear_state {
    float *W, *b, *W_grad, *b_grad;
    int64_t offset;
} ttt_linear_state;

/* Initial state from the layer parameters ("TTTLinear.ttt": W1, b1 tiled over
 * the batch, gradients zero).  W0 [H, D, D] and b0 [H, D] fp32 device,
 * contiguous.  Sets offset = 0. */
ttt_status ttt_linear_state_init(const ttt_linear_cfg *cfg, const float *W0, const float *b0,
                                 ttt_linear_state *state, void *stream);

/* Process L tokens of every (b, h) chain starting at state->offset.
 * ("TTTBase.forward" + "TTTLinear.ttt" + "compute_mini_batch".)
 *  XQ, XK, XV: [B, H, L, D] in cfg->in_dtype; eta as above (L per chain);
 *  ln_w, ln_b: [H, D] fp32 device, contiguous (per-head LN gamma, beta);
 *  out: [B, H, L, D] in cfg->out_dtype.
 * Tokens that complete an open mini-batch and a trailing partial mini-batch
 * run token by token (primal form); whole mini-batches run in the dual form
 * on MFMA.  On success state->offset += L. */
ttt_status ttt_linear_prefill(const ttt_linear_cfg *cfg, int32_t L, ttt_tensor XQ, ttt_tensor XK,
                              ttt_tensor XV, ttt_eta eta, const float *ln_w, const float *ln_b,
                              ttt_linear_state *state, ttt_tensor out, void *stream);

/* Same function of (state, tokens) as ttt_linear_prefill, for a few tokens
 * (typically T = 1): every token runs in the primal form ("compute_mini_batch",
 * primal branch), the step is committed when a token closes a mini-batch.
 * On success state->offset += T. */
ttt_status ttt_linear_decode(const ttt_linear_cfg *cfg, int32_t T, ttt_tensor XQ, ttt_tensor XK,
                             ttt_tensor XV, ttt_eta eta, const float *ln_w, const float *ln_b,
                             ttt_linear_state *state, ttt_tensor out, void *stream);

typedef struct ttt_mlp_cfg {
    int32_t B, H;
    int32_t D;           /* 64 */
    int32_t F;           /* hidden width of the inner MLP, 256 */
    int32_t K;           /* mini-batch size 1..16 (16 runs whole mini-batches on MFMA) */
    int32_t in_dtype, out_dtype;
    int32_t rope;
    float rope_base;
    float ln_eps;
    int32_t grad_layout; /* ttt_grad_layout of the *_grad state (0: dense) */
} ttt_mlp_cfg;

/* Carried state of TTT-MLP (fp32, device, contiguous):
 *   W1 [B, H, D, F], b1 [B, H, F], W2 [B, H, F, D], b2 [B, H, D],
 *   W1_grad, b1_grad, W2_grad, b2_grad of the same shapes (open mini-batch),
 *   offset (host).
 * The open mini-batch's gradient sums are G1 = sum_j k_j^T (eta_j g1_j) and
 * G2 = sum_j x2_j^T (eta_j g2_j) (x2_j = GELU(k_j W1 + b1) at the mini-batch
 * start).  In TTT_GRAD_DENSE, W1_grad and W2_grad hold G1 and G2.  In
 * TTT_GRAD_ROWS they hold the rows that make them up: per chain W1_grad is
 * read as [D*F / (D+F), D+F] with row j = [k_j (D) | eta_j g1_j (F)], and
 * W2_grad as rows [x2_j (F) | eta_j g2_j (D)], for j < offset % K (rows past
 * that are undefined).  b1_grad, b2_grad are dense in both layouts.  The
 * rows layout keeps a decode call's state traffic at W1, W2 plus ~2.5 KB per
 * open token instead of W1, W2 and both dense gradients read and written. */
typedef struct ttt_mlp_state {
    float *W1, *b1, *W2, *b2;
    float *W1_grad, *b1_grad, *W2_grad, *b2_grad;
    int64_t offset;
} ttt_mlp_state;

/* Initial state from the layer parameters.  The pages give only the linear
 * layer's initial state ("TTTLinear.ttt": W1, b1 tiled over the batch) and
 * describe TTT-MLP as two such layers stacked ("代码连连看——TTT", the remark
 * after compute_mini_batch); this call applies the same tiling to all four
 * parameters.  W1 [H, D, F], b1 [H, F], W2 [H, F, D], b2 [H, D] fp32 device,
 * contiguous.  Tiles them over the batch, zeroes the gradients, sets
 * offset = 0. */
ttt_status ttt_mlp_state_init(const ttt_mlp_cfg *cfg, const float *W1, const float *b1, const float *W2,
                              const float *b2, ttt_mlp_state *state, void *stream);

/* TTT-MLP over L tokens, continuing from the state at any offset (the
 * TTT-Linear step applied to both layers of the inner MLP: "代码连连看——TTT",
 * closing remark).  With K = 16 and bf16 inputs, tokens that complete an open
 * mini-batch run one at a time (primal form), whole mini-batches in the dual
 * form on MFMA (fp16 operands, fp32 accumulation); a trailing partial
 * mini-batch is computed with its outputs and left open: the parameters stay
 * at the mini-batch start and the *_grad arrays hold its accumulated
 * eta-weighted gradients.  fp32 inputs and K != 16 run every token in the
 * primal form (fp32 arithmetic).  On success state->offset += L. */
ttt_status ttt_mlp_prefill(const ttt_mlp_cfg *cfg, int32_t L, ttt_tensor XQ, ttt_tensor XK, ttt_tensor XV,
                           ttt_eta eta, const float *ln_w, const float *ln_b, ttt_mlp_state *state,
                           ttt_tensor out, void *stream);

/* TTT-MLP decode: T tokens (typically 1) one at a time in the primal form
 * (compute_mini_batch, primal branch, on both layers; fp32 arithmetic); the
 * step is committed when a token closes a mini-batch.  Same arguments and
 * errors as ttt_mlp_prefill.  On success state->offset += T. */
ttt_status ttt_mlp_decode(const ttt_mlp_cfg *cfg, int32_t T, ttt_tensor XQ, ttt_tensor XK, ttt_tensor XV,
                          ttt_eta eta, const float *ln_w, const float *ln_b, ttt_mlp_state *state,
                          ttt_tensor out, void *stream);

/* ---- Post-norm and output projection: the steps after the layer ----
 *
 * "代码连连看——TTT", TTTBase.forward: after the scan the heads' outputs are
 * concatenated to [B, L, width] (width = H * D), then go through post_norm, a
 * LayerNorm over the width, and o_proj, a linear map.  With y that output as
 * M = B * L rows of K = width values (the prefill's out written with
 * sB = L*H*D, sH = D, sL = H*D is this layout) and Wo [K, N]:
 *   out[m, :] = ((y[m, :] - mean_m) / sqrt(var_m + eps) * gamma + beta) Wo + bias
 * (var_m the population variance of row m).  The pages do not show the
 * constructors of post_norm and o_proj; bias may be NULL (none).
 *
 * Arithmetic: bf16 operands, fp32 accumulation.  The weights enter as
 * W' = bf16(diag(gamma) Wo) with c1 = column sums of W' and
 * c2 = beta^T Wo + bias, and out = r (y W') - r mean c1 + c2 per row, which is
 * the LayerNorm followed by the product with W'.  The row statistics are
 * sums over the bf16 values of y in fp32 (mean of squares minus squared mean:
 * rows whose mean is many standard deviations from zero lose precision).
 *
 * ttt_post_proj_prepared_bytes(K, N): size of the prepared-weights buffer,
 * K * N * 2 + N * 8 bytes (0 for K or N <= 0).
 *
 * ttt_post_proj_prepare: forms the prepared weights from gamma, beta [K],
 * Wo [K, N] row-major and bias [N] (or NULL), fp32 device arrays, into
 * `prepared` (device, 16-byte aligned, caller-owned, prepared_bytes long),
 * enqueued on `stream`; done once per weight set.  K must be a positive
 * multiple of 64 and N of 256 (TTT_ERR_SHAPE); NULL pointers give
 * TTT_ERR_NULL; `prepared` overlapping an input gives TTT_ERR_ALIAS.
 *
 * ttt_post_proj: y [M, K] bf16 device rows of stride ldy elements (ldy >= K,
 * a multiple of 8; y 16-byte aligned), `prepared` from ttt_post_proj_prepare
 * with the same K, N, out [M, N] device rows of stride ldo (>= N; out
 * 16-byte aligned and ldo a multiple of 16 bytes) in out_dtype (TTT_F32 or
 * TTT_BF16), eps > 0.  Enqueued on `stream`; reads y
 * and prepared, writes out only.  Errors as above, plus TTT_ERR_DTYPE for
 * out_dtype, TTT_ERR_ALIGN for y / prepared / out alignment, TTT_ERR_ALIAS
 * when out overlaps y or prepared, TTT_ERR_HIP when a launch fails. */
size_t ttt_post_proj_prepared_bytes(int32_t K, int32_t N);
ttt_status ttt_post_proj_prepare(int32_t K, int32_t N, const float *gamma, const float *beta, const float *Wo,
                                 const float *bias, void *prepared, void *stream);
ttt_status ttt_post_proj(int32_t M, int32_t K, int32_t N, const void *y, int64_t ldy, float eps,
                         const void *prepared, void *out, int64_t ldo, int32_t out_dtype, void *stream);

const char *ttt_status_string(ttt_status s);
const char *ttt_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* TTT_H */
