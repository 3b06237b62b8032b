/*
 * ttt_oracle.c -- plain, slow CPU reference of the TTT layer hot path.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the CPU
 * baseline leg of the benchmark may load this library.  The product path
 * (libttt and its kernels) never links, includes or calls it, and shares no
 * code, header, table or helper with it.
 *
 * Arithmetic is IEEE double throughout.  Inputs arrive as doubles holding the
 * exact values the GPU reads (bf16 or fp32 numbers widened without rounding).
 *
 * Sources (web pages, cited by title and listing/section):
 *   [P1] ttt-lm-pytorch README, German machine translation (downcodes.com)
 *   [P2] "测试时学习（TTT）原理解析：ttt-lm-pytorch如何让模型在推理时持续学习"
 *        (nanhubrain.csdn.net): sections "TTT的核心创新" (TTTLinear init),
 *        "TTT缓存机制" (TTTCache)
 *   [P3] "代码连连看——TTT" (jiafeimiao.top): listings TTTBase.forward,
 *        TTTLinear.ttt and compute_mini_batch (dual and primal branches)
 *
 * What is computed.  Each (batch, head) pair is an independent chain whose
 * hidden state is a small model f (linear: z = x W + b; MLP:
 * z = GELU(x W1 + b1) W2 + b2).  Tokens are grouped in mini-batches of K
 * aligned at absolute positions that are multiples of K.  Every token j of a
 * mini-batch contributes the loss  l_j = 1/2 || LN(f(k_j)) - (v_j - k_j) ||^2
 * evaluated at the mini-batch-start parameters; the prediction for token i
 * uses the parameters after one gradient step on the losses of tokens
 * j <= i of its mini-batch, each scaled by that token's learning rate eta_j,
 * and the output is  q_i + LN(f_i(q_i)).  At a mini-batch boundary the step
 * over the whole mini-batch is committed.  [P3 compute_mini_batch, primal
 * branch; P3 TTTLinear.ttt, NOTE on dual/primal]
 *
 * The main routines follow the primal form token by token.  A dual-form
 * routine (whole mini-batches, in the order of the pages' dual branch) is
 * kept only so the tests can check the two formulations against each other.
 *
 * Readings where the pages are silent (each is listed in the design notes):
 *   - loss is 1/2 ||r||^2 (no factor 2 in the gradient);
 *   - LayerNorm uses the population variance and eps inside the square root,
 *     for both the forward and the fused backward (bodies not on the pages);
 *   - eta_ij = token_eta_i * lr_j: lr_j is the learning rate of key token j
 *     ("ttt_lr_eta"), token_eta_i the scale of output row i within its
 *     mini-batch ("token_eta"; te == NULL means all ones); the step committed
 *     at a boundary uses the last row, token_eta_{K-1}; the diagonal of the
 *     causal mask is included;
 *   - rotary embedding is rotate-half (pairs i, i + D/2), angle
 *     p * base^(-2i/D) with p = absolute position mod K, applied to q and k
 *     before everything else (target and residual use the rotated values);
 *   - mid-mini-batch state keeps the mini-batch-start W, b and the
 *     accumulated eta-weighted gradients; they are committed and zeroed at
 *     the boundary (TTTCache body not on the pages);
 *   - TTT-MLP: f(x) = GELU(x W1 + b1) W2 + b2 with the exact erf GELU.
 *
 * Parity pins: see tests/test_oracle_pins.py.  Every routine here is pinned
 * by at least one check that does not re-type its formula.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* ---------------------------------------------------------------------- */
/* LayerNorm pieces (bodies of ln_fwd / ln_fused_l2_bwd are not printed;   */
/* named in [P3 compute_mini_batch]).                                      */
/* ---------------------------------------------------------------------- */

/* mean and sqrt(population variance + eps) of one row of length D */
static void ln_stats(const double *z, int D, double eps, double *mu, double *s)
{
    double m = 0.0;
    for (int c = 0; c < D; ++c) m += z[c];
    m /= D;
    double var = 0.0;
    for (int c = 0; c < D; ++c) var += (z[c] - m) * (z[c] - m);
    var /= D;
    *mu = m;
    *s = sqrt(var + eps);
}

/* y = gamma * (z - mu) / s + beta   [P3 compute_mini_batch: ln_fwd] */
void oracle_ln_fwd(const double *z, const double *gamma, const double *beta,
                   int D, double eps, double *y)
{
    double mu, s;
    ln_stats(z, D, eps, &mu, &s);
    for (int c = 0; c < D; ++c) y[c] = gamma[c] * ((z[c] - mu) / s) + beta[c];
}

/* Gradient w.r.t. z of 1/2 || LN(z) - target ||^2.
 * [P3 compute_mini_batch: ln_fused_l2_bwd(Z1, reconstruction_target, ...)]
 * With xh = (z - mu)/s and u = gamma * (LN(z) - target), the chain rule
 * through the normalisation gives g = (u - mean(u) - xh * mean(u * xh)) / s. */
void oracle_ln_l2_grad(const double *z, const double *target,
                       const double *gamma, const double *beta, int D,
                       double eps, double *g)
{
    double mu, s;
    ln_stats(z, D, eps, &mu, &s);
    double mean_u = 0.0, mean_uxh = 0.0;
    for (int c = 0; c < D; ++c) {
        double xh = (z[c] - mu) / s;
        double u = gamma[c] * (gamma[c] * xh + beta[c] - target[c]);
        mean_u += u;
        mean_uxh += u * xh;
    }
    mean_u /= D;
    mean_uxh /= D;
    for (int c = 0; c < D; ++c) {
        double xh = (z[c] - mu) / s;
        double u = gamma[c] * (gamma[c] * xh + beta[c] - target[c]);
        g[c] = (u - mean_u - xh * mean_uxh) / s;
    }
}

/* Rotary embedding of one row at integer position p (rotate-half pairing).
 * [P3 TTTBase.forward: rotary_emb at position_ids % mini_batch_size] */
void oracle_rope_row(const double *x, int D, int64_t p, double base, double *y)
{
    int h = D / 2;
    for (int i = 0; i < h; ++i) {
        double theta = (double)p * pow(base, -2.0 * (double)i / (double)D);
        double c = cos(theta), s = sin(theta);
        double a = x[i], bb = x[i + h];
        y[i] = a * c - bb * s;
        y[i + h] = bb * c + a * s;
    }
}

/* exact GELU and its derivative (reading for TTT-MLP; [P1], [P3] say only
 * "two-layer MLP" / "TTTLinear stacked twice") */
double oracle_gelu(double x) { return 0.5 * x * (1.0 + erf(x / sqrt(2.0))); }
double oracle_gelu_grad(double x)
{
    double cdf = 0.5 * (1.0 + erf(x / sqrt(2.0)));
    double pdf = exp(-0.5 * x * x) / sqrt(2.0 * M_PI);
    return cdf + x * pdf;
}

static void maybe_rope(const double *x, int D, int rope, int64_t pos, int K,
                       double base, double *y)
{
    if (rope)
        oracle_rope_row(x, D, pos % K, base, y);
    else
        memcpy(y, x, sizeof(double) * (size_t)D);
}

/* ---------------------------------------------------------------------- */
/* TTT-Linear, primal form, one chain.                                    */
/* [P3 compute_mini_batch, primal branch; P3 TTTLinear.ttt; P2 TTTCache]   */
/*                                                                        */
/* q, k, v, out: L rows of D, row stride ld (elements).                   */
/* eta: L values with stride eta_st (the learning rate of each token).   */
/* te: K values, token_eta by position in the mini-batch (NULL = ones).   */
/* W: D x D row-major, W[r*D + c] maps input dim r to output dim c        */
/*    (row vector times W, as in "X1 @ W1_init").                         */
/* b: D.  G, gb: accumulated eta-weighted gradients of the open           */
/* mini-batch (the pages' W1_grad, b1_grad).  offset: absolute position   */
/* of the first token.  All of W, b, G, gb are updated in place.          */
/* ---------------------------------------------------------------------- */
void oracle_linear_chain(int D, int K, int L, int64_t offset,
                         const double *q, const double *k, const double *v,
                         int64_t ld, const double *eta, int64_t eta_st,
                         const double *te, const double *gamma,
                         const double *beta, int rope, double rope_base,
                         double eps, double *W, double *b, double *G,
                         double *gb, double *out, int64_t ld_out)
{
    double *qr = malloc(sizeof(double) * D), *kr = malloc(sizeof(double) * D);
    double *z = malloc(sizeof(double) * D), *tgt = malloc(sizeof(double) * D);
    double *g = malloc(sizeof(double) * D), *zb = malloc(sizeof(double) * D);
    double *y = malloc(sizeof(double) * D);
    for (int t = 0; t < L; ++t) {
        int64_t pos = offset + t;
        const double *qt = q + (int64_t)t * ld, *kt = k + (int64_t)t * ld;
        const double *vt = v + (int64_t)t * ld;
        double e = eta[(int64_t)t * eta_st];
        maybe_rope(qt, D, rope, pos, K, rope_base, qr);
        maybe_rope(kt, D, rope, pos, K, rope_base, kr);
        /* Z1 = X1 @ W1_init + b1_init at the mini-batch-start state */
        for (int c = 0; c < D; ++c) {
            double acc = b[c];
            for (int r = 0; r < D; ++r) acc += kr[r] * W[r * D + c];
            z[c] = acc;
        }
        /* reconstruction_target = XV - XK */
        for (int c = 0; c < D; ++c) tgt[c] = vt[c] - kr[c];
        oracle_ln_l2_grad(z, tgt, gamma, beta, D, eps, g);
        /* grad_W1 += lr_t * x_t (x) g_t ; grad_b1 += lr_t * g_t */
        for (int r = 0; r < D; ++r)
            for (int c = 0; c < D; ++c) G[r * D + c] += e * kr[r] * g[c];
        for (int c = 0; c < D; ++c) gb[c] += e * g[c];
        /* W1_bar = W1_init - token_eta * grad_W1 ; Z1_bar = XQ @ W1_bar + b1_bar */
        double tp = te ? te[pos % K] : 1.0;
        for (int c = 0; c < D; ++c) {
            double acc = b[c] - tp * gb[c];
            for (int r = 0; r < D; ++r) acc += qr[r] * (W[r * D + c] - tp * G[r * D + c]);
            zb[c] = acc;
        }
        /* XQW = XQ + ln_fwd(Z1_bar) */
        oracle_ln_fwd(zb, gamma, beta, D, eps, y);
        double *ot = out + (int64_t)t * ld_out;
        for (int c = 0; c < D; ++c) ot[c] = qr[c] + y[c];
        /* mini-batch boundary: commit the step of the last row (W1_last =
         * W1_bar of token K-1), clear the gradients */
        if ((pos + 1) % K == 0) {
            for (int i = 0; i < D * D; ++i) { W[i] -= tp * G[i]; G[i] = 0.0; }
            for (int c = 0; c < D; ++c) { b[c] -= tp * gb[c]; gb[c] = 0.0; }
        }
    }
    free(qr); free(kr); free(z); free(tgt); free(g); free(zb); free(y);
}

/* ---------------------------------------------------------------------- */
/* TTT-Linear, dual form, one chain, whole aligned mini-batches only.     */
/* Self-check of the primal routine.  Steps in the order of              */
/* [P3 compute_mini_batch, dual branch].  Requires offset % K == 0 and    */
/* L % K == 0 and G = gb = 0; returns -1 otherwise.                       */
/* ---------------------------------------------------------------------- */
int oracle_linear_chain_dual(int D, int K, int L, int64_t offset,
                             const double *q, const double *k, const double *v,
                             int64_t ld, const double *eta, int64_t eta_st,
                             const double *te, const double *gamma,
                             const double *beta, int rope, double rope_base,
                             double eps, double *W, double *b, double *out,
                             int64_t ld_out)
{
    if (offset % K != 0 || L % K != 0) return -1;
    size_t KD = (size_t)K * D;
    double *XQ = malloc(sizeof(double) * KD), *X1 = malloc(sizeof(double) * KD);
    double *Z1 = malloc(sizeof(double) * KD), *tgt = malloc(sizeof(double) * D);
    double *gZ = malloc(sizeof(double) * KD), *Zb = malloc(sizeof(double) * KD);
    double *Attn = malloc(sizeof(double) * K * K), *y = malloc(sizeof(double) * D);
    double *E = malloc(sizeof(double) * K * K);
    for (int n = 0; n < L / K; ++n) {
        for (int i = 0; i < K; ++i) {
            int t = n * K + i;
            maybe_rope(q + (int64_t)t * ld, D, rope, offset + t, K, rope_base, XQ + (size_t)i * D);
            maybe_rope(k + (int64_t)t * ld, D, rope, offset + t, K, rope_base, X1 + (size_t)i * D);
        }
        /* the [K, K] eta of the block: E_ij = token_eta_i * lr_j */
        for (int i = 0; i < K; ++i)
            for (int j = 0; j < K; ++j)
                E[i * K + j] = (te ? te[i] : 1.0) * eta[(int64_t)(n * K + j) * eta_st];
        /* Z1 = X1 @ W1_init + b1_init ; target = XV - XK ; grad */
        for (int i = 0; i < K; ++i) {
            for (int c = 0; c < D; ++c) {
                double acc = b[c];
                for (int r = 0; r < D; ++r) acc += X1[i * D + r] * W[r * D + c];
                Z1[i * D + c] = acc;
            }
            const double *vt = v + (int64_t)(n * K + i) * ld;
            for (int c = 0; c < D; ++c) tgt[c] = vt[c] - X1[i * D + c];
            oracle_ln_l2_grad(Z1 + i * D, tgt, gamma, beta, D, eps, gZ + i * D);
        }
        /* Attn1 = tril(XQ @ X1^T) */
        for (int i = 0; i < K; ++i)
            for (int j = 0; j < K; ++j) {
                double acc = 0.0;
                if (j <= i)
                    for (int r = 0; r < D; ++r) acc += XQ[i * D + r] * X1[j * D + r];
                Attn[i * K + j] = acc;
            }
        /* b1_bar = b1_init - tril(eta) @ grad ;
         * Z1_bar = XQ @ W1_init - (eta * Attn1) @ grad + b1_bar */
        for (int i = 0; i < K; ++i)
            for (int c = 0; c < D; ++c) {
                double bbar = b[c];
                for (int j = 0; j <= i; ++j) bbar -= E[i * K + j] * gZ[j * D + c];
                double acc = 0.0;
                for (int r = 0; r < D; ++r) acc += XQ[i * D + r] * W[r * D + c];
                for (int j = 0; j <= i; ++j) acc -= E[i * K + j] * Attn[i * K + j] * gZ[j * D + c];
                Zb[i * D + c] = acc + bbar;
            }
        /* XQW = XQ + ln_fwd(Z1_bar) */
        for (int i = 0; i < K; ++i) {
            oracle_ln_fwd(Zb + i * D, gamma, beta, D, eps, y);
            double *ot = out + (int64_t)(n * K + i) * ld_out;
            for (int c = 0; c < D; ++c) ot[c] = XQ[i * D + c] + y[c];
        }
        /* W1_last = W1_init - (last_eta * X1)^T @ grad ;
         * b1_last = b1_init - sum(last_eta * grad), last_eta = row K-1 of eta */
        const double *le = E + (size_t)(K - 1) * K;
        for (int r = 0; r < D; ++r)
            for (int c = 0; c < D; ++c) {
                double acc = 0.0;
                for (int j = 0; j < K; ++j) acc += le[j] * X1[j * D + r] * gZ[j * D + c];
                W[r * D + c] -= acc;
            }
        for (int c = 0; c < D; ++c) {
            double acc = 0.0;
            for (int j = 0; j < K; ++j) acc += le[j] * gZ[j * D + c];
            b[c] -= acc;
        }
    }
    free(XQ); free(X1); free(Z1); free(tgt); free(gZ); free(Zb); free(Attn);
    free(y); free(E);
    return 0;
}

/* ---------------------------------------------------------------------- */
/* TTT-MLP, primal form, one chain.  f(x) = GELU(x W1 + b1) W2 + b2.      */
/* Gradients at the mini-batch-start parameters, accumulated with each    */
/* token's learning rate; the prediction for token i uses the parameters  */
/* minus the accumulated gradients; commit at the boundary.  Same scheme  */
/* as the linear routine with f the two-layer MLP.  [P1 intro; P2 "TTT的   */
/* 核心创新"; P3 closing remark: TTT-MLP is TTT-Linear stacked twice]       */
/* W1: D x F, b1: F, W2: F x D, b2: D, row-major; G1.. the accumulators.  */
/* ---------------------------------------------------------------------- */
void oracle_mlp_chain(int D, int F, int K, int L, int64_t offset,
                      const double *q, const double *k, const double *v,
                      int64_t ld, const double *eta, int64_t eta_st,
                      const double *te, const double *gamma,
                      const double *beta, int rope, double rope_base,
                      double eps, double *W1, double *b1, double *W2,
                      double *b2, double *G1, double *gb1, double *G2,
                      double *gb2, double *out, int64_t ld_out)
{
    double *qr = malloc(sizeof(double) * D), *kr = malloc(sizeof(double) * D);
    double *z1 = malloc(sizeof(double) * F), *x2 = malloc(sizeof(double) * F);
    double *z2 = malloc(sizeof(double) * D), *tgt = malloc(sizeof(double) * D);
    double *g2 = malloc(sizeof(double) * D), *g1 = malloc(sizeof(double) * F);
    double *zb1 = malloc(sizeof(double) * F), *xb2 = malloc(sizeof(double) * F);
    double *zb2 = malloc(sizeof(double) * D), *y = malloc(sizeof(double) * D);
    for (int t = 0; t < L; ++t) {
        int64_t pos = offset + t;
        const double *vt = v + (int64_t)t * ld;
        double e = eta[(int64_t)t * eta_st];
        maybe_rope(q + (int64_t)t * ld, D, rope, pos, K, rope_base, qr);
        maybe_rope(k + (int64_t)t * ld, D, rope, pos, K, rope_base, kr);
        /* forward of the inner model at the mini-batch-start parameters */
        for (int f = 0; f < F; ++f) {
            double acc = b1[f];
            for (int r = 0; r < D; ++r) acc += kr[r] * W1[r * F + f];
            z1[f] = acc;
            x2[f] = oracle_gelu(acc);
        }
        for (int c = 0; c < D; ++c) {
            double acc = b2[c];
            for (int f = 0; f < F; ++f) acc += x2[f] * W2[f * D + c];
            z2[c] = acc;
        }
        for (int c = 0; c < D; ++c) tgt[c] = vt[c] - kr[c];
        oracle_ln_l2_grad(z2, tgt, gamma, beta, D, eps, g2);
        /* backward into the first layer */
        for (int f = 0; f < F; ++f) {
            double acc = 0.0;
            for (int c = 0; c < D; ++c) acc += g2[c] * W2[f * D + c];
            g1[f] = acc * oracle_gelu_grad(z1[f]);
        }
        for (int r = 0; r < D; ++r)
            for (int f = 0; f < F; ++f) G1[r * F + f] += e * kr[r] * g1[f];
        for (int f = 0; f < F; ++f) gb1[f] += e * g1[f];
        for (int f = 0; f < F; ++f)
            for (int c = 0; c < D; ++c) G2[f * D + c] += e * x2[f] * g2[c];
        for (int c = 0; c < D; ++c) gb2[c] += e * g2[c];
        /* prediction with the stepped parameters (step scaled by token_eta) */
        double tp = te ? te[pos % K] : 1.0;
        for (int f = 0; f < F; ++f) {
            double acc = b1[f] - tp * gb1[f];
            for (int r = 0; r < D; ++r) acc += qr[r] * (W1[r * F + f] - tp * G1[r * F + f]);
            zb1[f] = acc;
            xb2[f] = oracle_gelu(acc);
        }
        for (int c = 0; c < D; ++c) {
            double acc = b2[c] - tp * gb2[c];
            for (int f = 0; f < F; ++f) acc += xb2[f] * (W2[f * D + c] - tp * G2[f * D + c]);
            zb2[c] = acc;
        }
        oracle_ln_fwd(zb2, gamma, beta, D, eps, y);
        double *ot = out + (int64_t)t * ld_out;
        for (int c = 0; c < D; ++c) ot[c] = qr[c] + y[c];
        if ((pos + 1) % K == 0) {
            for (int i = 0; i < D * F; ++i) { W1[i] -= tp * G1[i]; G1[i] = 0.0; }
            for (int i = 0; i < F * D; ++i) { W2[i] -= tp * G2[i]; G2[i] = 0.0; }
            for (int f = 0; f < F; ++f) { b1[f] -= tp * gb1[f]; gb1[f] = 0.0; }
            for (int c = 0; c < D; ++c) { b2[c] -= tp * gb2[c]; gb2[c] = 0.0; }
        }
    }
    free(qr); free(kr); free(z1); free(x2); free(z2); free(tgt); free(g2);
    free(g1); free(zb1); free(xb2); free(zb2); free(y);
}

/* ---------------------------------------------------------------------- */
/* TTT-MLP, dual form, whole aligned mini-batches (self-check only).      */
/* The dual identity of the linear layer applied to each layer of f:      */
/* Z1_bar = XQ W1 + b1 - tril(eta * (XQ X1^T + 1)) g1, X2_bar = GELU(.),  */
/* Z2_bar = X2_bar W2 + b2 - tril(eta * (X2_bar X2^T + 1)) g2.            */
/* ---------------------------------------------------------------------- */
int oracle_mlp_chain_dual(int D, int F, int K, int L, int64_t offset,
                          const double *q, const double *k, const double *v,
                          int64_t ld, const double *eta, int64_t eta_st,
                          const double *te, const double *gamma,
                          const double *beta, int rope, double rope_base,
                          double eps, double *W1, double *b1, double *W2,
                          double *b2, double *out, int64_t ld_out)
{
    if (offset % K != 0 || L % K != 0) return -1;
    double *XQ = malloc(sizeof(double) * K * D), *X1 = malloc(sizeof(double) * K * D);
    double *Z1 = malloc(sizeof(double) * K * F), *X2 = malloc(sizeof(double) * K * F);
    double *Z2 = malloc(sizeof(double) * K * D), *tgt = malloc(sizeof(double) * D);
    double *g2 = malloc(sizeof(double) * K * D), *g1 = malloc(sizeof(double) * K * F);
    double *Zb1 = malloc(sizeof(double) * K * F), *Xb2 = malloc(sizeof(double) * K * F);
    double *Zb2 = malloc(sizeof(double) * K * D), *y = malloc(sizeof(double) * D);
    double *E = malloc(sizeof(double) * K * K);
    for (int n = 0; n < L / K; ++n) {
        for (int i = 0; i < K; ++i) {
            int t = n * K + i;
            maybe_rope(q + (int64_t)t * ld, D, rope, offset + t, K, rope_base, XQ + i * D);
            maybe_rope(k + (int64_t)t * ld, D, rope, offset + t, K, rope_base, X1 + i * D);
        }
        /* E_ij = token_eta_i * lr_j, as for the linear layer */
        for (int i = 0; i < K; ++i)
            for (int j = 0; j < K; ++j)
                E[i * K + j] = (te ? te[i] : 1.0) * eta[(int64_t)(n * K + j) * eta_st];
        for (int i = 0; i < K; ++i) {
            for (int f = 0; f < F; ++f) {
                double acc = b1[f];
                for (int r = 0; r < D; ++r) acc += X1[i * D + r] * W1[r * F + f];
                Z1[i * F + f] = acc;
                X2[i * F + f] = oracle_gelu(acc);
            }
            for (int c = 0; c < D; ++c) {
                double acc = b2[c];
                for (int f = 0; f < F; ++f) acc += X2[i * F + f] * W2[f * D + c];
                Z2[i * D + c] = acc;
            }
            const double *vt = v + (int64_t)(n * K + i) * ld;
            for (int c = 0; c < D; ++c) tgt[c] = vt[c] - X1[i * D + c];
            oracle_ln_l2_grad(Z2 + i * D, tgt, gamma, beta, D, eps, g2 + i * D);
            for (int f = 0; f < F; ++f) {
                double acc = 0.0;
                for (int c = 0; c < D; ++c) acc += g2[i * D + c] * W2[f * D + c];
                g1[i * F + f] = acc * oracle_gelu_grad(Z1[i * F + f]);
            }
        }
        /* first layer of the prediction */
        for (int i = 0; i < K; ++i)
            for (int f = 0; f < F; ++f) {
                double acc = b1[f];
                for (int r = 0; r < D; ++r) acc += XQ[i * D + r] * W1[r * F + f];
                for (int j = 0; j <= i; ++j) {
                    double a = 1.0;
                    for (int r = 0; r < D; ++r) a += XQ[i * D + r] * X1[j * D + r];
                    acc -= E[i * K + j] * a * g1[j * F + f];
                }
                Zb1[i * F + f] = acc;
                Xb2[i * F + f] = oracle_gelu(acc);
            }
        /* second layer of the prediction */
        for (int i = 0; i < K; ++i)
            for (int c = 0; c < D; ++c) {
                double acc = b2[c];
                for (int f = 0; f < F; ++f) acc += Xb2[i * F + f] * W2[f * D + c];
                for (int j = 0; j <= i; ++j) {
                    double a = 1.0;
                    for (int f = 0; f < F; ++f) a += Xb2[i * F + f] * X2[j * F + f];
                    acc -= E[i * K + j] * a * g2[j * D + c];
                }
                Zb2[i * D + c] = acc;
            }
        for (int i = 0; i < K; ++i) {
            oracle_ln_fwd(Zb2 + i * D, gamma, beta, D, eps, y);
            double *ot = out + (int64_t)(n * K + i) * ld_out;
            for (int c = 0; c < D; ++c) ot[c] = XQ[i * D + c] + y[c];
        }
        /* step over the whole mini-batch, with the last row of eta */
        const double *le = E + (size_t)(K - 1) * K;
        for (int r = 0; r < D; ++r)
            for (int f = 0; f < F; ++f) {
                double acc = 0.0;
                for (int j = 0; j < K; ++j) acc += le[j] * X1[j * D + r] * g1[j * F + f];
                W1[r * F + f] -= acc;
            }
        for (int f = 0; f < F; ++f) {
            double acc = 0.0;
            for (int j = 0; j < K; ++j) acc += le[j] * g1[j * F + f];
            b1[f] -= acc;
        }
        for (int f = 0; f < F; ++f)
            for (int c = 0; c < D; ++c) {
                double acc = 0.0;
                for (int j = 0; j < K; ++j) acc += le[j] * X2[j * F + f] * g2[j * D + c];
                W2[f * D + c] -= acc;
            }
        for (int c = 0; c < D; ++c) {
            double acc = 0.0;
            for (int j = 0; j < K; ++j) acc += le[j] * g2[j * D + c];
            b2[c] -= acc;
        }
    }
    free(XQ); free(X1); free(Z1); free(X2); free(Z2); free(tgt); free(g2);
    free(g1); free(Zb1); free(Xb2); free(Zb2); free(y); free(E);
    return 0;
}

/* ---------------------------------------------------------------------- */
/* Batched drivers: independent (b, h) chains, OpenMP over chains.        */
/* Inputs [B, H, L, D] contiguous; eta [B, H, L] with batch stride        */
/* eta_sB (0 = shared over the batch); te [K] or NULL; ln params [H, D]; */
/* state arrays                                                           */
/* [B, H, ...] contiguous; out [B, H, L, D].  W0 tiling over the batch    */
/* is done by the caller ([P3 TTTLinear.ttt: torch.tile of W1, b1]).      */
/* ---------------------------------------------------------------------- */
void oracle_linear_batch(int B, int H, int D, int K, int L, int64_t offset,
                         const double *XQ, const double *XK, const double *XV,
                         const double *eta, int64_t eta_sB, const double *te,
                         const double *ln_w, const double *ln_b, int rope,
                         double rope_base, double eps, double *W, double *b,
                         double *G, double *gb, double *out)
{
    int64_t n = (int64_t)B * H;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t ch = 0; ch < n; ++ch) {
        int64_t bi = ch / H, hi = ch % H;
        int64_t xo = ch * (int64_t)L * D;
        oracle_linear_chain(D, K, L, offset, XQ + xo, XK + xo, XV + xo, D,
                            eta + bi * eta_sB + hi * (int64_t)L, 1, te,
                            ln_w + hi * D, ln_b + hi * D, rope, rope_base, eps,
                            W + ch * D * D, b + ch * D, G + ch * D * D,
                            gb + ch * D, out + xo, D);
    }
}

void oracle_mlp_batch(int B, int H, int D, int F, int K, int L, int64_t offset,
                      const double *XQ, const double *XK, const double *XV,
                      const double *eta, int64_t eta_sB, const double *te,
                      const double *ln_w, const double *ln_b, int rope,
                      double rope_base,
                      double eps, double *W1, double *b1, double *W2,
                      double *b2, double *G1, double *gb1, double *G2,
                      double *gb2, double *out)
{
    int64_t n = (int64_t)B * H;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t ch = 0; ch < n; ++ch) {
        int64_t bi = ch / H, hi = ch % H;
        int64_t xo = ch * (int64_t)L * D;
        oracle_mlp_chain(D, F, K, L, offset, XQ + xo, XK + xo, XV + xo, D,
                         eta + bi * eta_sB + hi * (int64_t)L, 1, te,
                         ln_w + hi * D, ln_b + hi * D, rope, rope_base, eps,
                         W1 + ch * D * F, b1 + ch * F, W2 + ch * F * D,
                         b2 + ch * D, G1 + ch * D * F, gb1 + ch * F,
                         G2 + ch * F * D, gb2 + ch * D, out + xo, D);
    }
}

/* ---------------------------------------------------------------------- */
/* Post-norm and output projection of the layer output.  [P3 TTTBase.forward:
 * after the scan the heads' outputs are concatenated to [B, L, width]
 * (width = heads x head_dim), then post_norm, a LayerNorm over the width,
 * then o_proj, a linear map.]  The LayerNorm is the one of ln_fwd above
 * (population variance, eps inside the square root).  The pages show
 * neither module's constructor: o_proj is read as a plain matrix Wo
 * [K, N] with an optional bias (NULL for none).
 * y [M, K] (rows = tokens), gamma, beta [K], Wo [K, N], out [M, N].
 * Rows are independent: a caller may pass any subset of rows.           */
/* ---------------------------------------------------------------------- */
void oracle_post_proj(int64_t M, int K, int N, const double *y,
                      const double *gamma, const double *beta, double eps,
                      const double *Wo, const double *bias, double *out)
{
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; ++m) {
        double *x = (double *)malloc((size_t)K * sizeof(double));
        oracle_ln_fwd(y + m * K, gamma, beta, K, eps, x);
        for (int n = 0; n < N; ++n) {
            double acc = bias ? bias[n] : 0.0;
            for (int k = 0; k < K; ++k) acc += x[k] * Wo[(int64_t)k * N + n];
            out[m * N + n] = acc;
        }
        free(x);
    }
}

int oracle_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Thread count of the batch drivers' parallel loops from now on (n >= 1). */
void oracle_set_threads(int n)
{
#ifdef _OPENMP
    if (n >= 1) omp_set_num_threads(n);
#else
    (void)n;
#endif
}
