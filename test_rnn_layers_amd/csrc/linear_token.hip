// linear_token.hip -- TTT-Linear one token at a time (primal form) and the
// state initialisation kernels.
//
// Primal form of "代码连连看——TTT", compute_mini_batch, primal branch: for
// each token the gradient of its LN + L2 reconstruction loss is taken at the
// mini-batch-start W, b; the eta-weighted gradients accumulate into W_grad,
// b_grad (the pages' carried "W1_grad", "b1_grad"); the prediction of the
// token at position p of its mini-batch uses W - token_eta_p W_grad,
// b - token_eta_p b_grad ("W1_bar"); at a mini-batch boundary the step of the
// last position is committed and the gradients cleared (TTTCache
// continuation, "TTTLinear.ttt").
//
// One wave per (batch, head) chain.  Lane c owns column c of W and W_grad
// for all 64 rows, in registers for the whole call, so a call over T tokens
// reads and writes the 33 KB state once, and every product of a token is an
// in-lane multiply-add chain over the token's q or k, which the lanes read
// from LDS as broadcasts.  The only cross-lane work is the LayerNorm sums
// (DPP within 16-lane rows, then the four row totals through scalar
// registers); there are no barriers.  2048 chains take 2048 waves, which the
// chip holds at once.
// Used for decoding, for the tokens that complete an open mini-batch before a
// prefill, for a trailing partial mini-batch, and for mini-batch sizes the
// dual-form MFMA kernel does not take.
#include <algorithm>

#include "device_common.hpp"
#include "launch.hpp"

namespace ttt {

constexpr int kRP = 68;  // f32 pitch of the open rows of k (rows 4 banks apart)

// ROWS: W_grad holds the open mini-batch's rows [k_j | eta_j g_j] instead of
// their sum G.  Then q (W_s - G) = q W_s - sum_j (q . k_j) eta_j g_j: lane j
// forms q . k_j for the open rows j, and the sum runs over those scalars; the
// state read per call is W_s and the open rows, and a call writes only the
// rows it adds (and W_s, b_s at a commit).
template <typename Tin, typename Tout, bool ROWS>
__global__ __launch_bounds__(64, 2) void linear_token_kernel(LinearArgs a) {
    const int ch = blockIdx.x;
    const int bi = ch / a.H, hi = ch % a.H;
    const int c = threadIdx.x;  // column

    __shared__ __align__(16) float sq[kD], sk[kD];
    // rotary cos and signed sin at position p (mod K <= 16) for column c
    __shared__ float rcs[16][kD], rsn[16][kD];
    // ROWS: k_j and eta_j g_j of the open rows j < 16 of the current mini-batch
    __shared__ __align__(16) float kr[ROWS ? 16 : 1][ROWS ? kRP : 4];
    __shared__ float er[ROWS ? 16 : 1][kD];

    float *Wc = a.W + (int64_t)ch * kD * kD;
    float *Gc = a.Wg + (int64_t)ch * kD * kD;
    const int K = a.K;
    const int p0 = (int)(a.pos0 % K);  // rows of the open mini-batch at the start
    // a call that starts on a mini-batch boundary finds the accumulated
    // gradients cleared (every commit clears them), so it does not read them
    const bool g_clear = p0 == 0;

    const Tin *qp = (const Tin *)a.q.p + bi * a.q.sB + hi * a.q.sH;
    const Tin *kp = (const Tin *)a.k.p + bi * a.k.sB + hi * a.k.sH;
    const Tin *vp = (const Tin *)a.v.p + bi * a.v.sB + hi * a.v.sH;
    const float *ep = a.eta + bi * a.eta_sB + hi * a.eta_sH;
    Tout *op = (Tout *)a.out.p + bi * a.out.sB + hi * a.out.sH;
    // a token's inputs for column c (and the rotary partner column c ^ 32)
    struct TokIn {
        Tin q, k, v, qo, ko;
        float e;
    };
    auto load_tok = [&](int tok) {
        TokIn r;
        r.q = qp[(int64_t)tok * a.q.sL + c];
        r.k = kp[(int64_t)tok * a.k.sL + c];
        r.v = vp[(int64_t)tok * a.v.sL + c];
        r.e = ep[tok];
        if (a.rope) {
            r.qo = qp[(int64_t)tok * a.q.sL + (c ^ 32)];
            r.ko = kp[(int64_t)tok * a.k.sL + (c ^ 32)];
        }
        return r;
    };
    // every load of the state and of the first token is issued before the
    // first wait, so a call pays one memory round trip before its compute;
    // the open rows go first, so the work that needs only them can start
    // while W_s is still arriving
    float kk[ROWS ? 16 : 1], ee[ROWS ? 16 : 1];
    if constexpr (ROWS) {
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            if (j < p0) {
                kk[j] = Gc[j * 2 * kD + c];
                ee[j] = Gc[j * 2 * kD + kD + c];
            }
        }
    }
    TokIn nxt = load_tok(a.t0);
    // token_eta of position c of the mini-batch (lanes c < K), 1 without it
    const float te_c = (a.te != nullptr && c < K) ? a.te[c] : 1.f;
    float bs = a.b[(int64_t)ch * kD + c];
    float gbs = g_clear ? 0.f : a.bg[(int64_t)ch * kD + c];
    const float gam = a.ln_w[hi * kD + c];
    const float bet = a.ln_b[hi * kD + c];
    float Ws[kD], Gs[ROWS ? 1 : kD];
#pragma unroll
    for (int i = 0; i < kD; ++i) Ws[i] = Wc[i * kD + c];
    if constexpr (ROWS) {
        // rows past the open ones hold zeros, so the sum over the 16 rows in
        // the prediction needs no bound
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            kr[j][c] = j < p0 ? kk[j] : 0.f;
            er[j][c] = j < p0 ? ee[j] : 0.f;
        }
        wave_lds_order();
    } else if (g_clear) {
#pragma unroll
        for (int i = 0; i < kD; ++i) Gs[i] = 0.f;
    } else {
#pragma unroll
        for (int i = 0; i < kD; ++i) Gs[i] = Gc[i * kD + c];
    }
    bool committed = false;  // W_s, b_s change only at a commit

    if (a.rope) {
        // angle p * base^(-2i/D) for the pair (i, i + 32) holding column c, at
        // the positions p (mod K) this call's tokens take
        const int np = a.ntok < K ? a.ntok : K;
        for (int n = 0; n < np; ++n) {
            const int p = (p0 + n) % K;
            const double th = (double)p * pow((double)a.rope_base, -2.0 * (double)(c & 31) / (double)kD);
            rcs[p][c] = (float)cos(th);
            rsn[p][c] = (c < 32 ? -1.f : 1.f) * (float)sin(th);  // x*cos - x_pair*sin | x*cos + x_pair*sin
        }
    }

    for (int t = 0; t < a.ntok; ++t) {
        const int tok = a.t0 + t;
        const int64_t pos = a.pos0 + t;
        const int p = (int)(pos % K);  // row of this token in its mini-batch
        const TokIn in = nxt;
        // the step this token's prediction sees, and the step committed at
        // the end of the mini-batch, are scaled by token_eta of its position
        const float tp = lane_value(te_c, p);
        // the next token's inputs load during this token (the last token
        // reloads its own: no branch in the loop)
        nxt = load_tok(t + 1 < a.ntok ? tok + 1 : tok);
        float qv = to_f32(in.q);
        float kv = to_f32(in.k);
        const float vv = to_f32(in.v);
        const float e = in.e;
        if (a.rope) {
            const float cs = rcs[p][c], sg = rsn[p][c];
            qv = qv * cs + to_f32(in.qo) * sg;
            kv = kv * cs + to_f32(in.ko) * sg;
        }
        // one wave: its LDS accesses execute in order, so the reads below see
        // these writes (and the next token's writes follow these reads)
        sq[c] = qv;
        sk[c] = kv;
        wave_lds_order();

        // z = k W + b at the mini-batch-start state (four interleaved chains)
        float z4[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int i = 0; i < kD; i += 4) {
            const f32x4 k4 = *(const f32x4 *)&sk[i];
#pragma unroll
            for (int j = 0; j < 4; ++j) z4[j] = fmaf(k4[j], Ws[i + j], z4[j]);
        }
        const float z = ((z4[0] + z4[1]) + (z4[2] + z4[3])) + bs;

        // gradient of 1/2 ||LN(z) - (v - k)||^2; mean and mean square in one
        // reduction, as do mean(u) and mean(u xhat)
        float s1 = z, s2 = z * z;
        wave_sum2(s1, s2);
        const float mu = s1 * (1.f / kD);
        const float var = fmaxf(fmaf(-mu, mu, s2 * (1.f / kD)), 0.f);
        const float rs = rsqrtf(var + a.eps);
        const float xh = (z - mu) * rs;
        const float u = gam * (gam * xh + bet - (vv - kv));
        float su = u, sux = u * xh;
        wave_sum2(su, sux);
        su *= (1.f / kD);
        sux *= (1.f / kD);
        const float g = (u - su - xh * sux) * rs;

        // accumulate the eta-weighted gradient; prediction with W - W_grad
        const float eg = e * g;
        gbs += eg;
        float zb;
        if constexpr (ROWS) {
            kr[p][c] = kv;
            er[p][c] = eg;
            wave_lds_order();
            // lane j <= p: q . k_j over the open rows, this token's included
            float sj = 0.f;
            if (c <= p) {
                float d4[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int i = 0; i < kD; i += 4) {
                    const f32x4 q4 = *(const f32x4 *)&sq[i];
                    const f32x4 k4 = *(const f32x4 *)&kr[c][i];
#pragma unroll
                    for (int j = 0; j < 4; ++j) d4[j] = fmaf(q4[j], k4[j], d4[j]);
                }
                sj = (d4[0] + d4[1]) + (d4[2] + d4[3]);
            }
            float zq4[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int i = 0; i < kD; i += 4) {
                const f32x4 q4 = *(const f32x4 *)&sq[i];
#pragma unroll
                for (int j = 0; j < 4; ++j) zq4[j] = fmaf(q4[j], Ws[i + j], zq4[j]);
            }
            // (q G)[c] = sum_j (q . k_j) eta_j g_j[c]; rows j > p add zero
            // (sj is zero on lanes past p, and those rows are finite)
            float qg4[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int j = 0; j < 16; ++j) qg4[j & 3] = fmaf(lane_value(sj, j), er[j][c], qg4[j & 3]);
            const float qg = (qg4[0] + qg4[1]) + (qg4[2] + qg4[3]);
            zb = fmaf(-tp, qg, (zq4[0] + zq4[1]) + (zq4[2] + zq4[3])) + fmaf(-tp, gbs, bs);
        } else {
            float zb4[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int i = 0; i < kD; i += 4) {
                const f32x4 k4 = *(const f32x4 *)&sk[i];
                const f32x4 q4 = *(const f32x4 *)&sq[i];
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    Gs[i + j] = fmaf(k4[j], eg, Gs[i + j]);
                    zb4[j] = fmaf(q4[j], fmaf(-tp, Gs[i + j], Ws[i + j]), zb4[j]);
                }
            }
            zb = ((zb4[0] + zb4[1]) + (zb4[2] + zb4[3])) + fmaf(-tp, gbs, bs);
        }
        float t1 = zb, t2 = zb * zb;
        wave_sum2(t1, t2);
        const float mu2 = t1 * (1.f / kD);
        const float rs2 = rsqrtf(fmaxf(fmaf(-mu2, mu2, t2 * (1.f / kD)), 0.f) + a.eps);
        op[(int64_t)tok * a.out.sL + c] = from_f32<Tout>(qv + gam * (zb - mu2) * rs2 + bet);

        if (p == K - 1) {
            if constexpr (ROWS) {
                // W_s -= sum_j k_j^T (eta_j g_j), summed over j in token order
                float acc[kD];
#pragma unroll
                for (int i = 0; i < kD; ++i) acc[i] = 0.f;
                for (int j = 0; j < K; ++j) {
                    const float ej = er[j][c];
#pragma unroll
                    for (int i = 0; i < kD; i += 4) {
                        const f32x4 k4 = *(const f32x4 *)&kr[j][i];
#pragma unroll
                        for (int l = 0; l < 4; ++l) acc[i + l] = fmaf(k4[l], ej, acc[i + l]);
                    }
                }
#pragma unroll
                for (int i = 0; i < kD; ++i) Ws[i] = fmaf(-tp, acc[i], Ws[i]);
            } else {
#pragma unroll
                for (int i = 0; i < kD; ++i) {
                    Ws[i] = fmaf(-tp, Gs[i], Ws[i]);
                    Gs[i] = 0.f;
                }
            }
            bs = fmaf(-tp, gbs, bs);
            gbs = 0.f;
            committed = true;
        }
    }
    // write back what changed: W_s, b_s after a commit; the gradients unless
    // they were clear in memory and are clear again
    const int p_end = (int)((a.pos0 + a.ntok) % K);
    const bool g_clear_out = p_end == 0;
    if (committed) {
#pragma unroll
        for (int i = 0; i < kD; ++i) Wc[i * kD + c] = Ws[i];
        a.b[(int64_t)ch * kD + c] = bs;
    }
    if constexpr (ROWS) {
        // the rows this call added to the mini-batch left open
        for (int j = committed ? 0 : p0; j < p_end; ++j) {
            Gc[j * 2 * kD + c] = kr[j][c];
            Gc[j * 2 * kD + kD + c] = er[j][c];
        }
    } else if (!(g_clear && g_clear_out)) {
#pragma unroll
        for (int i = 0; i < kD; ++i) Gc[i * kD + c] = Gs[i];
    }
    if (!(g_clear && g_clear_out)) a.bg[(int64_t)ch * kD + c] = gbs;
}

// Segment y of one launch: dst[i] = src[i % per] for i < total (a per-head
// parameter tiled over the batch), or zeros with src == nullptr.  VEC: every
// pointer 16-byte aligned and per, total multiples of 4 (float4 accesses).
template <bool VEC>
__global__ void tile_kernel(TileList t) {
    const TileSeg sg = t.seg[blockIdx.y];
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    if constexpr (VEC) {
        const int64_t n4 = sg.total / 4, p4 = sg.per >= 4 ? sg.per / 4 : 1;
        for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n4; i += stride)
            ((float4 *)sg.dst)[i] = sg.src ? ((const float4 *)sg.src)[i % p4] : float4{0.f, 0.f, 0.f, 0.f};
    } else {
        for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < sg.total; i += stride)
            sg.dst[i] = sg.src ? sg.src[i % sg.per] : 0.f;
    }
}

template <bool ROWS>
void launch_token_layout(const LinearArgs &a, int in_bf16, int out_bf16, hipStream_t s) {
    dim3 grid(a.B * a.H), block(kWave);
    if (in_bf16 && out_bf16)
        hipLaunchKernelGGL((linear_token_kernel<__bf16, __bf16, ROWS>), grid, block, 0, s, a);
    else if (in_bf16)
        hipLaunchKernelGGL((linear_token_kernel<__bf16, float, ROWS>), grid, block, 0, s, a);
    else if (out_bf16)
        hipLaunchKernelGGL((linear_token_kernel<float, __bf16, ROWS>), grid, block, 0, s, a);
    else
        hipLaunchKernelGGL((linear_token_kernel<float, float, ROWS>), grid, block, 0, s, a);
}

hipError_t launch_linear_token(const LinearArgs &a, int in_bf16, int out_bf16, hipStream_t s) {
    if (a.grad_rows)
        launch_token_layout<true>(a, in_bf16, out_bf16, s);
    else
        launch_token_layout<false>(a, in_bf16, out_bf16, s);
    return hipGetLastError();
}

hipError_t launch_tiles(const TileList &t, hipStream_t s) {
    if (t.n <= 0) return hipSuccess;
    int64_t most = 0;
    bool vec = true;
    for (int i = 0; i < t.n; ++i) {
        const TileSeg &g = t.seg[i];
        most = g.total > most ? g.total : most;
        vec = vec && (g.src == nullptr || g.per % 4 == 0) && g.total % 4 == 0 && ((uintptr_t)g.dst & 15) == 0 &&
              ((uintptr_t)g.src & 15) == 0;
    }
    const int64_t items = vec ? most / 4 : most;
    const int64_t nb = std::min<int64_t>((items + 255) / 256, 2048);
    if (nb <= 0) return hipSuccess;
    const dim3 grid((unsigned)nb, (unsigned)t.n);
    if (vec)
        hipLaunchKernelGGL(tile_kernel<true>, grid, dim3(256), 0, s, t);
    else
        hipLaunchKernelGGL(tile_kernel<false>, grid, dim3(256), 0, s, t);
    return hipGetLastError();
}

}  // namespace ttt
