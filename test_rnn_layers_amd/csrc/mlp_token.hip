// mlp_token.hip -- TTT-MLP one token at a time (primal form): decoding, the
// tokens that complete an open mini-batch, and the calls the dual-form MLP
// kernel does not take (fp32 inputs, mini-batch sizes other than 16).
//
// The hidden state is f(x) = GELU(x W1 + b1) W2 + b2 (D = 64 -> F = 256 -> D),
// TTT-Linear stacked twice ("代码连连看——TTT", closing remark; README: the
// hidden state of TTT-MLP is a two-layer MLP).  Per token, as in the primal
// branch of compute_mini_batch applied to both layers:
//   z1 = k W1 + b1, x2 = GELU(z1), z2 = x2 W2 + b2          (block-start state)
//   g2 = d/dz2 of 1/2 ||LN(z2) - (v - k)||^2,  g1 = (g2 W2^T) o GELU'(z1)
//   G1 += eta k^T g1, gb1 += eta g1, G2 += eta x2^T g2, gb2 += eta g2
//   zb1 = q (W1 - t_p G1) + b1 - t_p gb1, xb2 = GELU(zb1)
//   zb2 = xb2 (W2 - t_p G2) + b2 - t_p gb2, out = q + LN(zb2)
// with t_p the token_eta of the token's position p in its mini-batch; at the
// end of a mini-batch W -= t_p G, b -= t_p gb and the gradients are cleared.
//
// One workgroup of 256 threads per (batch, head) chain; thread f owns hidden
// unit f: column f of W1 and G1 stays in registers for the whole call, row f
// of W2 and G2 is read from memory when needed.  The 64-wide sums over the
// hidden units (x2 W2, xb2 W2) are split over the four waves (64 units each,
// lane = output column) and added by wave 0, which also runs both LayerNorms.
// The prediction needs the G2 of all units after this token's update; it is
// formed from the G2 before the update plus the rank-one term
// eta (xb2 . x2) g2, so no thread reads a G2 row another thread is writing.
#include "device_common.hpp"
#include "gelu.hpp"
#include "launch.hpp"

namespace ttt {
namespace {

constexpr int kF = 256;

template <typename Tin, typename Tout>
__global__ __launch_bounds__(256, 1) void mlp_token_kernel(MlpArgs a) {
    const int ch = blockIdx.x;
    const int bi = ch / a.H, hi = ch % a.H;
    const int f = threadIdx.x;          // hidden unit
    const int w = f >> 6, c = f & 63;   // wave; lane = output column in the sums over units

    __shared__ __align__(16) float sq[kD], sk[kD];
    __shared__ __align__(16) float x2s[kF], xb2s[kF];
    __shared__ __align__(16) float g2s[kD];
    __shared__ float part[4][kD];
    __shared__ float red[4];
    __shared__ float rcs[16][kD], rsn[16][kD];

    const int64_t cD = (int64_t)ch * kD;
    float *W1c = a.W1 + cD * kF, *G1c = a.W1g + cD * kF;  // [D][F]
    float *W2c = a.W2 + cD * kF, *G2c = a.W2g + cD * kF;  // [F][D]
    const int K = a.K;
    const int p0 = (int)(a.pos0 % K);
    // a call that starts on a mini-batch boundary finds the gradients cleared
    const bool g_clear = p0 == 0;

    const Tin *qp = (const Tin *)a.q.p + bi * a.q.sB + hi * a.q.sH;
    const Tin *kp = (const Tin *)a.k.p + bi * a.k.sB + hi * a.k.sH;
    const Tin *vp = (const Tin *)a.v.p + bi * a.v.sB + hi * a.v.sH;
    const float *ep = a.eta + bi * a.eta_sB + hi * a.eta_sH;
    Tout *op = (Tout *)a.out.p + bi * a.out.sB + hi * a.out.sH;

    // state of unit f
    float W1r[kD], G1r[kD];
#pragma unroll
    for (int i = 0; i < kD; ++i) W1r[i] = W1c[i * kF + f];
    if (g_clear) {
#pragma unroll
        for (int i = 0; i < kD; ++i) G1r[i] = 0.f;
    } else {
#pragma unroll
        for (int i = 0; i < kD; ++i) G1r[i] = G1c[i * kF + f];
    }
    float b1 = a.b1[(int64_t)ch * kF + f];
    float gb1 = g_clear ? 0.f : a.b1g[(int64_t)ch * kF + f];
    // wave 0: column c of b2, gb2 and of the LayerNorm parameters
    float b2 = 0.f, gb2 = 0.f, gam = 0.f, bet = 0.f;
    if (w == 0) {
        b2 = a.b2[cD + c];
        gb2 = g_clear ? 0.f : a.b2g[cD + c];
        gam = a.ln_w[hi * kD + c];
        bet = a.ln_b[hi * kD + c];
    }
    // token_eta of position c of the mini-batch (lanes c < K of every wave), 1 without it
    const float te_c = (a.te != nullptr && c < K) ? a.te[c] : 1.f;
    bool committed = false;  // W, b change only at a commit

    if (a.rope && w == 0) {
        // angle p * base^(-2i/D) for the pair (i, i + 32) holding column c, at
        // the positions p (mod K) this call's tokens take
        const int np = a.ntok < K ? a.ntok : K;
        for (int n = 0; n < np; ++n) {
            const int p = (p0 + n) % K;
            const double th = (double)p * pow((double)a.rope_base, -2.0 * (double)(c & 31) / (double)kD);
            rcs[p][c] = (float)cos(th);
            rsn[p][c] = (c < 32 ? -1.f : 1.f) * (float)sin(th);
        }
    }

    for (int t = 0; t < a.ntok; ++t) {
        const int tok = a.t0 + t;
        const int p = (int)((a.pos0 + t) % K);
        const float e = ep[tok];
        const float tp = lane_value(te_c, p);  // the same in every wave
        // the first token of a mini-batch finds G2 cleared (by the commit
        // before it, or at a call that starts on a boundary): not read
        const bool g2_zero = p == 0;
        float qv = 0.f, kv = 0.f, vv = 0.f;
        if (w == 0) {
            qv = to_f32(qp[(int64_t)tok * a.q.sL + c]);
            kv = to_f32(kp[(int64_t)tok * a.k.sL + c]);
            vv = to_f32(vp[(int64_t)tok * a.v.sL + c]);
            if (a.rope) {
                const float qo = to_f32(qp[(int64_t)tok * a.q.sL + (c ^ 32)]);
                const float ko = to_f32(kp[(int64_t)tok * a.k.sL + (c ^ 32)]);
                const float cs = rcs[p][c], sg = rsn[p][c];
                qv = qv * cs + qo * sg;
                kv = kv * cs + ko * sg;
            }
            sq[c] = qv;
            sk[c] = kv;
        }
        __syncthreads();

        // z1 = k W1 + b1 at the block-start state; GELU and GELU'
        float z4[4] = {b1, 0.f, 0.f, 0.f};
#pragma unroll
        for (int i = 0; i < kD; i += 4) {
            const f32x4 k4 = *(const f32x4 *)&sk[i];
#pragma unroll
            for (int j = 0; j < 4; ++j) z4[j] = fmaf(k4[j], W1r[i + j], z4[j]);
        }
        const Gelu gz = gelu_both((z4[0] + z4[1]) + (z4[2] + z4[3]));
        const float x2 = gz.g;
        x2s[f] = x2;
        __syncthreads();

        // z2 = x2 W2 + b2: wave w sums units 64w .. 64w+63 for column c
        {
            const float *w2 = W2c + (int64_t)(64 * w) * kD + c;
            float s4[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 16
            for (int j = 0; j < 64; ++j) s4[j & 3] = fmaf(x2s[64 * w + j], w2[j * kD], s4[j & 3]);
            part[w][c] = (s4[0] + s4[1]) + (s4[2] + s4[3]);
        }
        __syncthreads();

        // wave 0: the LayerNorm backward of the reconstruction loss -> g2
        float g2 = 0.f;
        if (w == 0) {
            const float z = ((part[0][c] + part[1][c]) + (part[2][c] + part[3][c])) + b2;
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
            g2 = (u - su - xh * sux) * rs;
            g2s[c] = g2;
        }
        __syncthreads();

        // unit f: g1 = (W2[f, :] . g2) GELU'(z1); accumulate the gradients of W1, b1
        float dw = 0.f;
        {
            const f32x4 *w2r = (const f32x4 *)(W2c + (int64_t)f * kD);
            float d4[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
            for (int m = 0; m < kD / 4; ++m) {
                const f32x4 wv = w2r[m];
                const f32x4 gv = *(const f32x4 *)&g2s[4 * m];
#pragma unroll
                for (int j = 0; j < 4; ++j) d4[j] = fmaf(wv[j], gv[j], d4[j]);
            }
            dw = (d4[0] + d4[1]) + (d4[2] + d4[3]);
        }
        const float eg1 = e * (dw * gz.dg);
        gb1 += eg1;
        // prediction of the first layer with W1 - t_p G1, b1 - t_p gb1
        float zb4[4] = {fmaf(-tp, gb1, b1), 0.f, 0.f, 0.f};
#pragma unroll
        for (int i = 0; i < kD; i += 4) {
            const f32x4 k4 = *(const f32x4 *)&sk[i];
            const f32x4 q4 = *(const f32x4 *)&sq[i];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                G1r[i + j] = fmaf(k4[j], eg1, G1r[i + j]);
                zb4[j] = fmaf(q4[j], fmaf(-tp, G1r[i + j], W1r[i + j]), zb4[j]);
            }
        }
        const float xb2 = gelu((zb4[0] + zb4[1]) + (zb4[2] + zb4[3]));
        xb2s[f] = xb2;
        // xb2 . x2 over the units, for the rank-one part of this token's G2 step
        float dot = xb2 * x2, dummy = 0.f;
        wave_sum2(dot, dummy);
        if (c == 0) red[w] = dot;
        __syncthreads();

        // zb2 partial sums with the G2 before this token's step
        {
            const float *w2 = W2c + (int64_t)(64 * w) * kD + c;
            const float *g2p = G2c + (int64_t)(64 * w) * kD + c;
            float s4[4] = {0.f, 0.f, 0.f, 0.f};
            if (g2_zero) {
#pragma unroll 16
                for (int j = 0; j < 64; ++j) s4[j & 3] = fmaf(xb2s[64 * w + j], w2[j * kD], s4[j & 3]);
            } else {
#pragma unroll 8
                for (int j = 0; j < 64; ++j)
                    s4[j & 3] = fmaf(xb2s[64 * w + j], fmaf(-tp, g2p[j * kD], w2[j * kD]), s4[j & 3]);
            }
            part[w][c] = (s4[0] + s4[1]) + (s4[2] + s4[3]);
        }
        __syncthreads();

        // wave 0: zb2 = xb2 (W2 - t_p G2) + b2 - t_p gb2, out = q + LN(zb2)
        if (w == 0) {
            const float eg2 = e * g2;
            gb2 += eg2;
            const float sx = (red[0] + red[1]) + (red[2] + red[3]);
            float z = ((part[0][c] + part[1][c]) + (part[2][c] + part[3][c])) + fmaf(-tp, gb2, b2);
            z = fmaf(-tp * sx, eg2, z);
            float s1 = z, s2 = z * z;
            wave_sum2(s1, s2);
            const float mu = s1 * (1.f / kD);
            const float rs = rsqrtf(fmaxf(fmaf(-mu, mu, s2 * (1.f / kD)), 0.f) + a.eps);
            op[(int64_t)tok * a.out.sL + c] = from_f32<Tout>(qv + gam * (z - mu) * rs + bet);
        }

        // unit f: the G2 step of its row (and, at the end of the mini-batch,
        // the commit of W2's row); the LDS reads of g2 here end before the
        // next token's barriers let wave 0 overwrite it
        const bool commit = p == K - 1;
        {
            f32x4 *g2r = (f32x4 *)(G2c + (int64_t)f * kD);
            f32x4 *w2r = (f32x4 *)(W2c + (int64_t)f * kD);
            const float ex = e * x2;
#pragma unroll 4
            for (int m = 0; m < kD / 4; ++m) {
                const f32x4 gv = *(const f32x4 *)&g2s[4 * m];
                f32x4 gr = g2_zero ? f32x4{0.f, 0.f, 0.f, 0.f} : g2r[m];
#pragma unroll
                for (int j = 0; j < 4; ++j) gr[j] = fmaf(ex, gv[j], gr[j]);
                if (commit) {
                    f32x4 wr = w2r[m];
#pragma unroll
                    for (int j = 0; j < 4; ++j) wr[j] = fmaf(-tp, gr[j], wr[j]);
                    w2r[m] = wr;
                    gr = f32x4{0.f, 0.f, 0.f, 0.f};
                }
                g2r[m] = gr;
            }
        }
        if (commit) {
#pragma unroll
            for (int i = 0; i < kD; ++i) {
                W1r[i] = fmaf(-tp, G1r[i], W1r[i]);
                G1r[i] = 0.f;
            }
            b1 = fmaf(-tp, gb1, b1);
            gb1 = 0.f;
            if (w == 0) {
                b2 = fmaf(-tp, gb2, b2);
                gb2 = 0.f;
            }
            committed = true;
        }
        __syncthreads();  // G2 and W2 rows stored before the next token reads them
    }

    // write back W1 (after a commit), G1, and the biases
    if (committed) {
#pragma unroll
        for (int i = 0; i < kD; ++i) W1c[i * kF + f] = W1r[i];
        a.b1[(int64_t)ch * kF + f] = b1;
        if (w == 0) a.b2[cD + c] = b2;
    }
#pragma unroll
    for (int i = 0; i < kD; ++i) G1c[i * kF + f] = G1r[i];
    a.b1g[(int64_t)ch * kF + f] = gb1;
    if (w == 0) a.b2g[cD + c] = gb2;
}

template <typename Tin, typename Tout>
hipError_t launch_typed(const MlpArgs &a, hipStream_t s) {
    hipLaunchKernelGGL((mlp_token_kernel<Tin, Tout>), dim3(a.B * a.H), dim3(kF), 0, s, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_mlp_token(const MlpArgs &a, int in_bf16, int out_bf16, hipStream_t s) {
    if (in_bf16 && out_bf16) return launch_typed<__bf16, __bf16>(a, s);
    if (in_bf16) return launch_typed<__bf16, float>(a, s);
    if (out_bf16) return launch_typed<float, __bf16>(a, s);
    return launch_typed<float, float>(a, s);
}

}  // namespace ttt
