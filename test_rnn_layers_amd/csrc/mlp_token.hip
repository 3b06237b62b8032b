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
// One workgroup of 512 threads (8 waves) per (batch, head) chain; the whole
// state stays in registers for the call, 128 values per thread:
//  * unit waves 0..3: thread f = 64w + c holds column f of W1 and G1; they
//    form z1, GELU(z1), GELU'(z1), the G1 step and zb1 = q (W1 - t G1) + ...
//    as in-thread chains over the token's k or q (LDS broadcasts);
//  * block waves 4..7: lane c of wave 4 + v holds the block
//    W2[64v .. 64v+63][c] and the same block of G2; they form the sums over
//    their 64 units of x2 W2 and xb2 (W2 - t G2) for column c (added over the
//    four block waves by wave 0), the G2 step, and g2 W2^T: each lane writes
//    its 64 products to a per-wave LDS tile and reads back one row (one
//    wave's LDS accesses execute in order, so no barrier in between);
//  * wave 0 also loads the token and runs both LayerNorms.
// The two roles keep their state in the same two register arrays.  A call
// reads and writes the state once; per token it reads q, k, v, eta and
// writes one output row.
// ROWS: the gradient state holds the open mini-batch's rows [k_j | eta_j g1_j]
// and [x2_j | eta_j g2_j] instead of G1 and G2.  The call rebuilds its dense
// G1 columns and G2 blocks in registers from the rows (while W1, W2 are still
// arriving), runs as above, and stores only the rows its tokens add.
#include "device_common.hpp"
#include "gelu.hpp"
#include "launch.hpp"

namespace ttt {
namespace {

constexpr int kF = 256;
constexpr int kRow = kD + kF;  // floats per gradient row, both layers

template <typename Tin, typename Tout, bool ROWS>
__global__ __launch_bounds__(512, 1) void mlp_token_kernel(MlpArgs a) {
    const int ch = blockIdx.x;
    const int bi = ch / a.H, hi = ch % a.H;
    const int w = threadIdx.x >> 6, c = threadIdx.x & 63;
    const bool unit_wave = w < 4;
    const int f = threadIdx.x;        // unit waves: hidden unit of the W1 column
    const int v = w - 4;              // block waves: units 64v .. 64v+63, column c

    __shared__ __align__(16) float sq[kD], sk[kD];
    __shared__ __align__(16) float x2s[kF], xb2s[kF];
    __shared__ float dws[kF];          // (g2 W2^T)[u]
    __shared__ float g2s[kD];
    __shared__ float part[4][kD];
    // per block wave: products W2[64v + j][c] g2[c] at [j mod 32][c]; in the
    // rows layout first the open rows' x2 (before the token loop)
    __shared__ __align__(16) float trbuf[4 * (kD / 2) * (kD + 1)];
    float (*tr)[kD / 2][kD + 1] = reinterpret_cast<float (*)[kD / 2][kD + 1]>(trbuf);
    __shared__ __align__(16) float kr[ROWS ? 16 : 1][kD];  // ROWS: the open rows' k
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

    // the state: unit waves S = W1[:, f], T = G1[:, f]; block waves
    // S = W2[64v + j][c], T = G2[64v + j][c]
    float S[kD], T[kD];
    const int64_t blk = (int64_t)(64 * v) * kD + c;  // block waves: offset of W2[64v][c]
    if (unit_wave) {
#pragma unroll
        for (int j = 0; j < kD; ++j) S[j] = W1c[j * kF + f];
    } else {
#pragma unroll
        for (int j = 0; j < kD; ++j) S[j] = W2c[blk + j * kD];
    }
    if (g_clear || ROWS) {
#pragma unroll
        for (int j = 0; j < kD; ++j) T[j] = 0.f;
    } else if (unit_wave) {
#pragma unroll
        for (int j = 0; j < kD; ++j) T[j] = G1c[j * kF + f];
    } else {
#pragma unroll
        for (int j = 0; j < kD; ++j) T[j] = G2c[blk + j * kD];
    }
    float b1 = 0.f, gb1 = 0.f;
    if (unit_wave) {
        b1 = a.b1[(int64_t)ch * kF + f];
        gb1 = g_clear ? 0.f : a.b1g[(int64_t)ch * kF + f];
    }
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

    if constexpr (ROWS) {
        if (!g_clear) {
            // the open rows j < p0: unit thread f needs eta_j g1_j[f], block
            // thread (v, c) needs eta_j g2_j[c] (registers); k_j and x2_j are
            // read by many threads (LDS)
            float e[16];
#pragma unroll
            for (int j = 0; j < 16; ++j)
                if (j < p0) e[j] = unit_wave ? G1c[j * kRow + kD + f] : G2c[j * kRow + kF + c];
            float *x2r = trbuf;  // [16][kF]
            for (int i = threadIdx.x; i < p0 * kF; i += 512) x2r[i] = G2c[(i / kF) * kRow + (i % kF)];
            if (w == 0)
                for (int j = 0; j < p0; ++j) kr[j][c] = G1c[j * kRow + c];
            __syncthreads();
            // G1[:, f] = sum_j k_j eta_j g1_j[f];  G2[64v + u][c] = sum_j x2_j[64v + u] eta_j g2_j[c]
#pragma unroll
            for (int j = 0; j < 16; ++j) {
                if (j < p0) {
                    const float *src = unit_wave ? &kr[j][0] : &x2r[j * kF + 64 * v];
#pragma unroll
                    for (int i = 0; i < kD; i += 4) {
                        const f32x4 r4 = *(const f32x4 *)&src[i];
#pragma unroll
                        for (int l = 0; l < 4; ++l) T[i + l] = fmaf(r4[l], e[j], T[i + l]);
                    }
                }
            }
            __syncthreads();  // the x2 rows are read before the buffer becomes the product tile
        }
    }

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
            // ROWS: this token's row of k, unless it closes the mini-batch
            if (ROWS && p != K - 1) G1c[p * kRow + c] = kv;
        }
        __syncthreads();

        // unit waves: z1 = k W1 + b1 at the block-start state; GELU, GELU'
        float dg = 0.f;
        if (unit_wave) {
            float z4[4] = {b1, 0.f, 0.f, 0.f};
#pragma unroll
            for (int i = 0; i < kD; i += 4) {
                const f32x4 k4 = *(const f32x4 *)&sk[i];
#pragma unroll
                for (int j = 0; j < 4; ++j) z4[j] = fmaf(k4[j], S[i + j], z4[j]);
            }
            const Gelu gz = gelu_both((z4[0] + z4[1]) + (z4[2] + z4[3]));
            x2s[f] = gz.g;
            dg = gz.dg;
            if (ROWS && p != K - 1) G2c[p * kRow + f] = gz.g;
        }
        __syncthreads();

        // block waves: their units' part of z2 = x2 W2 for column c
        if (!unit_wave) {
            float s4[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int j = 0; j < kD; j += 4) {
                const f32x4 x4 = *(const f32x4 *)&x2s[64 * v + j];
#pragma unroll
                for (int l = 0; l < 4; ++l) s4[l] = fmaf(x4[l], S[j + l], s4[l]);
            }
            part[v][c] = (s4[0] + s4[1]) + (s4[2] + s4[3]);
        }
        __syncthreads();

        // wave 0: the LayerNorm backward of the reconstruction loss -> g2
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
            g2s[c] = (u - su - xh * sux) * rs;
        }
        __syncthreads();

        const float g2c = g2s[c];
        if (!unit_wave) {
            // g2 W2^T for unit 64v + c: row c of this wave's product tile, in
            // two halves of 32 units.  The reads take values other lanes wrote
            // (wave_lds_order keeps them after the writes).
#pragma unroll
            for (int h = 0; h < 2; ++h) {
#pragma unroll
                for (int j = 0; j < kD / 2; ++j) tr[v][j][c] = S[32 * h + j] * g2c;
                wave_lds_order();
                if ((c >> 5) == h) {
                    float d4[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int k = 0; k < kD; ++k) d4[k & 3] += tr[v][c & 31][k];
                    dws[64 * v + c] = (d4[0] + d4[1]) + (d4[2] + d4[3]);
                }
                wave_lds_order();
            }
            // the G2 step of the block: G2[u][c] += eta x2[u] g2[c]
            const float eg2c = e * g2c;
#pragma unroll
            for (int j = 0; j < kD; j += 4) {
                const f32x4 x4 = *(const f32x4 *)&x2s[64 * v + j];
#pragma unroll
                for (int l = 0; l < 4; ++l) T[j + l] = fmaf(x4[l], eg2c, T[j + l]);
            }
        }
        __syncthreads();

        // unit waves: g1 = (g2 W2^T) GELU'(z1); the G1 step; the prediction of
        // the first layer with W1 - t_p G1, b1 - t_p gb1
        if (unit_wave) {
            const float eg1 = e * (dws[f] * dg);
            gb1 += eg1;
            if (ROWS && p != K - 1) G1c[p * kRow + kD + f] = eg1;
            float zb4[4] = {fmaf(-tp, gb1, b1), 0.f, 0.f, 0.f};
#pragma unroll
            for (int i = 0; i < kD; i += 4) {
                const f32x4 k4 = *(const f32x4 *)&sk[i];
                const f32x4 q4 = *(const f32x4 *)&sq[i];
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    T[i + j] = fmaf(k4[j], eg1, T[i + j]);
                    zb4[j] = fmaf(q4[j], fmaf(-tp, T[i + j], S[i + j]), zb4[j]);
                }
            }
            xb2s[f] = gelu((zb4[0] + zb4[1]) + (zb4[2] + zb4[3]));
        }
        __syncthreads();

        // block waves: zb2 = xb2 (W2 - t_p G2) over their units for column c
        if (!unit_wave) {
            float s4[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int j = 0; j < kD; j += 4) {
                const f32x4 x4 = *(const f32x4 *)&xb2s[64 * v + j];
#pragma unroll
                for (int l = 0; l < 4; ++l) s4[l] = fmaf(x4[l], fmaf(-tp, T[j + l], S[j + l]), s4[l]);
            }
            part[v][c] = (s4[0] + s4[1]) + (s4[2] + s4[3]);
        }
        __syncthreads();

        // wave 0: out = q + LN(zb2 + b2 - t_p gb2)
        if (w == 0) {
            gb2 = fmaf(e, g2c, gb2);
            if (ROWS && p != K - 1) G2c[p * kRow + kF + c] = e * g2c;
            const float z = ((part[0][c] + part[1][c]) + (part[2][c] + part[3][c])) + fmaf(-tp, gb2, b2);
            float s1 = z, s2 = z * z;
            wave_sum2(s1, s2);
            const float mu = s1 * (1.f / kD);
            const float rs = rsqrtf(fmaxf(fmaf(-mu, mu, s2 * (1.f / kD)), 0.f) + a.eps);
            op[(int64_t)tok * a.out.sL + c] = from_f32<Tout>(qv + gam * (z - mu) * rs + bet);
        }

        if (p == K - 1) {
            // commit the mini-batch's step (scaled by the last position's token_eta)
#pragma unroll
            for (int j = 0; j < kD; ++j) {
                S[j] = fmaf(-tp, T[j], S[j]);
                T[j] = 0.f;
            }
            b1 = fmaf(-tp, gb1, b1);
            gb1 = 0.f;
            b2 = fmaf(-tp, gb2, b2);
            gb2 = 0.f;
            committed = true;
        }
    }

    // write back what changed: W, b after a commit; the gradients unless they
    // were clear in memory and are clear again
    const bool g_clear_out = (a.pos0 + a.ntok) % K == 0;
    if (committed) {
        if (unit_wave) {
#pragma unroll
            for (int j = 0; j < kD; ++j) W1c[j * kF + f] = S[j];
            a.b1[(int64_t)ch * kF + f] = b1;
        } else {
#pragma unroll
            for (int j = 0; j < kD; ++j) W2c[blk + j * kD] = S[j];
        }
        if (w == 0) a.b2[cD + c] = b2;
    }
    if (!(g_clear && g_clear_out)) {
        if (unit_wave) {
            if (!ROWS) {
#pragma unroll
                for (int j = 0; j < kD; ++j) G1c[j * kF + f] = T[j];
            }
            a.b1g[(int64_t)ch * kF + f] = gb1;
        } else if (!ROWS) {
#pragma unroll
            for (int j = 0; j < kD; ++j) G2c[blk + j * kD] = T[j];
        }
        if (w == 0) a.b2g[cD + c] = gb2;
    }
}

template <typename Tin, typename Tout>
hipError_t launch_typed(const MlpArgs &a, hipStream_t s) {
    if (a.grad_rows)
        hipLaunchKernelGGL((mlp_token_kernel<Tin, Tout, true>), dim3(a.B * a.H), dim3(512), 0, s, a);
    else
        hipLaunchKernelGGL((mlp_token_kernel<Tin, Tout, false>), dim3(a.B * a.H), dim3(512), 0, s, a);
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
