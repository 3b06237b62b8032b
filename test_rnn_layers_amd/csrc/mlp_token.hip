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
// and [x2_j | eta_j g2_j] instead of G1 and G2, and so does the call: the rows
// go to LDS, the threads keep only W1 and W2 in registers, and the prediction
// uses the rank form of the gradient sums,
//   q G1[:, f] = sum_j (q . k_j) eta_j g1_j[f],
//   xb2 G2[:, c] = sum_j (xb2 . x2_j) eta_j g2_j[c],
// with q . k_j formed by one lane per row and xb2 . x2_j by wave sums over
// the units.  The dense sums are formed only when a call closes the
// mini-batch (W -= t_K-1 sum_j ...).  A call stores only the rows it adds.
#include "device_common.hpp"
#include "gelu.hpp"
#include "launch.hpp"

namespace ttt {
namespace {

constexpr int kF = 256;
constexpr int kRow = kD + kF;  // floats per gradient row, both layers
constexpr int kKP = kD + 4;    // pitch of the k rows in LDS (lane j reads row j: rows 4 banks apart)

struct TokLds {
    float sq[kD], sk[kD];
    float x2s[kF], xb2s[kF];
    float dws[kF];                 // (g2 W2^T)[u]
    float g2s[kD];
    float part[4][kD];
    float tr[4][kD / 2][kD + 1];   // per block wave: products W2[64v + j][c] g2[c] at [j mod 32][c]
    float rcs[16][kD], rsn[16][kD];
};
struct RowLds {                    // ROWS: the open mini-batch's rows, j < 16
    float kr[16][kKP];             // k_j
    float x2r[16][kF];             // x2_j
    float e1r[16][kF];             // eta_j g1_j
    float e2r[16][kD];             // eta_j g2_j
    float ss[16];                  // q . k_j of the current token
    float dpart[4][16];            // per unit wave: its units' part of xb2 . x2_j
};
template <bool ROWS>
struct TokSmem {
    TokLds t;
    RowLds r;
};
template <>
struct TokSmem<false> {
    TokLds t;
};

template <typename Tin, typename Tout, bool ROWS>
__global__ __launch_bounds__(512, 1) void mlp_token_kernel(MlpArgs a) {
    extern __shared__ __align__(16) unsigned char smem_raw[];
    TokSmem<ROWS> &sm = *reinterpret_cast<TokSmem<ROWS> *>(smem_raw);
    TokLds &L = sm.t;
    const int ch = blockIdx.x;
    const int bi = ch / a.H, hi = ch % a.H;
    const int w = threadIdx.x >> 6, c = threadIdx.x & 63;
    const bool unit_wave = w < 4;
    const int f = threadIdx.x;        // unit waves: hidden unit of the W1 column
    const int v = w - 4;              // block waves: units 64v .. 64v+63, column c

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

    // the state: unit waves S = W1[:, f] (dense layout also T = G1[:, f]);
    // block waves S = W2[64v + j][c] (T = G2[64v + j][c])
    float S[kD], T[ROWS ? 1 : kD];
    const int64_t blk = (int64_t)(64 * v) * kD + c;  // block waves: offset of W2[64v][c]
    if constexpr (ROWS) {
        // the open rows j < p0 into LDS (their loads issued before W's)
        if (!g_clear) {
            RowLds &R = sm.r;
            for (int i = threadIdx.x; i < p0 * kF; i += 512) {
                const int j = i / kF, u = i % kF;
                R.x2r[j][u] = G2c[j * kRow + u];
                R.e1r[j][u] = G1c[j * kRow + kD + u];
            }
            for (int i = threadIdx.x; i < p0 * kD; i += 512) {
                const int j = i / kD, d = i % kD;
                R.kr[j][d] = G1c[j * kRow + d];
                R.e2r[j][d] = G2c[j * kRow + kF + d];
            }
        }
    }
    if (unit_wave) {
#pragma unroll
        for (int j = 0; j < kD; ++j) S[j] = W1c[j * kF + f];
    } else {
#pragma unroll
        for (int j = 0; j < kD; ++j) S[j] = W2c[blk + j * kD];
    }
    if constexpr (!ROWS) {
        if (g_clear) {
#pragma unroll
            for (int j = 0; j < kD; ++j) T[j] = 0.f;
        } else if (unit_wave) {
#pragma unroll
            for (int j = 0; j < kD; ++j) T[j] = G1c[j * kF + f];
        } else {
#pragma unroll
            for (int j = 0; j < kD; ++j) T[j] = G2c[blk + j * kD];
        }
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

    if (a.rope && w == 0) {
        // angle p * base^(-2i/D) for the pair (i, i + 32) holding column c, at
        // the positions p (mod K) this call's tokens take
        const int np = a.ntok < K ? a.ntok : K;
        for (int n = 0; n < np; ++n) {
            const int p = (p0 + n) % K;
            const double th = (double)p * pow((double)a.rope_base, -2.0 * (double)(c & 31) / (double)kD);
            L.rcs[p][c] = (float)cos(th);
            L.rsn[p][c] = (c < 32 ? -1.f : 1.f) * (float)sin(th);
        }
    }

    for (int t = 0; t < a.ntok; ++t) {
        const int tok = a.t0 + t;
        const int p = (int)((a.pos0 + t) % K);
        const bool keep = p != K - 1;  // ROWS: this token's row stays open (stored)
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
                const float cs = L.rcs[p][c], sg = L.rsn[p][c];
                qv = qv * cs + qo * sg;
                kv = kv * cs + ko * sg;
            }
            L.sq[c] = qv;
            L.sk[c] = kv;
            if constexpr (ROWS) {
                sm.r.kr[p][c] = kv;
                if (keep) G1c[p * kRow + c] = kv;
            }
        }
        __syncthreads();

        // unit waves: z1 = k W1 + b1 at the block-start state; GELU, GELU'
        float dg = 0.f, x2 = 0.f;
        if (unit_wave) {
            float z4[4] = {b1, 0.f, 0.f, 0.f};
#pragma unroll
            for (int i = 0; i < kD; i += 4) {
                const f32x4 k4 = *(const f32x4 *)&L.sk[i];
#pragma unroll
                for (int j = 0; j < 4; ++j) z4[j] = fmaf(k4[j], S[i + j], z4[j]);
            }
            const Gelu gz = gelu_both((z4[0] + z4[1]) + (z4[2] + z4[3]));
            x2 = gz.g;
            dg = gz.dg;
            L.x2s[f] = x2;
            if constexpr (ROWS) {
                sm.r.x2r[p][f] = x2;
                if (keep) G2c[p * kRow + f] = x2;
            }
        }
        if constexpr (ROWS) {
            if (!unit_wave && v == 0 && c <= p) {
                // q . k_j for the open rows, this token's included (lane j)
                float d4[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int i = 0; i < kD; i += 4) {
                    const f32x4 q4 = *(const f32x4 *)&L.sq[i];
                    const f32x4 k4 = *(const f32x4 *)&sm.r.kr[c][i];
#pragma unroll
                    for (int j = 0; j < 4; ++j) d4[j] = fmaf(q4[j], k4[j], d4[j]);
                }
                sm.r.ss[c] = (d4[0] + d4[1]) + (d4[2] + d4[3]);
            }
        }
        __syncthreads();

        // block waves: their units' part of z2 = x2 W2 for column c
        if (!unit_wave) {
            float s4[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int j = 0; j < kD; j += 4) {
                const f32x4 x4 = *(const f32x4 *)&L.x2s[64 * v + j];
#pragma unroll
                for (int l = 0; l < 4; ++l) s4[l] = fmaf(x4[l], S[j + l], s4[l]);
            }
            L.part[v][c] = (s4[0] + s4[1]) + (s4[2] + s4[3]);
        }
        __syncthreads();

        // wave 0: the LayerNorm backward of the reconstruction loss -> g2
        if (w == 0) {
            const float z = ((L.part[0][c] + L.part[1][c]) + (L.part[2][c] + L.part[3][c])) + b2;
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
            L.g2s[c] = (u - su - xh * sux) * rs;
        }
        __syncthreads();

        const float g2c = L.g2s[c];
        if (!unit_wave) {
            // g2 W2^T for unit 64v + c: row c of this wave's product tile, in
            // two halves of 32 units.  The reads take values other lanes wrote
            // (wave_lds_order keeps them after the writes).
#pragma unroll
            for (int h = 0; h < 2; ++h) {
#pragma unroll
                for (int j = 0; j < kD / 2; ++j) L.tr[v][j][c] = S[32 * h + j] * g2c;
                wave_lds_order();
                if ((c >> 5) == h) {
                    float d4[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int k = 0; k < kD; ++k) d4[k & 3] += L.tr[v][c & 31][k];
                    L.dws[64 * v + c] = (d4[0] + d4[1]) + (d4[2] + d4[3]);
                }
                wave_lds_order();
            }
            const float eg2c = e * g2c;
            if constexpr (ROWS) {
                if (v == 0) {
                    sm.r.e2r[p][c] = eg2c;
                    if (keep) G2c[p * kRow + kF + c] = eg2c;
                }
            } else {
                // the G2 step of the block: G2[u][c] += eta x2[u] g2[c]
#pragma unroll
                for (int j = 0; j < kD; j += 4) {
                    const f32x4 x4 = *(const f32x4 *)&L.x2s[64 * v + j];
#pragma unroll
                    for (int l = 0; l < 4; ++l) T[j + l] = fmaf(x4[l], eg2c, T[j + l]);
                }
            }
        }
        __syncthreads();

        // unit waves: g1 = (g2 W2^T) GELU'(z1); the prediction of the first
        // layer with W1 - t_p G1, b1 - t_p gb1
        if (unit_wave) {
            const float eg1 = e * (L.dws[f] * dg);
            gb1 += eg1;
            float zb4[4] = {fmaf(-tp, gb1, b1), 0.f, 0.f, 0.f};
            if constexpr (ROWS) {
                RowLds &R = sm.r;
                R.e1r[p][f] = eg1;
                if (keep) G1c[p * kRow + kD + f] = eg1;
#pragma unroll
                for (int i = 0; i < kD; i += 4) {
                    const f32x4 q4 = *(const f32x4 *)&L.sq[i];
#pragma unroll
                    for (int j = 0; j < 4; ++j) zb4[j] = fmaf(q4[j], S[i + j], zb4[j]);
                }
                float qg = 0.f;  // (q G1)[f] = sum_j (q . k_j) eta_j g1_j[f]
                for (int j = 0; j <= p; ++j) qg = fmaf(R.ss[j], R.e1r[j][f], qg);
                zb4[1] = fmaf(-tp, qg, zb4[1]);
            } else {
#pragma unroll
                for (int i = 0; i < kD; i += 4) {
                    const f32x4 k4 = *(const f32x4 *)&L.sk[i];
                    const f32x4 q4 = *(const f32x4 *)&L.sq[i];
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        T[i + j] = fmaf(k4[j], eg1, T[i + j]);
                        zb4[j] = fmaf(q4[j], fmaf(-tp, T[i + j], S[i + j]), zb4[j]);
                    }
                }
            }
            const float xb2 = gelu((zb4[0] + zb4[1]) + (zb4[2] + zb4[3]));
            L.xb2s[f] = xb2;
            if constexpr (ROWS) {
                // this wave's units' part of xb2 . x2_j for the open rows
                RowLds &R = sm.r;
                for (int j = 0; j <= p; j += 2) {
                    float d0 = xb2 * R.x2r[j][f];
                    float d1 = j + 1 <= p ? xb2 * R.x2r[j + 1][f] : 0.f;
                    wave_sum2(d0, d1);
                    if (c == 0) {
                        R.dpart[w][j] = d0;
                        if (j + 1 <= p) R.dpart[w][j + 1] = d1;
                    }
                }
            }
        }
        __syncthreads();

        // block waves: zb2 = xb2 (W2 - t_p G2) over their units for column c
        // (in the rows layout the G2 part is added by wave 0)
        if (!unit_wave) {
            float s4[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int j = 0; j < kD; j += 4) {
                const f32x4 x4 = *(const f32x4 *)&L.xb2s[64 * v + j];
#pragma unroll
                for (int l = 0; l < 4; ++l)
                    s4[l] = fmaf(x4[l], ROWS ? S[j + l] : fmaf(-tp, T[ROWS ? 0 : j + l], S[j + l]), s4[l]);
            }
            L.part[v][c] = (s4[0] + s4[1]) + (s4[2] + s4[3]);
        }
        __syncthreads();

        // wave 0: out = q + LN(zb2 + b2 - t_p gb2)
        if (w == 0) {
            gb2 = fmaf(e, g2c, gb2);
            float z = ((L.part[0][c] + L.part[1][c]) + (L.part[2][c] + L.part[3][c])) + fmaf(-tp, gb2, b2);
            if constexpr (ROWS) {
                // (xb2 G2)[c] = sum_j (xb2 . x2_j) eta_j g2_j[c]
                const RowLds &R = sm.r;
                float xg = 0.f;
                for (int j = 0; j <= p; ++j) {
                    const float dj = (R.dpart[0][j] + R.dpart[1][j]) + (R.dpart[2][j] + R.dpart[3][j]);
                    xg = fmaf(dj, R.e2r[j][c], xg);
                }
                z = fmaf(-tp, xg, z);
            }
            float s1 = z, s2 = z * z;
            wave_sum2(s1, s2);
            const float mu = s1 * (1.f / kD);
            const float rs = rsqrtf(fmaxf(fmaf(-mu, mu, s2 * (1.f / kD)), 0.f) + a.eps);
            op[(int64_t)tok * a.out.sL + c] = from_f32<Tout>(qv + gam * (z - mu) * rs + bet);
        }

        if (p == K - 1) {
            // commit the mini-batch's step (scaled by the last position's token_eta)
            if constexpr (ROWS) {
                // W -= t sum_j (outer product of row j), in token order
                const RowLds &R = sm.r;
                float acc[kD];
#pragma unroll
                for (int i = 0; i < kD; ++i) acc[i] = 0.f;
                for (int j = 0; j < K; ++j) {
                    const float ej = unit_wave ? R.e1r[j][f] : R.e2r[j][c];
                    const float *src = unit_wave ? &R.kr[j][0] : &R.x2r[j][64 * v];
#pragma unroll
                    for (int i = 0; i < kD; i += 4) {
                        const f32x4 r4 = *(const f32x4 *)&src[i];
#pragma unroll
                        for (int l = 0; l < 4; ++l) acc[i + l] = fmaf(r4[l], ej, acc[i + l]);
                    }
                }
#pragma unroll
                for (int i = 0; i < kD; ++i) S[i] = fmaf(-tp, acc[i], S[i]);
            } else {
#pragma unroll
                for (int j = 0; j < kD; ++j) {
                    S[j] = fmaf(-tp, T[j], S[j]);
                    T[j] = 0.f;
                }
            }
            b1 = fmaf(-tp, gb1, b1);
            gb1 = 0.f;
            b2 = fmaf(-tp, gb2, b2);
            gb2 = 0.f;
            committed = true;
        }
    }

    // write back what changed: W, b after a commit; the gradients unless they
    // were clear in memory and are clear again (rows: only b1_grad, b2_grad;
    // the rows were stored as they were made)
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
            if constexpr (!ROWS) {
#pragma unroll
                for (int j = 0; j < kD; ++j) G1c[j * kF + f] = T[j];
            }
            a.b1g[(int64_t)ch * kF + f] = gb1;
        } else {
            if constexpr (!ROWS) {
#pragma unroll
                for (int j = 0; j < kD; ++j) G2c[blk + j * kD] = T[j];
            }
        }
        if (w == 0) a.b2g[cD + c] = gb2;
    }
}

template <typename Tin, typename Tout, bool ROWS>
hipError_t launch_layout(const MlpArgs &a, hipStream_t s) {
    const void *fn = (const void *)&mlp_token_kernel<Tin, Tout, ROWS>;
    const size_t lds = sizeof(TokSmem<ROWS>);
    static std::atomic<uint64_t> configured{0};  // per instantiation: devices whose LDS limit is raised
    if (hipError_t e = ensure_lds_limit(fn, lds, configured); e != hipSuccess) return e;
    hipLaunchKernelGGL((mlp_token_kernel<Tin, Tout, ROWS>), dim3(a.B * a.H), dim3(512), lds, s, a);
    return hipGetLastError();
}

template <typename Tin, typename Tout>
hipError_t launch_typed(const MlpArgs &a, hipStream_t s) {
    return a.grad_rows ? launch_layout<Tin, Tout, true>(a, s) : launch_layout<Tin, Tout, false>(a, s);
}

}  // namespace

hipError_t launch_mlp_token(const MlpArgs &a, int in_bf16, int out_bf16, hipStream_t s) {
    if (in_bf16 && out_bf16) return launch_typed<__bf16, __bf16>(a, s);
    if (in_bf16) return launch_typed<__bf16, float>(a, s);
    if (out_bf16) return launch_typed<float, __bf16>(a, s);
    return launch_typed<float, float>(a, s);
}

}  // namespace ttt
