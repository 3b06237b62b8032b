// mlp_dual.hip -- TTT-MLP over mini-batches of 16 tokens in the dual form.
//
// The hidden state is a two-layer MLP f(x) = GELU(x W1 + b1) W2 + b2
// (D = 64 -> F = 256 -> D), the TTT-Linear step applied to each layer
// ("代码连连看——TTT": TTT-MLP is TTT-Linear stacked twice; README: the hidden
// state of TTT-MLP is a two-layer MLP).  Per mini-batch (K rows X = k, Q, V;
// T = diag(token_eta_i), t = token_eta of the last row):
//   Z1 = X W1 + b1, X2 = GELU(Z1), Z2 = X2 W2 + b2
//   ng2 = -eta * d/dZ2 of 1/2 ||LN(Z2) - (V - X)||^2
//   ng1 = (ng2 W2^T) o GELU'(Z1)
//   Zb1 = Q W1 + b1 + T tril(Q X^T + 1) ng1,  Xb2 = GELU(Zb1)
//   Zb2 = Xb2 W2 + b2 + T tril(Xb2 X2^T + 1) ng2,  out = Q + LN(Zb2)
//   W1 += t X^T ng1, b1 += t 1^T ng1, W2 += t X2^T ng2, b2 += t 1^T ng2
// A trailing partial mini-batch (r < 16 tokens) runs with eta = 0 on the
// missing rows; its step is not applied: the accumulated gradients go to
// the *_grad state instead (an open mini-batch).
//
// Design (gfx950, one workgroup of 8 waves per (batch, head)):
//  * wave w owns hidden units f in [32w, 32w+32): its 64x32 slab of W1 and
//    its 32x64 slab of W2, as fp32 MFMA accumulator tiles for the whole
//    chain; the backward product ng2 W2^T contracts over the other index of
//    W2, whose fragments come from this wave's tiles by identity products;
//  * Z1, Zb1, ng1, X2 stay in registers in accumulator layout, which is also
//    the operand layout of the M1 ng1 correction and of the three state
//    updates; X2, Xb2 and ng2 go through LDS where a row layout is needed;
//  * Z2 and Zb2 are sums over the 8 hidden slices: partial tiles in LDS,
//    summed by the LayerNorm waves 0..3 (16 lanes per token row, DPP sums),
//    which also leave a transposed fp16 copy of ng2 (its B fragments);
//  * waves 4..7 stage the next mini-batch while waves 0..3 run the LayerNorm
//    backward: rotated q, k as fp16 rows and a transposed copy of k (the K^T
//    fragments of the W1 step), and the LayerNorm operands in fp32;
//  * operands are fp16 (bf16 inputs), accumulation fp32; GELU in the erf form;
//  * range: ng2 (hence ng1) is carried as 2^8 of its value and the operands
//    it multiplies (the causal matrices, K^T, X2, the ones of the bias steps)
//    as 2^-8 of theirs: the products are unchanged (powers of two are exact),
//    dot products up to 2^8 * 65504 stay inside fp16 and small gradients stay
//    normal.  fp16 still bounds |q|, |k|, |W1|, |W2|, |GELU(Z1)| <= 65504
//    and |eta g2|, |eta g1| < 256 elementwise.
#include <type_traits>

#include "device_common.hpp"
#include "gelu.hpp"
#include "launch.hpp"

namespace ttt {
namespace {

constexpr int kM = 16;
constexpr int kF = 256;
constexpr int XP = 72;    // f16 row pitch of the 16x64 tiles
constexpr int HP = 268;   // f16 row pitch of the 16x256 tiles (134 dwords: the column writes of X2, Xb2 hit 32 distinct banks)
constexpr int NP = 68;    // f16 row pitch of the ng2 tile
constexpr int FP = 68;    // fp32 row pitch of the partial sums
constexpr int kParts = 8; // hidden slices
constexpr int TP = 20;    // f16 pitch of the transposed 64x16 tiles (rows 40 B apart)
// ng2, ng1 are carried scaled by kNgScale, the operands that multiply them by 1/kNgScale
constexpr float kNgScale = 256.f;
constexpr float kMatScale = 1.f / kNgScale;

typedef _Float16 h4 __attribute__((ext_vector_type(4)));
typedef _Float16 h8 __attribute__((ext_vector_type(8)));

struct Smem {
    _Float16 xs[2][kM][XP];   // K rows (rotated), double-buffered by mini-batch
    _Float16 qs[2][kM][XP];   // Q rows (rotated)
    _Float16 kT[2][kD][TP];   // K^T (rotated), [d][token], by parity
    _Float16 ng2T[kD][TP];    // ng2^T, [d][token]
    _Float16 x2[kM][HP];      // X2 = GELU(Z1), [token][hidden]
    _Float16 xb2[kM][HP];     // Xb2 = GELU(Zb1)
    _Float16 ng2[kM][NP];     // ng2, [token][d]
    float part[2][kParts][kM][FP];  // partial sums [slice][token][d]: [0] of Z2, [1] of Zb2
    float cel[2][kM][kD];     // eta (gamma (k - v) + gamma beta), by mini-batch parity
    float qres[2][kM][kD];    // q + beta (the residual of the output), by parity
    float eta[2][kM];         // learning rate per token, by parity
    float b2[kD];             // b2 at the start of the current mini-batch
    float b2n[kD];            // b2 after its step
    float gam[kD], gam2[kD], bet[kD], gb[kD];  // per-column LayerNorm constants
    float cs[kM][kD], sn[kM][kD];            // rotary cos / signed sin at position t, column c
};

__device__ __forceinline__ f32x4 mfma32(h8 a, h8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma16(h4 a, h4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ h4 to_h4(f32x4 x) {
    return h4{(_Float16)x[0], (_Float16)x[1], (_Float16)x[2], (_Float16)x[3]};
}
// two accumulator tiles (rows 4g+j and 16+4g+j) as a 16x16x32 B operand whose
// k slot 8g+i carries row 4g+i (i < 4) or 16+4g+i-4 (i >= 4)
__device__ __forceinline__ h8 pair_b(f32x4 lo, f32x4 hi) {
    return h8{(_Float16)lo[0], (_Float16)lo[1], (_Float16)lo[2], (_Float16)lo[3],
              (_Float16)hi[0], (_Float16)hi[1], (_Float16)hi[2], (_Float16)hi[3]};
}
// row n of a row-major f16 tile, columns c0 + {4g..4g+3, 16+4g..16+4g+3}
// (the same k permutation)
__device__ __forceinline__ h8 row_perm(const _Float16 *X, int pitch, int n, int g, int c0) {
    const h4 a = *(const h4 *)(X + n * pitch + c0 + 4 * g);
    const h4 b = *(const h4 *)(X + n * pitch + c0 + 16 + 4 * g);
    return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
    return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), CTRL, 0xF, 0xF, true));
}

// sums over the 16 lanes of the row of two values (interleaved chains)
__device__ __forceinline__ void row_sum16x2(float &x, float &y) {
    x += dpp<0xB1>(x);
    y += dpp<0xB1>(y);
    x += dpp<0x4E>(x);
    y += dpp<0x4E>(y);
    x += dpp<0x141>(x);
    y += dpp<0x141>(y);
    x += dpp<0x140>(x);
    y += dpp<0x140>(y);
}

// workgroup barrier that the instruction scheduler cannot move work across
// (s_barrier alone only orders memory operations)
__device__ __forceinline__ void phase_barrier() {
    __builtin_amdgcn_sched_barrier(0);
    __syncthreads();
    __builtin_amdgcn_sched_barrier(0);
}

template <typename Tin, typename Tout, bool ROPE>
__global__ __launch_bounds__(512, 1) void mlp_dual_kernel(MlpArgs a) {
    extern __shared__ __align__(16) unsigned char smem_raw[];
    Smem &sm = *reinterpret_cast<Smem *>(smem_raw);
    const int ch = blockIdx.x;
    const int bi = ch / a.H, hi = ch % a.H;
    const int w = threadIdx.x >> 6, l = threadIdx.x & 63, g = l >> 4, n = l & 15;
    const int NB = a.nblk;  // mini-batches; the last has a.tail tokens if a.tail > 0
    const bool lnw = w < 4; // LayerNorm waves 0..3 and staging waves 4..7: token row 4(w%4)+g, columns 4n..4n+3
    const int t = 4 * (w & 3) + g;

    // ---- state of hidden slice f in [32w, 32w+32) ----
    const int64_t cD = (int64_t)ch * kD;
    const float *W1g = a.W1 + cD * kF, *W2g = a.W2 + cD * kF;
    f32x4 W1s[2][4], W2s[2][4], b1t[2];
#pragma unroll
    for (int s = 0; s < 2; ++s) {
        const int f0 = 32 * w + 16 * s;
#pragma unroll
        for (int r = 0; r < 4; ++r)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                W1s[s][r][j] = W1g[(16 * r + 4 * g + j) * kF + f0 + n];   // W1[d][f]
                W2s[s][r][j] = W2g[(f0 + 4 * g + j) * kD + 16 * r + n];   // W2[f][d]
            }
        const float bv = a.b1[(int64_t)ch * kF + f0 + n];
        b1t[s] = f32x4{bv, bv, bv, bv};
    }
    if (threadIdx.x < kD) sm.b2[threadIdx.x] = a.b2[cD + threadIdx.x];

    // ---- per-column constants (LayerNorm, rotary at position t = row) ----
    for (int i = threadIdx.x; i < kD; i += 512) {
        const float gv = a.ln_w[hi * kD + i], bv = a.ln_b[hi * kD + i];
        sm.gam[i] = gv;
        sm.gam2[i] = gv * gv;
        sm.bet[i] = bv;
        sm.gb[i] = gv * bv;
    }
    for (int i = threadIdx.x; i < kM * kD; i += 512) {
        const int r = i / kD, c = i % kD;
        const double th = (double)r * pow((double)a.rope_base, -2.0 * (double)(c & 31) / (double)kD);
        sm.cs[r][c] = (float)cos(th);
        sm.sn[r][c] = (c < 32 ? -1.f : 1.f) * (float)sin(th);
    }
    const Tin *pq = (const Tin *)a.q.p + bi * a.q.sB + hi * a.q.sH + (int64_t)(a.t0 + t) * a.q.sL + 4 * n;
    const Tin *pk = (const Tin *)a.k.p + bi * a.k.sB + hi * a.k.sH + (int64_t)(a.t0 + t) * a.k.sL + 4 * n;
    const Tin *pv = (const Tin *)a.v.p + bi * a.v.sB + hi * a.v.sH + (int64_t)(a.t0 + t) * a.v.sL + 4 * n;
    const float *pe = a.eta + bi * a.eta_sB + hi * a.eta_sH + a.t0 + t;
    Tout *po = (Tout *)a.out.p + bi * a.out.sB + hi * a.out.sH + (int64_t)(a.t0 + t) * a.out.sL + 4 * n;

    // inputs of one mini-batch for this lane (raw), and the LayerNorm operands
    using Raw = typename std::conditional<std::is_same<Tin, __bf16>::value, uint2, uint4>::type;
    struct In {
        Raw q, k, v;
        float eta;
    };
    auto fetch = [&](In &x, int nb) {
        // rows past the last token (partial last mini-batch) read nothing and
        // get eta = 0, so they contribute no gradient
        const bool valid = !(nb == NB - 1 && a.tail > 0 && t >= a.tail);
        const int64_t tk = (int64_t)nb * kM;
        x.q = Raw{};
        x.k = Raw{};
        x.v = Raw{};
        x.eta = 0.f;
        if (valid) {
            x.q = *(const Raw *)(pq + tk * a.q.sL);
            x.k = *(const Raw *)(pk + tk * a.k.sL);
            x.v = *(const Raw *)(pv + tk * a.v.sL);
            x.eta = pe[tk];
        }
    };
    auto unpack = [](const Raw &u, float (&x)[4]) {
        if constexpr (std::is_same<Tin, __bf16>::value) {
            x[0] = __builtin_bit_cast(float, u.x << 16);
            x[1] = __builtin_bit_cast(float, u.x & 0xffff0000u);
            x[2] = __builtin_bit_cast(float, u.y << 16);
            x[3] = __builtin_bit_cast(float, u.y & 0xffff0000u);
        } else {
            x[0] = __builtin_bit_cast(float, u.x);
            x[1] = __builtin_bit_cast(float, u.y);
            x[2] = __builtin_bit_cast(float, u.z);
            x[3] = __builtin_bit_cast(float, u.w);
        }
    };
    // staging (waves 4..7): rotated q, k as fp16 rows; the LayerNorm operands
    // of the mini-batch into LDS for the LayerNorm waves
    auto stage = [&](const In &x, int buf) {
        float q[4], k[4], v[4];
        unpack(x.q, q);
        unpack(x.k, k);
        unpack(x.v, v);
        if constexpr (ROPE) {
            const f32x4 c4 = *(const f32x4 *)&sm.cs[t][4 * n], s4 = *(const f32x4 *)&sm.sn[t][4 * n];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float qo = dpp<0x128>(q[e]), ko = dpp<0x128>(k[e]);
                q[e] = q[e] * c4[e] + qo * s4[e];
                k[e] = k[e] * c4[e] + ko * s4[e];
            }
        }
        const h4 kh = h4{(_Float16)k[0], (_Float16)k[1], (_Float16)k[2], (_Float16)k[3]};
        *(h4 *)&sm.qs[buf][t][4 * n] = h4{(_Float16)q[0], (_Float16)q[1], (_Float16)q[2], (_Float16)q[3]};
        *(h4 *)&sm.xs[buf][t][4 * n] = kh;
        // K^T multiplies 2^8 ng1 in the W1 step: kept as 2^-8 K (exact scaling)
        const h4 khs = kh * (_Float16)kMatScale;
#pragma unroll
        for (int e = 0; e < 4; ++e) sm.kT[buf][4 * n + e][t] = khs[e];
        const f32x4 gm = *(const f32x4 *)&sm.gam[4 * n];
        const f32x4 bt = *(const f32x4 *)&sm.bet[4 * n], gbv = *(const f32x4 *)&sm.gb[4 * n];
        f32x4 ce, qr;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            ce[e] = x.eta * (gm[e] * (k[e] - v[e]) + gbv[e]);
            qr[e] = q[e] + bt[e];
        }
        *(f32x4 *)&sm.cel[buf][t][4 * n] = ce;
        *(f32x4 *)&sm.qres[buf][t][4 * n] = qr;
        if (n == 0) sm.eta[buf][t] = x.eta;
    };

    In pre;
    if (!lnw) fetch(pre, 0);
    phase_barrier();  // constants in LDS
    if (!lnw) {
        stage(pre, 0);
        if (NB > 1) fetch(pre, 1);
    }
    float gam2r[4];  // LayerNorm waves: gamma^2 at columns 4n .. 4n+3
#pragma unroll
    for (int e = 0; e < 4; ++e) gam2r[e] = sm.gam2[4 * n + e];
    // the ones of the bias steps, times 2^-8 (they multiply 2^8 ng1, 2^8 ng2)
    const h4 ones = h4{(_Float16)kMatScale, (_Float16)kMatScale, (_Float16)kMatScale, (_Float16)kMatScale};
    // token_eta of query row n, and of the last row (the committed step);
    // tn scales the causal matrices, which carry 2^-8
    const float tn = (a.te != nullptr ? a.te[n] : 1.f) * kMatScale;
    const float tl = a.te != nullptr ? a.te[kM - 1] : 1.f;
    const float tls = tl * kMatScale;
    const h4 onesl = h4{(_Float16)tls, (_Float16)tls, (_Float16)tls, (_Float16)tls};
    // the 16x16 identity as a B fragment (lane: I[4g+j][n])
    h4 ident;
#pragma unroll
    for (int j = 0; j < 4; ++j) ident[j] = (4 * g + j == n) ? (_Float16)1.f : (_Float16)0.f;
    const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
    phase_barrier();

    // operands of the last step, kept for an open last mini-batch (the K^T
    // and ng2 fragments are re-read from LDS, which keeps the last block's)
    h4 n1k[2], x2h[2];
    for (int nb = 0; nb < NB; ++nb) {
        const int buf = nb & 1;
        const bool open = (nb == NB - 1) && a.tail > 0;  // partial last mini-batch: keep W, emit grads

        // ---- P0: Z1, P1 = Q W1 + b1, GELU, M1, K^T fragments ----
        const h8 xp0 = row_perm(&sm.xs[buf][0][0], XP, n, g, 0), xp1 = row_perm(&sm.xs[buf][0][0], XP, n, g, 32);
        const h8 qp0 = row_perm(&sm.qs[buf][0][0], XP, n, g, 0), qp1 = row_perm(&sm.qs[buf][0][0], XP, n, g, 32);
        f32x4 X2[2], D1[2], P1[2];
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            const h8 wb0 = pair_b(W1s[s][0], W1s[s][1]), wb1 = pair_b(W1s[s][2], W1s[s][3]);
            const f32x4 z1 = mfma32(xp1, wb1, mfma32(xp0, wb0, b1t[s]));
            P1[s] = mfma32(qp1, wb1, mfma32(qp0, wb0, b1t[s]));
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const Gelu gg = gelu_both(z1[j]);
                X2[s][j] = gg.g;
                D1[s][j] = gg.dg;
                sm.x2[4 * g + j][32 * w + 16 * s + n] = (_Float16)X2[s][j];
            }
        }
        h4 M1;
        {
            const f32x4 st = mfma32(xp1, qp1, mfma32(xp0, qp0, zero));  // lane: S[query n][key 4g+j]
            f32x4 m;
#pragma unroll
            for (int j = 0; j < 4; ++j) m[j] = (4 * g + j <= n) ? fmaf(st[j], tn, tn) : 0.f;
            M1 = to_h4(m);
        }
        if (nb > 0 && threadIdx.x < kD) sm.b2[threadIdx.x] = sm.b2n[threadIdx.x];  // previous step
        // P1 reads only this wave's own columns of X2, written above: a
        // wave-local fence, no barrier (P1 writes the Z2 partials, which only
        // P2 reads, behind B2; the previous block's P5 reads the Zb2 partials)
        wave_lds_order();

        // ---- P1: partial Z2 over this hidden slice ----
        const h8 x2p = row_perm(&sm.x2[0][0], HP, n, g, 32 * w);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const f32x4 z2 = mfma32(x2p, pair_b(W2s[0][r], W2s[1][r]), zero);
#pragma unroll
            for (int j = 0; j < 4; ++j) sm.part[0][w][4 * g + j][16 * r + n] = z2[j];
        }
        phase_barrier();  // B2

        // ---- P2: Z2 = sum of slices + b2; LayerNorm backward -> ng2 ----
        if (lnw) {
            f32x4 z = *(const f32x4 *)&sm.b2[4 * n];
#pragma unroll
            for (int p = 0; p < 8; ++p) z += *(const f32x4 *)&sm.part[0][p][t][4 * n];
            const f32x4 cel = *(const f32x4 *)&sm.cel[buf][t][4 * n];
            const float eta = sm.eta[buf][t];
            // mean and mean square in one reduction round
            float s1 = (z[0] + z[1]) + (z[2] + z[3]);
            float s2 = fmaf(z[0], z[0], z[1] * z[1]) + fmaf(z[2], z[2], z[3] * z[3]);
            row_sum16x2(s1, s2);
            const float mu = s1 * (1.f / kD);
            const float var = fmaxf(fmaf(-mu, mu, s2 * (1.f / kD)), 0.f);
            const float rs = __builtin_amdgcn_rsqf(var + a.eps);  // var + eps >= eps > 0
            const float mrs = -mu * rs;
            float xh[4], u[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                xh[e] = fmaf(z[e], rs, mrs);
                u[e] = fmaf(eta * gam2r[e], xh[e], cel[e]);
            }
            float su = (u[0] + u[1]) + (u[2] + u[3]);
            float sux = fmaf(u[0], xh[0], u[1] * xh[1]) + fmaf(u[2], xh[2], u[3] * xh[3]);
            row_sum16x2(su, sux);
            su *= (1.f / kD);
            sux *= (1.f / kD);
            h4 ngh;
#pragma unroll
            for (int e = 0; e < 4; ++e) ngh[e] = (_Float16)(-kNgScale * rs * (u[e] - su - xh[e] * sux));  // 2^8 ng2
            *(h4 *)&sm.ng2[t][4 * n] = ngh;
#pragma unroll
            for (int e = 0; e < 4; ++e) sm.ng2T[4 * n + e][t] = ngh[e];
        } else if (nb + 1 < NB) {
            // stage the next mini-batch (its buffers were last read in P0, P2, P3
            // and P5 of nb-1, all before B2 of this block)
            stage(pre, buf ^ 1);
            if (nb + 2 < NB) fetch(pre, nb + 2);
        }
        phase_barrier();  // B3: ng2 in LDS, mini-batch nb+1 staged

        // ---- P3: ng1, Zb1, Xb2; step of W1, b1, b2 ----
        // ng2 as A fragments by column block r (lane: ng2[n][16r+4g+j]), and
        // as B fragments (lane: ng2[4g+j][16r+n]) from the transposed copy
        h4 nr[4], G2[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            nr[r] = *(const h4 *)&sm.ng2[n][16 * r + 4 * g];
            G2[r] = *(const h4 *)&sm.ng2T[16 * r + n][4 * g];
        }
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            // ng1 = (ng2 W2^T) o GELU'(Z1).  W2^T fragments come from this
            // wave's W2 tiles: a tile used as the A operand against the
            // identity gives its transpose in the B layout (exact in fp16)
            f32x4 g1 = zero;
#pragma unroll
            for (int r = 0; r < 4; ++r) g1 = mfma16(nr[r], to_h4(mfma16(to_h4(W2s[s][r]), ident, zero)), g1);
            f32x4 ng1;
#pragma unroll
            for (int j = 0; j < 4; ++j) ng1[j] = g1[j] * D1[s][j];
            const h4 n1 = to_h4(ng1);
            const f32x4 zb1 = mfma16(M1, n1, P1[s]);
#pragma unroll
            for (int j = 0; j < 4; ++j) sm.xb2[4 * g + j][32 * w + 16 * s + n] = (_Float16)gelu(zb1[j]);
            // X2^T multiplies 2^8 ng2 in the W2 step: kept as 2^-8 X2
            x2h[s] = to_h4(f32x4{X2[s][0] * kMatScale, X2[s][1] * kMatScale, X2[s][2] * kMatScale,
                                 X2[s][3] * kMatScale});
            n1k[s] = n1;
            if (!open) {
                // W1 += t X^T ng1, with K^T rows 16r .. 16r+15 as A fragments
                // (lane: K[4g+j][16r+n], from the transposed copy)
                const h4 n1t = a.te != nullptr ? to_h4(f32x4{ng1[0] * tl, ng1[1] * tl, ng1[2] * tl, ng1[3] * tl})
                                               : n1;
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    W1s[s][r] = mfma16(*(const h4 *)&sm.kT[buf][16 * r + n][4 * g], n1t, W1s[s][r]);
                b1t[s] = mfma16(ones, n1t, b1t[s]);
            }
        }
        if (w == 0) {
            // b2 after the step: b2 + t (column sums of ng2); an open block
            // keeps the unscaled sums (its accumulated gradient)
            const h4 ob = open ? ones : onesl;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float bv = sm.b2[16 * r + n];
                const f32x4 bn = mfma16(ob, G2[r], f32x4{bv, bv, bv, bv});
                if (g == 0) sm.b2n[16 * r + n] = bn[0];
            }
        }
        // P4 reads only this wave's own columns of Xb2 (and of X2), written by
        // this wave above: a wave's LDS accesses run in order, so no barrier,
        // only a fence that keeps the compiler from hoisting the reads
        wave_lds_order();

        // ---- P4: partial Zb2 over this hidden slice, with this slice's part
        // of the causal term: tril(Xb2 X2^T + 1) ng2 is the sum over the
        // slices of tril(Xb2_s X2_s^T) ng2, plus tril(1) ng2 (wave 0) ----
        {
            const h8 xb2p = row_perm(&sm.xb2[0][0], HP, n, g, 32 * w);
            const h8 x2p = row_perm(&sm.x2[0][0], HP, n, g, 32 * w);
            const f32x4 st = mfma32(x2p, xb2p, zero);  // lane: S[query n][key 4g+j] over the slice
            f32x4 mm;
#pragma unroll
            for (int j = 0; j < 4; ++j) mm[j] = (4 * g + j <= n) ? fmaf(st[j], tn, w == 0 ? tn : 0.f) : 0.f;
            const h4 M2 = to_h4(mm);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const f32x4 z = mfma16(M2, G2[r], mfma32(xb2p, pair_b(W2s[0][r], W2s[1][r]), zero));
                const float b2v = w == 0 ? sm.b2[16 * r + n] : 0.f;  // b2 (current) rides in slice 0
#pragma unroll
                for (int j = 0; j < 4; ++j) sm.part[1][w][4 * g + j][16 * r + n] = z[j] + b2v;
            }
        }
        // step of W2 (W2 += t X2^T ng2), after its last use at the block start
        if (!open) {
#pragma unroll
            for (int s = 0; s < 2; ++s) {
                const h4 x2t = a.te != nullptr
                                   ? to_h4(f32x4{X2[s][0] * tls, X2[s][1] * tls, X2[s][2] * tls, X2[s][3] * tls})
                                   : x2h[s];
#pragma unroll
                for (int r = 0; r < 4; ++r) W2s[s][r] = mfma16(x2t, G2[r], W2s[s][r]);
            }
        }
        phase_barrier();  // B5

        // ---- P5 (LayerNorm waves): Zb2, out = q + LN(Zb2) ----
        if (lnw) {
            f32x4 z = *(const f32x4 *)&sm.part[1][0][t][4 * n];  // includes b2
#pragma unroll
            for (int p = 1; p < kParts; ++p) z += *(const f32x4 *)&sm.part[1][p][t][4 * n];
            const f32x4 qres = *(const f32x4 *)&sm.qres[buf][t][4 * n];
            float s1 = (z[0] + z[1]) + (z[2] + z[3]);
            float s2 = fmaf(z[0], z[0], z[1] * z[1]) + fmaf(z[2], z[2], z[3] * z[3]);
            row_sum16x2(s1, s2);
            const float mu = s1 * (1.f / kD);
            const float var = fmaxf(fmaf(-mu, mu, s2 * (1.f / kD)), 0.f);
            const float rs = __builtin_amdgcn_rsqf(var + a.eps);  // var + eps >= eps > 0
            const f32x4 gm = *(const f32x4 *)&sm.gam[4 * n];
            float y[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) y[e] = (z[e] - mu) * (rs * gm[e]) + qres[e];
            const bool valid = !(open && t >= a.tail);
            if (valid) {
                Tout *o = po + (int64_t)nb * kM * a.out.sL;
                if constexpr (std::is_same<Tout, float>::value) {
                    *(float4 *)o = float4{y[0], y[1], y[2], y[3]};
                } else {
                    typedef __bf16 b4 __attribute__((ext_vector_type(4)));
                    *(b4 *)o = b4{(__bf16)y[0], (__bf16)y[1], (__bf16)y[2], (__bf16)y[3]};
                }
            }
        }
        // no barrier here: the LayerNorm waves' P5 overlaps the other waves' P0
        // and P1 of the next block, which write none of what P5 reads (the Zb2
        // partials are next written in P4, behind B2; b2 rides in slice 0)
    }

    // ---- final state (an open last mini-batch left W, b at its start) ----
    const bool open_end = a.tail > 0;
    if (open_end) {
        // the pages' accumulated gradients of the open mini-batch: -step
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            const int f0 = 32 * w + 16 * s;
            float *g1p = a.W1g + cD * kF + (4 * g) * kF + f0 + n;
            float *g2p = a.W2g + cD * kF + (f0 + 4 * g) * kD + n;
            const int lb = (NB - 1) & 1;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const h4 kt = *(const h4 *)&sm.kT[lb][16 * r + n][4 * g];
                const h4 g2 = *(const h4 *)&sm.ng2T[16 * r + n][4 * g];
                const f32x4 d1 = mfma16(kt, n1k[s], zero), d2 = mfma16(x2h[s], g2, zero);
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    g1p[(16 * r + j) * kF] = -d1[j];
                    g2p[j * kD + 16 * r] = -d2[j];
                }
            }
            const f32x4 db = mfma16(ones, n1k[s], zero);
            if (g == 0) a.b1g[(int64_t)ch * kF + f0 + n] = -db[0];
        }
    }
    if (threadIdx.x < kD) {
        const int d = threadIdx.x;
        // closed: b2 after the last step; open: b2 at the open block's start
        a.b2[cD + d] = open_end ? sm.b2[d] : sm.b2n[d];
        if (open_end) a.b2g[cD + d] = -(sm.b2n[d] - sm.b2[d]);
    }
    float *W1o = a.W1 + cD * kF, *W2o = a.W2 + cD * kF;
#pragma unroll
    for (int s = 0; s < 2; ++s) {
        const int f0 = 32 * w + 16 * s;
#pragma unroll
        for (int r = 0; r < 4; ++r)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                W1o[(16 * r + 4 * g + j) * kF + f0 + n] = W1s[s][r][j];
                W2o[(f0 + 4 * g + j) * kD + 16 * r + n] = W2s[s][r][j];
            }
        if (g == 0) a.b1[(int64_t)ch * kF + f0 + n] = b1t[s][0];
    }
}

template <typename Tin, typename Tout, bool ROPE>
hipError_t launch_typed(const MlpArgs &a, hipStream_t s) {
    const void *fn = (const void *)&mlp_dual_kernel<Tin, Tout, ROPE>;
    static std::atomic<uint64_t> configured{0};  // per instantiation: devices whose LDS limit is raised
    if (hipError_t e = ensure_lds_limit(fn, sizeof(Smem), configured); e != hipSuccess) return e;
    hipLaunchKernelGGL((mlp_dual_kernel<Tin, Tout, ROPE>), dim3(a.B * a.H), dim3(512), sizeof(Smem), s, a);
    return hipGetLastError();
}

template <typename Tin, typename Tout>
hipError_t launch_rope(const MlpArgs &a, hipStream_t s) {
    return a.rope ? launch_typed<Tin, Tout, true>(a, s) : launch_typed<Tin, Tout, false>(a, s);
}

}  // namespace

// bf16 inputs only (the fp16 operand rounding is sized for them)
hipError_t launch_mlp_dual(const MlpArgs &a, int in_bf16, int out_bf16, hipStream_t s) {
    if (!in_bf16) return hipErrorInvalidValue;
    return out_bf16 ? launch_rope<__bf16, __bf16>(a, s) : launch_rope<__bf16, float>(a, s);
}

}  // namespace ttt
