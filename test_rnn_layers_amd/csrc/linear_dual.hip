// linear_dual.hip -- TTT-Linear over whole mini-batches in the dual form
// ("代码连连看——TTT", compute_mini_batch, dual branch; "TTTLinear.ttt": the
// scan over mini-batches carrying W, b).
//
// Per mini-batch n of 16 tokens (rows of Q_n, K_n, V_n; eta_j per key token):
//   Z_n    = K_n W_n + b_n                          (16x64x64)
//   g      = d/dZ of 1/2 ||LN(Z_n) - (V_n - K_n)||^2, row by row
//   ng_n   = -eta_j g_j                             (rows scaled and negated)
//   Zbar_n = Q_n W_n + b_n + tril(Q_n K_n^T + 1) ng_n
//            (the pages' Attn1 and b1_bar folded into one 16x16x64 product)
//   out_n  = Q_n + LN(Zbar_n)
//   W_n+1  = W_n + K_n^T ng_n ,  b_n+1 = b_n + 1^T ng_n   (W1_last, b1_last)
//
// Design (gfx950, one persistent workgroup of 4 waves per (batch, head)):
//  * Wave w owns the 64x16 column slab W[:, 16w..16w+15] as four MFMA
//    accumulator tiles (fp32) for the whole chain, and b as a fifth tile whose
//    rows all hold b.  Every product keeps that slab as its B operand.
//  * Look-ahead: Z_n+1 = K_n+1 W_n + b_n + (K_n+1 K_n^T + 1) ng_n.  The first
//    term (Y_n+1) is formed while mini-batch n is still in flight, so the
//    sequential chain per mini-batch is one 16x16x16 product, a LayerNorm
//    backward and two barriers.
//  * Row-wise LayerNorm work: 16 lanes per row, 4 columns per lane, row sums
//    with DPP butterflies; results cross between the row and the column
//    layouts through LDS (Z, Zbar out; ng back as MFMA B fragments).
//  * Operands: bf16 inputs run the products on fp16 MFMA (inputs, the W slab,
//    ng and the 16x16 matrices rounded to fp16, fp32 accumulation; ~2^-11
//    relative per operand); fp32 inputs run them on fp32 MFMA.
//  * Inputs stream through a 4-deep LDS ring; each thread fetches its share
//    of a mini-batch 3 mini-batches ahead into registers.
#include <type_traits>

#include "device_common.hpp"
#include "launch.hpp"

namespace ttt {
namespace {

constexpr int kM = 16;     // mini-batch size of this kernel
constexpr int kRing = 4;   // LDS stages: n-1, n, n+1, n+2
constexpr int kAhead = 3;  // register prefetch depth (mini-batches)
constexpr int kFP = 68;    // fp32 row pitch (16 B aligned, skews banks)

typedef _Float16 h4 __attribute__((ext_vector_type(4)));
typedef _Float16 h8 __attribute__((ext_vector_type(8)));

// ---------------------------------------------------------------------------
// operand policies
// ---------------------------------------------------------------------------
template <typename T>
struct Op;

// fp16 operands: 16x16x32 (k = 64 products, two steps) and 16x16x16 MFMAs.
template <>
struct Op<_Float16> {
    static constexpr int XP = 72;  // row pitch of X tiles (144 B)
    static constexpr int TP = 24;  // token pitch of the transposed K tile
    using F4 = h4;
    struct XF {
        h8 v[2];
    };
    using WF = XF;
    // Row n of a 16x64 tile with the k permutation matching the accumulator
    // layout of W: slot 8g+i <- column 32s + 4g + i (i < 4), 32s + 16 + 4g + i-4.
    __device__ static XF load_x(const _Float16 *X, int n, int g) {
        XF x;
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            const h4 a = *(const h4 *)(X + n * XP + 32 * s + 4 * g);
            const h4 b = *(const h4 *)(X + n * XP + 32 * s + 16 + 4 * g);
            x.v[s] = __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
        }
        return x;
    }
    __device__ static WF cvt_w(const f32x4 (&Wt)[4]) {
        WF w;
#pragma unroll
        for (int s = 0; s < 2; ++s)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                w.v[s][i] = (_Float16)Wt[2 * s][i];
                w.v[s][4 + i] = (_Float16)Wt[2 * s + 1][i];
            }
        return w;
    }
    __device__ static f32x4 xx(const XF &a, const XF &b, f32x4 acc) {
#pragma unroll
        for (int s = 0; s < 2; ++s) acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(a.v[s], b.v[s], acc, 0, 0, 0);
        return acc;
    }
    __device__ static f32x4 mma16(F4 a, F4 b, f32x4 acc) {
        return __builtin_amdgcn_mfma_f32_16x16x16f16(a, b, acc, 0, 0, 0);
    }
    __device__ static F4 make(float x0, float x1, float x2, float x3) {
        return F4{(_Float16)x0, (_Float16)x1, (_Float16)x2, (_Float16)x3};
    }
    __device__ static void put(_Float16 *p, float x) { *p = (_Float16)x; }
    __device__ static void put2(_Float16 *p, float x0, float x1) {
        typedef _Float16 h2 __attribute__((ext_vector_type(2)));
        *(h2 *)p = h2{(_Float16)x0, (_Float16)x1};
    }
};

// fp32 operands: 16x16x4 fp32 MFMAs (A lane (g,n) holds A[n][g], B holds B[g][n]).
template <>
struct Op<float> {
    static constexpr int XP = 68;
    static constexpr int TP = 20;
    using F4 = f32x4;
    struct XF {
        f32x4 v[4];  // v[r][j] = X[n][16r + 4g + j]
    };
    using WF = XF;
    __device__ static XF load_x(const float *X, int n, int g) {
        XF x;
#pragma unroll
        for (int r = 0; r < 4; ++r) x.v[r] = *(const f32x4 *)(X + n * XP + 16 * r + 4 * g);
        return x;
    }
    __device__ static WF cvt_w(const f32x4 (&Wt)[4]) {
        WF w;
#pragma unroll
        for (int r = 0; r < 4; ++r) w.v[r] = Wt[r];
        return w;
    }
    // contraction index d = 16r + 4g + j: step (r, j) pairs A = X[n][d], B = W[d][n']
    __device__ static f32x4 xx(const XF &a, const XF &b, f32x4 acc) {
#pragma unroll
        for (int r = 0; r < 4; ++r)
#pragma unroll
            for (int j = 0; j < 4; ++j) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.v[r][j], b.v[r][j], acc, 0, 0, 0);
        return acc;
    }
    // contraction over tokens 4g + j
    __device__ static f32x4 mma16(F4 a, F4 b, f32x4 acc) {
#pragma unroll
        for (int j = 0; j < 4; ++j) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[j], b[j], acc, 0, 0, 0);
        return acc;
    }
    __device__ static F4 make(float x0, float x1, float x2, float x3) { return F4{x0, x1, x2, x3}; }
    __device__ static void put(float *p, float x) { *p = x; }
    __device__ static void put2(float *p, float x0, float x1) { *(float2 *)p = float2{x0, x1}; }
};

// ---------------------------------------------------------------------------
// LDS
// ---------------------------------------------------------------------------
template <typename T>
struct Stage {
    T kx[kM][Op<T>::XP];        // K rows (rotated), operand type
    T qx[kM][Op<T>::XP];        // Q rows (rotated)
    T kt[kD][Op<T>::TP];        // K transposed: kt[d][token]
    float cel[kM][kFP];         // gamma * (beta - v + k), per element
    float qres[kM][kFP];        // q + beta
    float eta[kM];
};

template <typename T>
struct Smem {
    Stage<T> st[kRing];
    float zbuf[kM][kFP];                 // Z_n (column layout in, row layout out)
    float zbbuf[kM][kFP];                // Zbar_n-1
    typename Op<T>::F4 gop[kD][4];       // ng as B fragments: [column][token group]
    typename Op<T>::F4 mop[64];          // tril(Q K^T + 1) as A fragments, per lane
    typename Op<T>::F4 cop[64];          // K_n+1 K_n^T + 1 as A fragments, per lane
};

// ---------------------------------------------------------------------------
// row reductions over the 16 lanes of a DPP row (all lanes get the sum)
// ---------------------------------------------------------------------------
template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
    return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), CTRL, 0xF, 0xF, true));
}
__device__ __forceinline__ float row_sum16(float x) {
    x += dpp<0xB1>(x);   // quad_perm [1,0,3,2]
    x += dpp<0x4E>(x);   // quad_perm [2,3,0,1]
    x += dpp<0x141>(x);  // row_half_mirror
    x += dpp<0x140>(x);  // row_mirror
    return x;
}

// ---------------------------------------------------------------------------
// per-thread share of one mini-batch's inputs: row tid/16, columns
// c0 = 2*(tid%16), c0+1 and c0+32, c0+33 of each of q, k, v
// ---------------------------------------------------------------------------
template <typename Tin>
struct Pref;
template <>
struct Pref<__bf16> {
    uint32_t q[2], k[2], v[2];  // two bf16 each
    float eta;
    __device__ static void unpack(uint32_t u, float &a, float &b) {
        a = __builtin_bit_cast(float, u << 16);
        b = __builtin_bit_cast(float, u & 0xffff0000u);
    }
};
template <>
struct Pref<float> {
    float2 q[2], k[2], v[2];
    float eta;
    __device__ static void unpack(float2 u, float &a, float &b) {
        a = u.x;
        b = u.y;
    }
};

template <typename Tin>
struct InPtr {
    const Tin *q, *k, *v;  // at (b, h, token t0, column c0) of this thread
    const float *eta;      // at (b, h, token t0)
    int64_t sq, sk, sv;    // token strides
};

template <typename Tin>
__device__ __forceinline__ void fetch(Pref<Tin> &p, const InPtr<Tin> &ip, int blk, int row, int tid) {
    using U = decltype(p.q[0]);
    using UU = typename std::remove_reference<U>::type;
    const int64_t t = (int64_t)blk * kM + row;
    const Tin *q = ip.q + t * ip.sq, *k = ip.k + t * ip.sk, *v = ip.v + t * ip.sv;
    p.q[0] = *(const UU *)q;
    p.q[1] = *(const UU *)(q + 32);
    p.k[0] = *(const UU *)k;
    p.k[1] = *(const UU *)(k + 32);
    p.v[0] = *(const UU *)v;
    p.v[1] = *(const UU *)(v + 32);
    if (tid < kM) p.eta = ip.eta[(int64_t)blk * kM + tid];
}

// per-thread constants of the staging step (its 4 columns and its row)
struct StageConst {
    float cs[2], sn[2];     // rotary cos/sin at position `row` for columns c0, c0+1
    float gam[4], gb[4];    // gamma, gamma*beta for c0, c0+1, c0+32, c0+33
    float bet[4];
};

template <typename Tin, typename T>
__device__ __forceinline__ void stage(Stage<T> &S, const Pref<Tin> &p, const StageConst &sc, int rope, int row,
                                      int c0, int tid) {
    float q[4], k[4], v[4];
    Pref<Tin>::unpack(p.q[0], q[0], q[1]);
    Pref<Tin>::unpack(p.q[1], q[2], q[3]);
    Pref<Tin>::unpack(p.k[0], k[0], k[1]);
    Pref<Tin>::unpack(p.k[1], k[2], k[3]);
    Pref<Tin>::unpack(p.v[0], v[0], v[1]);
    Pref<Tin>::unpack(p.v[1], v[2], v[3]);
    if (rope) {
        // pairs (c, c + 32): first half x*cos - x'*sin, second half x'*cos + x*sin
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const float q1 = q[i] * sc.cs[i] - q[i + 2] * sc.sn[i];
            const float q2 = q[i + 2] * sc.cs[i] + q[i] * sc.sn[i];
            const float k1 = k[i] * sc.cs[i] - k[i + 2] * sc.sn[i];
            const float k2 = k[i + 2] * sc.cs[i] + k[i] * sc.sn[i];
            q[i] = q1;
            q[i + 2] = q2;
            k[i] = k1;
            k[i + 2] = k2;
        }
    }
    Op<T>::put2(&S.qx[row][c0], q[0], q[1]);
    Op<T>::put2(&S.qx[row][c0 + 32], q[2], q[3]);
    Op<T>::put2(&S.kx[row][c0], k[0], k[1]);
    Op<T>::put2(&S.kx[row][c0 + 32], k[2], k[3]);
    Op<T>::put(&S.kt[c0][row], k[0]);
    Op<T>::put(&S.kt[c0 + 1][row], k[1]);
    Op<T>::put(&S.kt[c0 + 32][row], k[2]);
    Op<T>::put(&S.kt[c0 + 33][row], k[3]);
    float ce[4], qr[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        ce[e] = sc.gam[e] * (k[e] - v[e]) + sc.gb[e];
        qr[e] = q[e] + sc.bet[e];
    }
    *(float2 *)&S.cel[row][c0] = float2{ce[0], ce[1]};
    *(float2 *)&S.cel[row][c0 + 32] = float2{ce[2], ce[3]};
    *(float2 *)&S.qres[row][c0] = float2{qr[0], qr[1]};
    *(float2 *)&S.qres[row][c0 + 32] = float2{qr[2], qr[3]};
    if (tid < kM) S.eta[tid] = p.eta;
}

// causal matrix tril(S + 1) from S^T in accumulator layout (lane: query n, keys 4g+j)
__device__ __forceinline__ f32x4 causal(f32x4 st, int n, int g) {
    f32x4 m;
#pragma unroll
    for (int j = 0; j < 4; ++j) m[j] = (4 * g + j <= n) ? st[j] + 1.f : 0.f;
    return m;
}

template <typename Tin, typename Tout, typename T>
__global__ __launch_bounds__(256, 1) void linear_dual_kernel(LinearArgs a) {
    using O = Op<T>;
    using F4 = typename O::F4;
    using XF = typename O::XF;
    extern __shared__ __align__(16) unsigned char smem_raw[];
    Smem<T> &sm = *reinterpret_cast<Smem<T> *>(smem_raw);

    const int ch = blockIdx.x;
    const int bi = ch / a.H, hi = ch % a.H;
    const int tid = threadIdx.x;
    const int w = tid >> 6, l = tid & 63, g = l >> 4, n = l & 15;
    const int N = a.ntok;  // whole mini-batches

    // ---- per-thread constants ----
    const int srow = tid >> 4, c0 = 2 * (tid & 15);
    StageConst sc;
    {
        const int cols[4] = {c0, c0 + 1, c0 + 32, c0 + 33};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            sc.gam[e] = a.ln_w[hi * kD + cols[e]];
            sc.bet[e] = a.ln_b[hi * kD + cols[e]];
            sc.gb[e] = sc.gam[e] * sc.bet[e];
        }
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            // blocks are aligned: position mod 16 == row
            const double th = (double)srow * pow((double)a.rope_base, -2.0 * (double)(c0 + i) / (double)kD);
            sc.cs[i] = (float)cos(th);
            sc.sn[i] = (float)sin(th);
        }
    }
    // row-phase constants: row 4w + g, columns 4n .. 4n+3
    const int rrow = 4 * w + g;
    float rg[4], rg2[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        rg[e] = a.ln_w[hi * kD + 4 * n + e];
        rg2[e] = rg[e] * rg[e];
    }

    InPtr<Tin> ip;
    ip.q = (const Tin *)a.q.p + bi * a.q.sB + hi * a.q.sH + (int64_t)a.t0 * a.q.sL + c0;
    ip.k = (const Tin *)a.k.p + bi * a.k.sB + hi * a.k.sH + (int64_t)a.t0 * a.k.sL + c0;
    ip.v = (const Tin *)a.v.p + bi * a.v.sB + hi * a.v.sH + (int64_t)a.t0 * a.v.sL + c0;
    ip.eta = a.eta + bi * a.eta_sB + hi * a.eta_sH + a.t0;
    ip.sq = a.q.sL;
    ip.sk = a.k.sL;
    ip.sv = a.v.sL;
    Tout *op = (Tout *)a.out.p + bi * a.out.sB + hi * a.out.sH + (int64_t)a.t0 * a.out.sL + 4 * n;

    // ---- state: W slab (rows 16r + 4g + j, column 16w + n), bias tile ----
    f32x4 Wt[4], Bt;
    {
        const float *Wc = a.W + (int64_t)ch * kD * kD;
#pragma unroll
        for (int r = 0; r < 4; ++r)
#pragma unroll
            for (int j = 0; j < 4; ++j) Wt[r][j] = Wc[(16 * r + 4 * g + j) * kD + 16 * w + n];
        const float bv = a.b[(int64_t)ch * kD + 16 * w + n];
        Bt = f32x4{bv, bv, bv, bv};
    }
    const F4 ones = O::make(1.f, 1.f, 1.f, 1.f);

    // ---- prologue: mini-batches 0 and 1 staged, 2 .. 2+kAhead-1 in flight ----
    Pref<Tin> pf[kAhead];
    {
        Pref<Tin> p0, p1;
        fetch(p0, ip, 0, srow, tid);
        if (N > 1) fetch(p1, ip, 1, srow, tid);
#pragma unroll
        for (int i = 0; i < kAhead; ++i)
            if (2 + i < N) fetch(pf[(2 + i) % kAhead], ip, 2 + i, srow, tid);
        stage<Tin, T>(sm.st[0], p0, sc, a.rope, srow, c0, tid);
        if (N > 1) stage<Tin, T>(sm.st[1], p1, sc, a.rope, srow, c0, tid);
    }
    __syncthreads();

    f32x4 Y, P;  // Y_n+1 = K_n+1 W_n + b_n ; P_n = Q_n W_n + b_n

    // Column phase of mini-batch n: P_n, Y_n+1, and (waves 0/1) the 16x16
    // matrices of mini-batch n.  Z_0 is written here when n == 0.
    auto column_products = [&](int nb) {
        const Stage<T> &S = sm.st[nb % kRing];
        const typename O::WF wf = O::cvt_w(Wt);
        const XF qx = O::load_x(&S.qx[0][0], n, g);
        P = O::xx(qx, wf, Bt);
        if (nb == 0) {
            const XF kx = O::load_x(&S.kx[0][0], n, g);
            const f32x4 Z0 = O::xx(kx, wf, Bt);
#pragma unroll
            for (int j = 0; j < 4; ++j) sm.zbuf[4 * g + j][16 * w + n] = Z0[j];
        }
        if (nb + 1 < N) {
            const XF kx1 = O::load_x(&sm.st[(nb + 1) % kRing].kx[0][0], n, g);
            Y = O::xx(kx1, wf, Bt);
        }
        if (w == 0) {
            // S^T[key m][query n'] = k_m . q_n'  ->  lane holds S[n][4g+j]
            const XF kx = O::load_x(&S.kx[0][0], n, g);
            const f32x4 st = O::xx(kx, qx, f32x4{0.f, 0.f, 0.f, 0.f});
            const f32x4 m = causal(st, n, g);
            sm.mop[l] = O::make(m[0], m[1], m[2], m[3]);
        } else if (w == 1 && nb + 1 < N) {
            // C[query i of n+1][key j of n] = k_n+1,i . k_n,j + 1
            const XF kx = O::load_x(&S.kx[0][0], n, g);
            const XF kx1 = O::load_x(&sm.st[(nb + 1) % kRing].kx[0][0], n, g);
            const f32x4 c = O::xx(kx, kx1, f32x4{1.f, 1.f, 1.f, 1.f});
            sm.cop[l] = O::make(c[0], c[1], c[2], c[3]);
        }
    };

    // Row phase, LayerNorm backward of Z_nb: ng = -eta * dL/dZ into gop.
    auto ln_backward = [&](int nb) {
        const Stage<T> &S = sm.st[nb % kRing];
        const f32x4 z = *(const f32x4 *)&sm.zbuf[rrow][4 * n];
        const f32x4 ce = *(const f32x4 *)&S.cel[rrow][4 * n];
        const float eta = S.eta[rrow];
        const float mu = row_sum16(z[0] + z[1] + z[2] + z[3]) * (1.f / kD);
        f32x4 d;
#pragma unroll
        for (int e = 0; e < 4; ++e) d[e] = z[e] - mu;
        const float var = row_sum16(d[0] * d[0] + d[1] * d[1] + d[2] * d[2] + d[3] * d[3]) * (1.f / kD);
        const float rs = rsqrtf(var + a.eps);
        f32x4 xh, u;
        float su = 0.f, sux = 0.f;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            xh[e] = d[e] * rs;
            u[e] = rg2[e] * xh[e] + ce[e];  // gamma * (LN(z) - (v - k))
            su += u[e];
            sux += u[e] * xh[e];
        }
        su = row_sum16(su) * (1.f / kD);
        sux = row_sum16(sux) * (1.f / kD);
        // ng = -eta * rs * (u - mean(u) - xh * mean(u xh))
        const float A = -eta * rs;
        const float C0 = -A * su, C1 = -A * sux;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const float ng = u[e] * A + (xh[e] * C1 + C0);
            // token rrow = 4w + g: fragment (column 4n+e, token group w), element g
            O::put(reinterpret_cast<T *>(&sm.gop[4 * n + e][w]) + g, ng);
        }
    };

    // Row phase, LayerNorm forward of Zbar_nb: out = q + LN(Zbar).
    auto ln_forward = [&](int nb) {
        const Stage<T> &S = sm.st[nb % kRing];
        const f32x4 zb = *(const f32x4 *)&sm.zbbuf[rrow][4 * n];
        const f32x4 qr = *(const f32x4 *)&S.qres[rrow][4 * n];
        const float mu = row_sum16(zb[0] + zb[1] + zb[2] + zb[3]) * (1.f / kD);
        f32x4 d;
#pragma unroll
        for (int e = 0; e < 4; ++e) d[e] = zb[e] - mu;
        const float var = row_sum16(d[0] * d[0] + d[1] * d[1] + d[2] * d[2] + d[3] * d[3]) * (1.f / kD);
        const float rs = rsqrtf(var + a.eps);
        Tout *o = op + (int64_t)(nb * kM + rrow) * a.out.sL;
        float y[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) y[e] = d[e] * (rs * rg[e]) + qr[e];
        if constexpr (std::is_same<Tout, float>::value) {
            *(f32x4 *)o = f32x4{y[0], y[1], y[2], y[3]};
        } else {
            typedef __bf16 b4 __attribute__((ext_vector_type(4)));
            *(b4 *)o = b4{(__bf16)y[0], (__bf16)y[1], (__bf16)y[2], (__bf16)y[3]};
        }
    };

    // Column phase 1 of mini-batch nb (nb >= 1): consume ng_nb-1.
    auto apply_step = [&](int nb, bool last) {
        const Stage<T> &Sp = sm.st[(nb - 1) % kRing];
        const F4 gf = sm.gop[16 * w + n][g];
        if (!last) {
            const f32x4 Z = O::mma16(sm.cop[l], gf, Y);
#pragma unroll
            for (int j = 0; j < 4; ++j) sm.zbuf[4 * g + j][16 * w + n] = Z[j];
        }
        const f32x4 ZB = O::mma16(sm.mop[l], gf, P);
#pragma unroll
        for (int j = 0; j < 4; ++j) sm.zbbuf[4 * g + j][16 * w + n] = ZB[j];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const F4 kt = *(const F4 *)&Sp.kt[16 * r + n][4 * g];
            Wt[r] = O::mma16(kt, gf, Wt[r]);
        }
        Bt = O::mma16(ones, gf, Bt);
    };

    auto stage_ahead = [&](int nb, Pref<Tin> &pr) {
        // stage mini-batch nb + 2 from registers, fetch nb + 2 + kAhead
        if (nb + 2 < N) {
            stage<Tin, T>(sm.st[(nb + 2) % kRing], pr, sc, a.rope, srow, c0, tid);
            if (nb + 2 + kAhead < N) fetch(pr, ip, nb + 2 + kAhead, srow, tid);
        }
    };

    // ---- mini-batch 0: Z_0 directly, then its LayerNorm backward ----
    column_products(0);
    __syncthreads();
    ln_backward(0);
    stage_ahead(0, pf[2 % kAhead]);
    __syncthreads();

    // ---- steady state ----
    auto iteration = [&](int nb, Pref<Tin> &pr) {
        apply_step(nb, false);  // Z_nb, Zbar_nb-1, W_nb, b_nb
        __syncthreads();
        column_products(nb);    // P_nb, Y_nb+1, M_nb, C_nb
        ln_backward(nb);        // ng_nb
        ln_forward(nb - 1);     // out_nb-1
        stage_ahead(nb, pr);
        __syncthreads();
    };
    // register set of mini-batch m is pf[m % kAhead]; nb = 1 + kAhead*i here
    static_assert(kAhead == 3, "the unrolled loop below names the register sets");
    int nb = 1;
    for (; nb + kAhead <= N; nb += kAhead) {
        iteration(nb, pf[0]);
        iteration(nb + 1, pf[1]);
        iteration(nb + 2, pf[2]);
    }
    // fewer than kAhead mini-batches left: nb >= N - 2, nothing left to stage
    for (; nb < N; ++nb) {
        apply_step(nb, false);
        __syncthreads();
        column_products(nb);
        ln_backward(nb);
        ln_forward(nb - 1);
        __syncthreads();
    }

    // ---- epilogue: Zbar of the last mini-batch, final step ----
    apply_step(N, true);
    __syncthreads();
    ln_forward(N - 1);

    float *Wo = a.W + (int64_t)ch * kD * kD;
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int j = 0; j < 4; ++j) Wo[(16 * r + 4 * g + j) * kD + 16 * w + n] = Wt[r][j];
    if (g == 0) a.b[(int64_t)ch * kD + 16 * w + n] = Bt[0];
}

template <typename Tin, typename Tout, typename T>
hipError_t launch_typed(const LinearArgs &a, hipStream_t s) {
    const void *fn = (const void *)&linear_dual_kernel<Tin, Tout, T>;
    const size_t lds = sizeof(Smem<T>);
    static bool configured = false;  // per instantiation
    if (!configured) {
        hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
        configured = true;
    }
    hipLaunchKernelGGL((linear_dual_kernel<Tin, Tout, T>), dim3(a.B * a.H), dim3(256), lds, s, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_linear_dual(const LinearArgs &a, int in_bf16, int out_bf16, hipStream_t s) {
    if (in_bf16 && out_bf16) return launch_typed<__bf16, __bf16, _Float16>(a, s);
    if (in_bf16) return launch_typed<__bf16, float, _Float16>(a, s);
    if (out_bf16) return launch_typed<float, __bf16, float>(a, s);
    return launch_typed<float, float, float>(a, s);
}

}  // namespace ttt
