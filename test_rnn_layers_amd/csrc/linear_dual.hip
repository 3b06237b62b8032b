// linear_dual.hip -- TTT-Linear over whole mini-batches in the dual form
// ("代码连连看——TTT", compute_mini_batch, dual branch; "TTTLinear.ttt": the
// scan over mini-batches carrying W, b).
//
// Per mini-batch n of 16 tokens (rows of Q_n, K_n, V_n; eta_j per key token;
// t_i = token_eta of row i, t = t_15 the last row's):
//   Z_n    = K_n W_n + b_n                          (16x64x64)
//   g      = d/dZ of 1/2 ||LN(Z_n) - (V_n - K_n)||^2, row by row
//   ng_n   = -eta_j g_j                             (rows scaled and negated)
//   Zbar_n = Q_n W_n + b_n + diag(t_i) tril(Q_n K_n^T + 1) ng_n
//            (the pages' Attn1 and b1_bar folded into one 16x16x64 product,
//            their [K, K] eta being t_i eta_j)
//   out_n  = Q_n + LN(Zbar_n)
//   W_n+1  = W_n + t K_n^T ng_n ,  b_n+1 = b_n + t 1^T ng_n  (W1_last, b1_last)
//
// Design (gfx950, one persistent workgroup of 8 waves per (batch, head)):
//  * Column waves 0..3: wave c owns the 64x16 slab W[:, 16c..16c+15] as four
//    fp32 MFMA accumulator tiles for the whole chain (and b as a tile whose
//    rows all hold b) and runs every product of the step.
//  * Row waves 4..7: 16 lanes per token row, 4 columns per lane.  They fetch
//    the inputs of mini-batch n+6, stage n+2 into LDS as MFMA row fragments,
//    keep the LayerNorm target and the residual in registers, and run the
//    LayerNorm backward (-> ng, to LDS as MFMA B fragments) and forward
//    (-> out, stored to HBM) with DPP row reductions.
//  * Look-ahead on the sequential chain:
//      Z_n+1 = K_n+1 W_n + b_n + t (K_n+1 K_n^T + 1) ng_n,
//    the first term formed while ng_n is being computed, so each mini-batch
//    costs one 16x16x16 product, one LayerNorm backward and two barriers on
//    the critical path.  The two wave roles share each SIMD and overlap.
//  * K^T fragments for the state step come from an MFMA of K against a 0/t
//    selection pattern (exact for t = 1), instead of a transposed copy in LDS.
//  * Operands: bf16 inputs run the products on fp16 MFMA (inputs, W, ng and
//    the 16x16 matrices rounded to fp16; fp32 accumulation); fp32 inputs run
//    them on fp32 MFMA.
//  * Range: ng is carried as 2^8 ng and the 16x16 matrices (and the K^T and
//    ones operands of the state step) as 2^-8 of their values, so every
//    product is unchanged (powers of two are exact) while dot products of q
//    and k up to 2^8 * 65504 = 1.7e7 stay inside fp16, and ng values down to
//    2^-22 stay normal.  What fp16 still bounds: |q|, |k|, |W| <= 65504 and
//    |eta g| < 256 elementwise.
#include <type_traits>

#include "device_common.hpp"
#include "launch.hpp"

namespace ttt {
namespace {

constexpr int kM = 16;     // mini-batch size of this kernel
constexpr int kRing = 4;   // LDS stages and register sets (mini-batch mod 4)
constexpr int kFP = 68;    // fp32 row pitch of the exchange buffers
// ng is carried scaled by kNgScale, the matrices that multiply it by 1/kNgScale
constexpr float kNgScale = 256.f;
constexpr float kMatScale = 1.f / kNgScale;

typedef _Float16 h4 __attribute__((ext_vector_type(4)));
typedef _Float16 h8 __attribute__((ext_vector_type(8)));

// ---------------------------------------------------------------------------
// operand policies
// ---------------------------------------------------------------------------
template <typename T>
struct Op;

// fp16 operands: 16x16x32 MFMAs for the k = 64 products (two steps),
// 16x16x16 for the k = 16 ones.  Lane (g, n): A row n, B column n, k slots
// 8g..8g+7 (resp. 4g..4g+3); C rows 4g..4g+3, column n.
template <>
struct Op<_Float16> {
    static constexpr int XP = 72;  // row pitch of X tiles (144 B)
    static constexpr int GP = 68;  // row pitch of the ng tile: rows 4 apart land 8 banks apart
    using F4 = h4;
    struct XF {
        h8 v[2];
    };
    // B fragment of a row-major [token][column] tile: tokens 4g..4g+3 of column col
    __device__ static F4 load_b(const _Float16 *G, int col, int g) {
        return F4{G[(4 * g) * GP + col], G[(4 * g + 1) * GP + col], G[(4 * g + 2) * GP + col],
                  G[(4 * g + 3) * GP + col]};
    }
    // selection patterns for K^T: element i of pattern h is t where slot
    // 8g+i carries column 16r + n of the output tile (r = 2s + h)
    struct Sel {
        h8 p[2];
    };
    // Row n of a 16x64 tile, k permuted to match the accumulator layout of W:
    // slot 8g+i <- column 32s + 4g + i (i < 4), 32s + 16 + 4g + i - 4 (i >= 4).
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
    __device__ static XF cvt_w(const f32x4 (&Wt)[4]) {
        XF w;
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
    __device__ static F4 make(f32x4 x) { return F4{(_Float16)x[0], (_Float16)x[1], (_Float16)x[2], (_Float16)x[3]}; }
    __device__ static Sel sel(int n, int g, float t) {
        Sel s;
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int i = 0; i < 8; ++i)
                s.p[h][i] = (i / 4 == h && 4 * g + (i & 3) == n) ? (_Float16)t : (_Float16)0.f;
        return s;
    }
    // tile r of K (rows = tokens, columns 16r..16r+15) in accumulator layout,
    // i.e. the A fragment of K^T rows 16r..16r+15: lane holds K[4g+j][16r+n]
    __device__ static void kt_frags(const XF &k, const Sel &s, F4 (&kt)[4]) {
#pragma unroll
        for (int r = 0; r < 4; ++r)
            kt[r] = make(__builtin_amdgcn_mfma_f32_16x16x32_f16(k.v[r >> 1], s.p[r & 1], f32x4{0.f, 0.f, 0.f, 0.f},
                                                                 0, 0, 0));
    }
    __device__ static void put4(_Float16 *p, float x0, float x1, float x2, float x3) {
        *(h4 *)p = h4{(_Float16)x0, (_Float16)x1, (_Float16)x2, (_Float16)x3};
    }
    __device__ static void put(_Float16 *p, float x) { *p = (_Float16)x; }
};

// fp32 operands: 16x16x4 fp32 MFMAs (A lane (g,n) holds A[n][g], B holds B[g][n]).
template <>
struct Op<float> {
    static constexpr int XP = 68;
    static constexpr int GP = 68;
    using F4 = f32x4;
    struct XF {
        f32x4 v[4];  // v[r][j] = X[n][16r + 4g + j]
    };
    __device__ static F4 load_b(const float *G, int col, int g) {
        return F4{G[(4 * g) * GP + col], G[(4 * g + 1) * GP + col], G[(4 * g + 2) * GP + col],
                  G[(4 * g + 3) * GP + col]};
    }
    struct Sel {
        float p[4];  // p[j] = t where 4g + j == n
    };
    __device__ static XF load_x(const float *X, int n, int g) {
        XF x;
#pragma unroll
        for (int r = 0; r < 4; ++r) x.v[r] = *(const f32x4 *)(X + n * XP + 16 * r + 4 * g);
        return x;
    }
    __device__ static XF cvt_w(const f32x4 (&Wt)[4]) {
        XF w;
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
    __device__ static F4 make(f32x4 x) { return x; }
    __device__ static Sel sel(int n, int g, float t) {
        Sel s;
#pragma unroll
        for (int j = 0; j < 4; ++j) s.p[j] = (4 * g + j == n) ? t : 0.f;
        return s;
    }
    __device__ static void kt_frags(const XF &k, const Sel &s, F4 (&kt)[4]) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int j = 0; j < 4; ++j) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(k.v[r][j], s.p[j], acc, 0, 0, 0);
            kt[r] = acc;
        }
    }
    __device__ static void put4(float *p, float x0, float x1, float x2, float x3) {
        *(f32x4 *)p = f32x4{x0, x1, x2, x3};
    }
    __device__ static void put(float *p, float x) { *p = x; }
};

// Phase stamps: in a build with TTT_PHASE_STAMPS defined (an instrumentation
// build; the library is built without it), lane 0 of each wave records the
// low 32 bits of the shader clock at the phase boundaries of mini-batches
// kStampFirst .. kStampFirst + kStampSteps - 1 in LDS; at the end, workgroup 0
// copies them to stamps[(j * 8 + wave) * 8 + k] (j = m - kStampFirst), a
// device buffer given by ttt_phase_stamps_set.  Otherwise the stamps compile
// to nothing.
#ifdef TTT_PHASE_STAMPS
constexpr int kStampFirst = 256, kStampSteps = 64;
__device__ unsigned int *g_phase_stamps;
struct Stamps {
    unsigned int t[kStampSteps][8][8];
};
__device__ __forceinline__ void phase_stamp(Stamps &st, int m, int k) {
    __builtin_amdgcn_sched_barrier(0);
    const unsigned int t = (unsigned int)__builtin_amdgcn_s_memtime();
    const int j = m - kStampFirst;
    if (j >= 0 && j < kStampSteps && (threadIdx.x & 63) == 0) st.t[j][threadIdx.x >> 6][k] = t;
    __builtin_amdgcn_sched_barrier(0);
}
__device__ __forceinline__ void stamps_out(const Stamps &st) {
    if (blockIdx.x != 0) return;
    const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
    for (int i = l; i < kStampSteps * 8; i += 64) {
        const int j = i >> 3, k = i & 7;
        g_phase_stamps[(j * 8 + w) * 8 + k] = st.t[j][w][k];
    }
}
#define PHASE_STAMP(m, k) phase_stamp(sm.stamps, m, k)
#else
#define PHASE_STAMP(m, k) ((void)0)
#endif

// ---------------------------------------------------------------------------
// LDS
// ---------------------------------------------------------------------------
template <typename T>
struct Stage {
    T kx[kM][Op<T>::XP];  // K rows (rotated), operand type
    T qx[kM][Op<T>::XP];  // Q rows (rotated)
};

template <typename T>
struct Smem {
    Stage<T> st[kRing];
    float zbuf[kM][kFP];            // Z_n: written by column waves, read by row waves
    float zbbuf[2][kM][kFP];        // Zbar_n, double-buffered (read two steps later)
    T gm[kM][Op<T>::GP];            // ng, row-major [token][column]
#ifdef TTT_PHASE_STAMPS
    Stamps stamps;
#endif
};

// ---------------------------------------------------------------------------
// DPP within a row of 16 lanes
// ---------------------------------------------------------------------------
template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
    return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), CTRL, 0xF, 0xF, true));
}
// sum over the 16 lanes of the row; every lane receives it
__device__ __forceinline__ float row_sum16(float x) {
    x += dpp<0xB1>(x);   // quad_perm [1,0,3,2]
    x += dpp<0x4E>(x);   // quad_perm [2,3,0,1]
    x += dpp<0x141>(x);  // row_half_mirror
    x += dpp<0x140>(x);  // row_mirror
    return x;
}
// value of lane (n + 8) mod 16 of the row (the lane holding columns +-32)
__device__ __forceinline__ float row_swap8(float x) { return dpp<0x128>(x); }  // row_ror:8


// workgroup barrier that the instruction scheduler cannot move work across
// (s_barrier alone only orders memory operations): work placed between two
// barriers runs in that phase
__device__ __forceinline__ void phase_barrier() {
    __builtin_amdgcn_sched_barrier(0);
    __syncthreads();
    __builtin_amdgcn_sched_barrier(0);
}

// ---------------------------------------------------------------------------
// row waves: inputs of one mini-batch for token row t, columns 4n .. 4n+3
// ---------------------------------------------------------------------------

template <typename Tin>
struct Raw;
template <>
struct Raw<__bf16> {
    uint2 q, k, v;  // 4 bf16 each
    float eta;
    using U = uint2;
    __device__ static void pin(Raw &r) {
        asm volatile("" : "+v"(r.q.x), "+v"(r.q.y), "+v"(r.k.x), "+v"(r.k.y), "+v"(r.v.x), "+v"(r.v.y), "+v"(r.eta));
    }
    __device__ static void unpack(uint2 u, float (&x)[4]) {
        x[0] = __builtin_bit_cast(float, u.x << 16);
        x[1] = __builtin_bit_cast(float, u.x & 0xffff0000u);
        x[2] = __builtin_bit_cast(float, u.y << 16);
        x[3] = __builtin_bit_cast(float, u.y & 0xffff0000u);
    }
};
template <>
struct Raw<float> {
    uint4 q, k, v;
    float eta;
    using U = uint4;
    __device__ static void pin(Raw &r) {
        asm volatile("" : "+v"(r.q.x), "+v"(r.q.y), "+v"(r.q.z), "+v"(r.q.w), "+v"(r.k.x), "+v"(r.k.y), "+v"(r.k.z),
                     "+v"(r.k.w), "+v"(r.v.x), "+v"(r.v.y), "+v"(r.v.z), "+v"(r.v.w), "+v"(r.eta));
    }
    __device__ static void unpack(uint4 u, float (&x)[4]) {
        x[0] = __builtin_bit_cast(float, u.x);
        x[1] = __builtin_bit_cast(float, u.y);
        x[2] = __builtin_bit_cast(float, u.z);
        x[3] = __builtin_bit_cast(float, u.w);
    }
};

// what the LayerNorm phases need of one mini-batch, per lane
struct RowRegs {
    float cel[4];   // gamma * (k - v + beta): the target term of u = gamma * (LN(z) - (v - k))
    float qres[4];  // q + beta
    float eta;      // learning rate of the token
};

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

template <typename Tin, typename Tout, typename T, bool ROPE>
struct RowWave {
    const LinearArgs &a;
    int t, n, rw;  // token row 4rw + g, lane n within the row
    int N;
    // inputs: wave-uniform byte pointers to the next mini-batch to fetch
    // (advanced by one mini-batch per fetch), bytes per mini-batch, and this
    // lane's byte offsets within a mini-batch (32-bit: the host bounds them)
    const char *fq, *fk, *fv, *fe;
    int64_t bq, bk, bv;
    uint32_t oq, ok, ov, oe;
    int nf;  // next mini-batch to fetch
    // output: wave-uniform byte pointer of mini-batch 0, bytes per
    // mini-batch, this lane's byte offset.  A global store: the compiler
    // separates a wide global store from a later write of its data registers
    // (it does not do so for a buffer store with a register soffset, and on
    // this chip such a write right after the store corrupts the stored data)
    char *fo;
    int64_t bo;
    uint32_t oo;
    float gam[4], gam2[4], bet[4], gb[4];
    float cs[4], sn[4];    // rotary cos and signed sin of columns 4n + e at position t

    // mini-batches are fetched in order; the pointers stop at the last one,
    // so fetches past the end re-read it (in bounds, never staged for use)
    __device__ void fetch(Raw<Tin> &r) {
        using U = typename Raw<Tin>::U;
        r.q = *(const U *)(fq + oq);
        r.k = *(const U *)(fk + ok);
        r.v = *(const U *)(fv + ov);
        r.eta = *(const float *)(fe + oe);
        const bool adv = ++nf < N;
        fq += adv ? bq : 0;
        fk += adv ? bk : 0;
        fv += adv ? bv : 0;
        fe += adv ? (int64_t)(kM * sizeof(float)) : 0;
    }

    // rotary, MFMA row fragments of q and k into LDS, LayerNorm operands into rr
    __device__ void stage(Stage<T> &S, const Raw<Tin> &in, RowRegs &rr) const {
        // the inputs are consumed here and not earlier: the empty asm reads and
        // redefines them, so the conversions below (and the wait for the loads
        // they need) cannot be scheduled ahead of this mini-batch
        Raw<Tin> r = in;
        Raw<Tin>::pin(r);
        float qv[4], kv[4], vv[4];
        Raw<Tin>::unpack(r.q, qv);
        Raw<Tin>::unpack(r.k, kv);
        Raw<Tin>::unpack(r.v, vv);
        if constexpr (ROPE) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float qo = row_swap8(qv[e]), ko = row_swap8(kv[e]);
                qv[e] = qv[e] * cs[e] + qo * sn[e];
                kv[e] = kv[e] * cs[e] + ko * sn[e];
            }
        }
        Op<T>::put4(&S.qx[t][4 * n], qv[0], qv[1], qv[2], qv[3]);
        Op<T>::put4(&S.kx[t][4 * n], kv[0], kv[1], kv[2], kv[3]);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            rr.cel[e] = fmaf(gam[e], kv[e] - vv[e], gb[e]);
            rr.qres[e] = qv[e] + bet[e];
        }
        rr.eta = r.eta;
    }

    // LayerNorm backward of Z_nb (row t) into the ng tile:
    //   u = gamma * (LN(z) - (v - k)) = gamma^2 xhat + cel
    //   ng = -eta * dL/dz = -eta * rs * (u - mean(u) - xhat * mean(u xhat))
    // Mean and mean square share one reduction round, as do the two means
    // of u (short dependency chains: this is on the sequential path).
    __device__ void ln_backward(Smem<T> &sm, const RowRegs &rr) const {
        const f32x4 z = *(const f32x4 *)&sm.zbuf[t][4 * n];
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
            u[e] = fmaf(gam2[e], xh[e], rr.cel[e]);
        }
        float su = (u[0] + u[1]) + (u[2] + u[3]);
        float sux = fmaf(u[0], xh[0], u[1] * xh[1]) + fmaf(u[2], xh[2], u[3] * xh[3]);
        row_sum16x2(su, sux);
        const float A = -kNgScale * rr.eta * rs;  // 2^8 ng
        const float C0 = -A * su * (1.f / kD), C1 = -A * sux * (1.f / kD);
        float ng[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) ng[e] = fmaf(u[e], A, fmaf(xh[e], C1, C0));
        Op<T>::put4(&sm.gm[t][4 * n], ng[0], ng[1], ng[2], ng[3]);
    }

    // LayerNorm forward of Zbar_nb (row t): out = q + LN(Zbar)
    __device__ void ln_forward(const Smem<T> &sm, const RowRegs &rr, int nb) const {
        const f32x4 zb = *(const f32x4 *)&sm.zbbuf[nb & 1][t][4 * n];
        float s1 = (zb[0] + zb[1]) + (zb[2] + zb[3]);
        float s2 = fmaf(zb[0], zb[0], zb[1] * zb[1]) + fmaf(zb[2], zb[2], zb[3] * zb[3]);
        row_sum16x2(s1, s2);
        const float mu = s1 * (1.f / kD);
        const float var = fmaxf(fmaf(-mu, mu, s2 * (1.f / kD)), 0.f);
        const float rs = __builtin_amdgcn_rsqf(var + a.eps);  // var + eps >= eps > 0
        const float mrs = -mu * rs;
        float y[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) y[e] = fmaf(fmaf(zb[e], rs, mrs), gam[e], rr.qres[e]);
        char *o = fo + (int64_t)nb * bo + oo;
        if constexpr (std::is_same<Tout, float>::value) {
            *(f32x4 *)o = f32x4{y[0], y[1], y[2], y[3]};
        } else {
            typedef __bf16 b4 __attribute__((ext_vector_type(4)));
            *(b4 *)o = b4{(__bf16)y[0], (__bf16)y[1], (__bf16)y[2], (__bf16)y[3]};
        }
    }
};

template <typename Tin, typename Tout, typename T, bool ROPE>
__device__ void row_main(const LinearArgs &a, Smem<T> &sm, int bi, int hi, int rw, int g, int n) {
    RowWave<Tin, Tout, T, ROPE> R{a};
    R.t = 4 * rw + g;
    R.n = n;
    R.rw = rw;
    R.N = a.ntok;
    const int N = a.ntok;
    constexpr int64_t ein = sizeof(Tin);
    R.fq = (const char *)((const Tin *)a.q.p + bi * a.q.sB + hi * a.q.sH + (int64_t)a.t0 * a.q.sL);
    R.fk = (const char *)((const Tin *)a.k.p + bi * a.k.sB + hi * a.k.sH + (int64_t)a.t0 * a.k.sL);
    R.fv = (const char *)((const Tin *)a.v.p + bi * a.v.sB + hi * a.v.sH + (int64_t)a.t0 * a.v.sL);
    R.fe = (const char *)(a.eta + bi * a.eta_sB + hi * a.eta_sH + a.t0);
    R.bq = kM * a.q.sL * ein;
    R.bk = kM * a.k.sL * ein;
    R.bv = kM * a.v.sL * ein;
    R.oq = (uint32_t)((R.t * a.q.sL + 4 * n) * ein);
    R.ok = (uint32_t)((R.t * a.k.sL + 4 * n) * ein);
    R.ov = (uint32_t)((R.t * a.v.sL + 4 * n) * ein);
    R.oe = (uint32_t)(R.t * sizeof(float));
    R.nf = 0;
    // output rows of this chain from the first token of the call
    R.fo = (char *)((Tout *)a.out.p + bi * a.out.sB + hi * a.out.sH + (int64_t)a.t0 * a.out.sL);
    R.oo = (uint32_t)((R.t * a.out.sL + 4 * n) * (int64_t)sizeof(Tout));
    R.bo = kM * a.out.sL * (int64_t)sizeof(Tout);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const int c = 4 * n + e;
        R.gam[e] = a.ln_w[hi * kD + c];
        R.bet[e] = a.ln_b[hi * kD + c];
        R.gam2[e] = R.gam[e] * R.gam[e];
        R.gb[e] = R.gam[e] * R.bet[e];
        // whole mini-batches start at multiples of 16: position mod 16 == t
        const int i = c & 31;
        const double th = (double)R.t * pow((double)a.rope_base, -2.0 * (double)i / (double)kD);
        R.cs[e] = (float)cos(th);
        R.sn[e] = (c < 32 ? -1.f : 1.f) * (float)sin(th);
    }

    Raw<Tin> pf[kRing];  // pf[m % 4]: inputs of mini-batch m, fetched 4 steps ahead
    RowRegs rr[kRing];   // rr[m % 4]: LayerNorm operands of mini-batch m
#pragma unroll
    for (int i = 0; i < kRing; ++i) R.fetch(pf[i]);  // 0 .. 3
    R.stage(sm.st[0], pf[0], rr[0]);
    R.fetch(pf[0]);  // 4
    R.stage(sm.st[1], pf[1], rr[1]);
    R.fetch(pf[1]);  // 5
    phase_barrier();  // mini-batches 0, 1 staged
    R.stage(sm.st[2], pf[2], rr[2]);
    R.fetch(pf[2]);  // 6
    phase_barrier();  // Z_0 written
    R.ln_backward(sm, rr[0]);
    phase_barrier();  // ng_0 ready

    // step m (1 <= m < N).  Phase 1 (off the sequential chain, while the
    // column waves form Z_m): forward LayerNorm of Zbar_m-2, stage m+2, fetch
    // m+6.  Phase 2: backward LayerNorm of Z_m -> ng_m (the column waves form
    // Zbar_m-1 and the products of mini-batch m meanwhile).
    // In the loop m = 2 + 4k + i, so every register-set index is static:
    // slot (m+2) % 4 = (m-2) % 4 = i, slot m % 4 = (2+i) % 4.
    auto step = [&](int m, auto I) {
        constexpr int i = decltype(I)::value;
        PHASE_STAMP(m, 0);
        R.ln_forward(sm, rr[i], m - 2);
        PHASE_STAMP(m, 1);
        // slot i is reused by the staging below: finish reading it first
        __builtin_amdgcn_sched_barrier(0);
        R.stage(sm.st[i], pf[i], rr[i]);
        PHASE_STAMP(m, 2);
        // consume the register set before refilling it, so the refill lands in
        // the same registers (no copies that would wait on the new loads)
        __builtin_amdgcn_sched_barrier(0);
        R.fetch(pf[i]);  // m + 6
        PHASE_STAMP(m, 3);
        phase_barrier();  // Z_m written
        PHASE_STAMP(m, 4);
        R.ln_backward(sm, rr[(2 + i) % kRing]);
        PHASE_STAMP(m, 5);
        phase_barrier();  // ng_m ready, Zbar_m-1 written
    };
    // after the last step, with N = m + r (m = 2 mod 4): Zbar_N-2, Zbar_N-1
    auto last = [&](auto I) {
        constexpr int r = decltype(I)::value;
        R.ln_forward(sm, rr[r % kRing], N - 2);
        phase_barrier();  // Zbar_N-1 written
        R.ln_forward(sm, rr[(r + 1) % kRing], N - 1);
    };
    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    using I2 = std::integral_constant<int, 2>;
    using I3 = std::integral_constant<int, 3>;
    if (N == 1) {
        phase_barrier();  // Zbar_0 written
        R.ln_forward(sm, rr[0], 0);
        return;
    }
    // step 1 (nothing to forward yet)
    R.stage(sm.st[3], pf[3], rr[3]);
    __builtin_amdgcn_sched_barrier(0);
    R.fetch(pf[3]);  // 7
    phase_barrier();  // Z_1 written
    R.ln_backward(sm, rr[1]);
    phase_barrier();  // ng_1 ready, Zbar_0 written
    int m = 2;
    for (; m + 3 < N; m += kRing) {  // branch-free steady state
        step(m, I0{});
        step(m + 1, I1{});
        step(m + 2, I2{});
        step(m + 3, I3{});
    }
    switch (N - m) {  // 0 .. 3 steps left
    case 0:
        last(I0{});
        break;
    case 1:
        step(m, I0{});
        last(I1{});
        break;
    case 2:
        step(m, I0{});
        step(m + 1, I1{});
        last(I2{});
        break;
    default:
        step(m, I0{});
        step(m + 1, I1{});
        step(m + 2, I2{});
        last(I3{});
        break;
    }
}

// causal matrix t_n tril(S + 1) from S^T in accumulator layout (lane: query
// n, keys 4g+j; t_n the query row's token_eta)
__device__ __forceinline__ f32x4 causal(f32x4 st, int n, int g, float tn) {
    f32x4 m;
#pragma unroll
    for (int j = 0; j < 4; ++j) m[j] = (4 * g + j <= n) ? fmaf(st[j], tn, tn) : 0.f;
    return m;
}

__device__ __forceinline__ f32x4 scaled(f32x4 x, float t) {
    return f32x4{x[0] * t, x[1] * t, x[2] * t, x[3] * t};
}

// TE: token_eta given (otherwise every scale is the constant 1 and the code is
// that of the plain dual form)
template <typename T, bool TE>
__device__ void col_main(const LinearArgs &a, Smem<T> &sm, int ch, int c, int g, int n) {
    using O = Op<T>;
    using F4 = typename O::F4;
    using XF = typename O::XF;
    const int N = a.ntok;

    // state: W slab (rows 16r + 4g + j, column 16c + n), bias tile
    f32x4 Wt[4], Bt;
    {
        const float *Wc = a.W + (int64_t)ch * kD * kD;
#pragma unroll
        for (int r = 0; r < 4; ++r)
#pragma unroll
            for (int j = 0; j < 4; ++j) Wt[r][j] = Wc[(16 * r + 4 * g + j) * kD + 16 * c + n];
        const float bv = a.b[(int64_t)ch * kD + 16 * c + n];
        Bt = f32x4{bv, bv, bv, bv};
    }
    // token_eta of query row n, and of the last row (the carried step), both
    // times 2^-8: the matrices and operands they scale multiply 2^8 ng
    const float tn = (TE ? a.te[n] : 1.f) * kMatScale;
    const float tl = (TE ? a.te[kM - 1] : 1.f) * kMatScale;
    const typename O::Sel sel = O::sel(n, g, tl);
    const F4 ones = O::make(f32x4{tl, tl, tl, tl});
    const f32x4 zero = {0.f, 0.f, 0.f, 0.f}, one = {1.f, 1.f, 1.f, 1.f};

    f32x4 Y, P;   // Y_m+1 = K_m+1 W_m + b_m ; P_m = Q_m W_m + b_m
    F4 Mf, Cf;    // t_i tril(Q_m K_m^T + 1), t (K_m+1 K_m^T + 1) (A fragments)
    F4 kt[4];     // t K_m^T rows 16r .. 16r+15 (A fragments)
    XF kxn;       // K_m row fragment

    phase_barrier();  // mini-batches 0, 1 staged
    {
        const XF wf = O::cvt_w(Wt);
        const XF kx0 = O::load_x(&sm.st[0].kx[0][0], n, g);
        const XF qx0 = O::load_x(&sm.st[0].qx[0][0], n, g);
        const f32x4 Z0 = O::xx(kx0, wf, Bt);
#pragma unroll
        for (int j = 0; j < 4; ++j) sm.zbuf[4 * g + j][16 * c + n] = Z0[j];
        P = O::xx(qx0, wf, Bt);
        Mf = O::make(causal(O::xx(kx0, qx0, zero), n, g, tn));
        const XF kx1 = O::load_x(&sm.st[1].kx[0][0], n, g);
        Y = O::xx(kx1, wf, Bt);
        Cf = O::make(scaled(O::xx(kx0, kx1, one), tl));
        O::kt_frags(kx0, sel, kt);
        kxn = kx1;
    }
    phase_barrier();  // Z_0 written
    phase_barrier();  // ng_0 ready

    for (int m = 1; m < N; ++m) {
        // phase 1, the sequential chain: Z_m = Y_m + C_m-1 ng_m-1
        PHASE_STAMP(m, 0);
        const F4 gf = O::load_b(&sm.gm[0][0], 16 * c + n, g);
        const f32x4 Z = O::mma16(Cf, gf, Y);
#pragma unroll
        for (int j = 0; j < 4; ++j) sm.zbuf[4 * g + j][16 * c + n] = Z[j];
        PHASE_STAMP(m, 1);
        phase_barrier();  // Z_m written
        PHASE_STAMP(m, 2);

        // phase 2 (row waves run the LayerNorm of Z_m): Zbar_m-1, W_m, b_m,
        // then the products of mini-batch m with W_m
        {
            const f32x4 ZB = O::mma16(Mf, gf, P);
#pragma unroll
            for (int j = 0; j < 4; ++j) sm.zbbuf[(m - 1) & 1][4 * g + j][16 * c + n] = ZB[j];
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) Wt[r] = O::mma16(kt[r], gf, Wt[r]);
        Bt = O::mma16(ones, gf, Bt);
        const XF wf = O::cvt_w(Wt);
        const XF qx = O::load_x(&sm.st[m % kRing].qx[0][0], n, g);
        const XF kx1 = O::load_x(&sm.st[(m + 1) % kRing].kx[0][0], n, g);  // stale past the end: unused
        P = O::xx(qx, wf, Bt);
        Y = O::xx(kx1, wf, Bt);
        Mf = O::make(causal(O::xx(kxn, qx, zero), n, g, tn));
        Cf = O::make(scaled(O::xx(kxn, kx1, one), tl));
        O::kt_frags(kxn, sel, kt);
        kxn = kx1;
        PHASE_STAMP(m, 3);
        phase_barrier();  // ng_m ready, Zbar_m-1 written
    }
    {
        const F4 gf = O::load_b(&sm.gm[0][0], 16 * c + n, g);
        const f32x4 ZB = O::mma16(Mf, gf, P);
#pragma unroll
        for (int j = 0; j < 4; ++j) sm.zbbuf[(N - 1) & 1][4 * g + j][16 * c + n] = ZB[j];
        phase_barrier();  // Zbar_N-1 written
#pragma unroll
        for (int r = 0; r < 4; ++r) Wt[r] = O::mma16(kt[r], gf, Wt[r]);
        Bt = O::mma16(ones, gf, Bt);
    }

    float *Wo = a.W + (int64_t)ch * kD * kD;
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int j = 0; j < 4; ++j) Wo[(16 * r + 4 * g + j) * kD + 16 * c + n] = Wt[r][j];
    if (g == 0) a.b[(int64_t)ch * kD + 16 * c + n] = Bt[0];
}

// fp16 operands fit 128 VGPRs, so two chains share a CU when there are more
// chains than CUs; the fp32-operand variant keeps its larger register file
template <typename T>
constexpr int kWavesPerSimd = std::is_same<T, _Float16>::value ? 4 : 1;

template <typename Tin, typename Tout, typename T, bool ROPE, bool TE>
__global__ __launch_bounds__(512, kWavesPerSimd<T>) void linear_dual_kernel(LinearArgs a) {
    extern __shared__ __align__(16) unsigned char smem_raw[];
    Smem<T> &sm = *reinterpret_cast<Smem<T> *>(smem_raw);
    const int ch = blockIdx.x;
    const int bi = ch / a.H, hi = ch % a.H;
    const int w = threadIdx.x >> 6, l = threadIdx.x & 63, g = l >> 4, n = l & 15;
    // both roles pass the same sequence of 2N + 2 barriers
    if (w < 4)
        col_main<T, TE>(a, sm, ch, w, g, n);
    else
        row_main<Tin, Tout, T, ROPE>(a, sm, bi, hi, w - 4, g, n);
#ifdef TTT_PHASE_STAMPS
    stamps_out(sm.stamps);
#endif
}

template <typename Tin, typename Tout, typename T, bool ROPE, bool TE>
hipError_t launch_typed(const LinearArgs &a, hipStream_t s) {
    const void *fn = (const void *)&linear_dual_kernel<Tin, Tout, T, ROPE, TE>;
    const size_t lds = sizeof(Smem<T>);
    static std::atomic<uint64_t> configured{0};  // per instantiation: devices whose LDS limit is raised
    if (hipError_t e = ensure_lds_limit(fn, lds, configured); e != hipSuccess) return e;
    hipLaunchKernelGGL((linear_dual_kernel<Tin, Tout, T, ROPE, TE>), dim3(a.B * a.H), dim3(512), lds, s, a);
    return hipGetLastError();
}

template <typename Tin, typename Tout, typename T>
hipError_t launch_rope(const LinearArgs &a, hipStream_t s) {
    if (a.te != nullptr)
        return a.rope ? launch_typed<Tin, Tout, T, true, true>(a, s) : launch_typed<Tin, Tout, T, false, true>(a, s);
    return a.rope ? launch_typed<Tin, Tout, T, true, false>(a, s) : launch_typed<Tin, Tout, T, false, false>(a, s);
}

}  // namespace

#ifdef TTT_PHASE_STAMPS
extern "C" int ttt_phase_stamps_set(unsigned int *buf) {
    return (int)hipMemcpyToSymbol(HIP_SYMBOL(g_phase_stamps), &buf, sizeof(buf));
}
#endif

hipError_t launch_linear_dual(const LinearArgs &a, int in_bf16, int out_bf16, hipStream_t s) {
    if (in_bf16 && out_bf16) return launch_rope<__bf16, __bf16, _Float16>(a, s);
    if (in_bf16) return launch_rope<__bf16, float, _Float16>(a, s);
    if (out_bf16) return launch_rope<float, __bf16, float>(a, s);
    return launch_rope<float, float, float>(a, s);
}

}  // namespace ttt
