// post_proj.hip -- the post-norm LayerNorm and output projection applied to
// the layer output ("代码连连看——TTT", TTTBase.forward: after the scan the
// heads' outputs, concatenated to [B, L, width], go through post_norm, a
// LayerNorm over the width, and o_proj, a linear map).
//
// With y the [M, K] output (M = B L token rows, K = width = H D) and Wo [K, N]:
//   out[m, :] = ((y[m, :] - mean_m) r_m * gamma + beta) Wo + bias,
//   r_m = 1 / sqrt(var_m + eps)  (population variance over the row).
// It runs as one bf16 GEMM with the LayerNorm taken out of its operand:
//   out[m, n] = r_m (y[m, :] . W'[:, n]) - r_m mean_m c1[n] + c2[n],
//   W' = bf16(diag(gamma) Wo),  c1[n] = sum_k W'[k, n],  c2 = beta^T Wo + bias,
// which is exactly LayerNorm-then-GEMM with the weights W' (c1 is summed from
// the rounded W'), so the GEMM reads y as it is (bf16) and never writes a
// normalised copy.
//
// Design (gfx950):
//  * post_proj_prepare_kernel forms W' once per weight set, stored transposed
//    ([N][K], K contiguous: each lane's 16x16x32 B fragment is 16 bytes), and
//    c1, c2;
//  * post_proj_kernel: 256x256 output tile per workgroup of 8 waves (2 x 4;
//    each wave 128 x 64 = 8 x 4 tiles of 16x16x32 bf16 MFMAs, fp32
//    accumulators), K in steps of 64 through a double-buffered LDS stage
//    (row pitch 144 B: a wave's 16-byte fragment reads hit 64 distinct banks);
//    the next step's global loads are issued before the current step's MFMAs;
//  * the row statistics come from the A fragments the waves already hold:
//    the waves of column block 0 accumulate sum y and sum y^2 with bf16 dot
//    products (v_dot2c_f32_bf16) beside their MFMAs;
//  * tile order: the N-tiles of one 256-row panel run on one XCD (blocks 8
//    apart go to the same XCD), so the panel is read from one L2.
#include <hip/hip_runtime.h>

#include <atomic>

#include "device_common.hpp"
#include "launch.hpp"
#include "post_proj.hpp"

namespace ttt {
namespace {

constexpr int BM = 256, BN = 256, BK = 64;
constexpr int AP = 72;  // LDS row pitch in bf16 (144 B)

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

struct PSmem {
    __bf16 A[2][BM][AP];  // y rows [m][k], by K-step parity
    __bf16 B[2][BN][AP];  // W'^T rows [n][k]
    float mu[BM], r[BM];  // row mean and 1 / sqrt(var + eps)
};

// W'^T [N][K] bf16, c1, c2 [N].  A workgroup takes 16 columns: thread
// (k-group kg, column cl) forms w = bf16(gamma_k Wo[k][col]) for k = kg mod 16
// (the 16 columns of a row are one 64-byte read), the rounded values go
// through LDS in chunks of 256 k so that every column's row of W'^T is
// written in 16-byte pieces, and the fp64 column sums of the 16 k-groups are
// added in a fixed order at the end.
constexpr int kPrepCols = 16, kPrepChunk = 256;
__global__ __launch_bounds__(256) void post_proj_prepare_kernel(PostPrepArgs p) {
    __shared__ __align__(16) __bf16 tile[kPrepCols][kPrepChunk + 8];  // [column][k in the chunk]
    __shared__ double red[2][16][kPrepCols];                           // [c1 | c2][k-group][column]
    const int t = threadIdx.x, cl = t & 15, kg = t >> 4;
    const int c0 = blockIdx.x * kPrepCols, col = c0 + cl;
    double c1 = 0.0, c2 = 0.0;
    for (int k0 = 0; k0 < p.K; k0 += kPrepChunk) {
        const int kn = min(kPrepChunk, p.K - k0);  // a multiple of 64
        for (int kk = kg; kk < kn; kk += 16) {
            const int k = k0 + kk;
            const float wo = p.Wo[(int64_t)k * p.N + col];
            const __bf16 w = (__bf16)(p.gamma[k] * wo);
            tile[cl][kk] = w;
            c1 += (double)(float)w;
            c2 += (double)p.beta[k] * (double)wo;
        }
        __syncthreads();
        const int pieces = kn / 8;  // 16-byte pieces per column
        for (int c = t; c < kPrepCols * pieces; c += 256) {
            const int cc = c / pieces, pc = c % pieces;
            *(uint4 *)(p.Wt + (int64_t)(c0 + cc) * p.K + k0 + 8 * pc) = *(const uint4 *)&tile[cc][8 * pc];
        }
        __syncthreads();
    }
    red[0][kg][cl] = c1;
    red[1][kg][cl] = c2;
    __syncthreads();
    if (t < kPrepCols) {
        double s1 = 0.0, s2 = 0.0;
        for (int q = 0; q < 16; ++q) {
            s1 += red[0][q][t];
            s2 += red[1][q][t];
        }
        p.c1[c0 + t] = (float)s1;
        p.c2[c0 + t] = (float)(s2 + (p.bias ? (double)p.bias[c0 + t] : 0.0));
    }
}

template <typename Tout>
__global__ __launch_bounds__(512, 1) void post_proj_kernel(PostArgs p) {
    extern __shared__ __align__(16) unsigned char smem_raw[];
    PSmem &sm = *reinterpret_cast<PSmem *>(smem_raw);
    const int MT = (p.M + BM - 1) / BM, NT = p.N / BN;
    int bm, bn;
    {
        const int b = blockIdx.x;
        if (MT % 8 == 0) {  // the NT tiles of panel bm on XCD b % 8
            const int x = b & 7, i = b >> 3;
            bm = (i / NT) * 8 + x;
            bn = i % NT;
        } else {
            bm = b / NT;
            bn = b % NT;
        }
    }
    const int m0 = bm * BM, n0 = bn * BN;
    const int t = threadIdx.x, w = t >> 6, l = t & 63, g = l >> 4, n = l & 15;
    const int wm = w & 1, wn = w >> 1;  // this wave: rows wm*128 .. +127, columns wn*64 .. +63
    const int KT = p.K / BK;

    // global -> LDS: chunk c = t + 512 i (i < 4) of each tile is row c / 8,
    // k offset 8 (c % 8); rows past M read row M-1 (their outputs are not stored)
    bf16x8 ra[4], rb[4];
    auto load_step = [&](int kt) {
        const int k0 = kt * BK;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int c = t + 512 * i, row = c >> 3, kc = (c & 7) * 8;
            const int m = min(m0 + row, p.M - 1);
            ra[i] = *(const bf16x8 *)(p.y + (int64_t)m * p.ldy + k0 + kc);
            rb[i] = *(const bf16x8 *)(p.Wt + (int64_t)(n0 + row) * p.K + k0 + kc);
        }
    };
    auto store_step = [&](int s) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int c = t + 512 * i, row = c >> 3, kc = (c & 7) * 8;
            *(bf16x8 *)&sm.A[s][row][kc] = ra[i];
            *(bf16x8 *)&sm.B[s][row][kc] = rb[i];
        }
    };

    f32x4 acc[8][4];
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    float sy[8], syy[8];  // row 16i + n of the wave: partial sums over this lane's k slices
#pragma unroll
    for (int i = 0; i < 8; ++i) sy[i] = syy[i] = 0.f;
    const bool stats = wn == 0;
    const bf16x2 one2 = {(__bf16)1.f, (__bf16)1.f};

    load_step(0);
    store_step(0);
    __syncthreads();
    for (int kt = 0; kt < KT; ++kt) {
        const int s = kt & 1;
        if (kt + 1 < KT) load_step(kt + 1);
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            bf16x8 af[8], bf[4];
#pragma unroll
            for (int i = 0; i < 8; ++i) af[i] = *(const bf16x8 *)&sm.A[s][wm * 128 + 16 * i + n][ks * 32 + 8 * g];
#pragma unroll
            for (int j = 0; j < 4; ++j) bf[j] = *(const bf16x8 *)&sm.B[s][wn * 64 + 16 * j + n][ks * 32 + 8 * g];
#pragma unroll
            for (int i = 0; i < 8; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], bf[j], acc[i][j], 0, 0, 0);
            if (stats) {
#pragma unroll
                for (int i = 0; i < 8; ++i)
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const bf16x2 pr = {af[i][2 * e], af[i][2 * e + 1]};
                        sy[i] = __builtin_amdgcn_fdot2_f32_bf16(pr, one2, sy[i], false);
                        syy[i] = __builtin_amdgcn_fdot2_f32_bf16(pr, pr, syy[i], false);
                    }
            }
        }
        if (kt + 1 < KT) store_step(s ^ 1);
        __syncthreads();
    }

    // row statistics: lanes n, n+16, n+32, n+48 hold the four k slices of row 16i + n
    if (stats) {
        const float inv_k = 1.f / (float)p.K;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            float a = sy[i], q = syy[i];
            a += __shfl_xor(a, 16);
            q += __shfl_xor(q, 16);
            a += __shfl_xor(a, 32);
            q += __shfl_xor(q, 32);
            if (g == 0) {
                const int row = wm * 128 + 16 * i + n;
                const float mean = a * inv_k;
                const float var = fmaxf(fmaf(-mean, mean, q * inv_k), 0.f);
                sm.mu[row] = mean;
                sm.r[row] = __builtin_amdgcn_rsqf(var + p.eps);  // var + eps >= eps > 0
            }
        }
    }
    __syncthreads();

    // out = r (y . W') - r mean c1 + c2, staged through LDS in two passes of
    // 128 rows (the waves of row block p write their tiles, then every thread
    // stores 16-byte pieces of whole rows)
    constexpr int OP = 256 + 16 / (int)sizeof(Tout);  // staging row pitch (elements)
    Tout *stage = reinterpret_cast<Tout *>(smem_raw);   // [128][OP], over the A/B stages
    Tout *out = (Tout *)p.out;
    float c1[4], c2[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int col = n0 + wn * 64 + 16 * j + n;
        c1[j] = p.c1[col];
        c2[j] = p.c2[col];
    }
    for (int pass = 0; pass < 2; ++pass) {
        if (wm == pass) {
#pragma unroll
            for (int i = 0; i < 8; ++i)
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) {
                    const int rl = 16 * i + 4 * g + jj, row = 128 * pass + rl;
                    const float r = sm.r[row], nmr = -r * sm.mu[row];
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        stage[rl * OP + wn * 64 + 16 * j + n] = (Tout)fmaf(r, acc[i][j][jj], fmaf(nmr, c1[j], c2[j]));
                }
        }
        __syncthreads();
        constexpr int per_row = 256 * (int)sizeof(Tout) / 16;  // 16-byte pieces per row
#pragma unroll 4
        for (int c = t; c < 128 * per_row; c += 512) {
            const int rl = c / per_row, piece = c % per_row;
            const int m = m0 + 128 * pass + rl;
            if (m < p.M)
                *(uint4 *)((char *)(out + (int64_t)m * p.ldo + n0) + 16 * piece) =
                    *(const uint4 *)((const char *)(stage + rl * OP) + 16 * piece);
        }
        __syncthreads();
    }
}

template <typename Tout>
hipError_t launch_gemm(const PostArgs &a, hipStream_t s) {
    const void *fn = (const void *)&post_proj_kernel<Tout>;
    static std::atomic<uint64_t> configured{0};
    if (hipError_t e = ensure_lds_limit(fn, sizeof(PSmem), configured); e != hipSuccess) return e;
    const int blocks = ((a.M + BM - 1) / BM) * (a.N / BN);
    hipLaunchKernelGGL((post_proj_kernel<Tout>), dim3(blocks), dim3(512), sizeof(PSmem), s, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_post_proj_prepare(const PostPrepArgs &a, hipStream_t s) {
    hipLaunchKernelGGL(post_proj_prepare_kernel, dim3(a.N / kPrepCols), dim3(256), 0, s, a);  // N % 256 == 0
    return hipGetLastError();
}

hipError_t launch_post_proj(const PostArgs &a, int out_bf16, hipStream_t s) {
    return out_bf16 ? launch_gemm<__bf16>(a, s) : launch_gemm<float>(a, s);
}

}  // namespace ttt
