// linear_token.hip -- TTT-Linear one token at a time (primal form) and the
// state initialisation kernels.
//
// Primal form of "代码连连看——TTT", compute_mini_batch, primal branch: for
// each token the gradient of its LN + L2 reconstruction loss is taken at the
// mini-batch-start W, b; the eta-weighted gradients accumulate into W_grad,
// b_grad (the pages' carried "W1_grad", "b1_grad"); the prediction uses
// W - W_grad, b - b_grad; at a mini-batch boundary the step is committed and
// the gradients cleared (TTTCache continuation, "TTTLinear.ttt").
//
// One workgroup of 256 threads per (batch, head) chain.  Thread t owns column
// c = t % 64 of W and W_grad for rows 16*(t/64) .. +15, in registers for the
// whole call, so a call over T tokens reads and writes the 33 KB state once.
// Used for decoding, for the tokens that complete an open mini-batch before a
// prefill, for a trailing partial mini-batch, and for mini-batch sizes the
// dual-form MFMA kernel does not take.
#include "device_common.hpp"
#include "launch.hpp"

namespace ttt {

template <typename Tin, typename Tout>
__global__ __launch_bounds__(256) void linear_token_kernel(LinearArgs a) {
    const int ch = blockIdx.x;
    const int bi = ch / a.H, hi = ch % a.H;
    const int tid = threadIdx.x;
    const int c = tid & 63;
    const int rg = tid >> 6;

    __shared__ float sq[2][kD], sk[2][kD], sv[2][kD];
    __shared__ float pz[2][4][kD], pzb[2][4][kD];
    // rotary cos and signed sin at position p (mod K <= 16) for column c
    __shared__ float rcs[16][kD], rsn[16][kD];

    float *Wc = a.W + (int64_t)ch * kD * kD;
    float *Gc = a.Wg + (int64_t)ch * kD * kD;
    // a call that starts on a mini-batch boundary finds the accumulated
    // gradients cleared (every commit clears them), so it does not read them
    const bool g_clear = a.pos0 % a.K == 0;
    float Ws[16], Gs[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        Ws[i] = Wc[(16 * rg + i) * kD + c];
        Gs[i] = g_clear ? 0.f : Gc[(16 * rg + i) * kD + c];
    }
    float bs = a.b[(int64_t)ch * kD + c];
    float gbs = g_clear ? 0.f : a.bg[(int64_t)ch * kD + c];
    bool committed = false;  // W_s, b_s change only at a commit
    const float gam = a.ln_w[hi * kD + c];
    const float bet = a.ln_b[hi * kD + c];

    const Tin *qp = (const Tin *)a.q.p + bi * a.q.sB + hi * a.q.sH;
    const Tin *kp = (const Tin *)a.k.p + bi * a.k.sB + hi * a.k.sH;
    const Tin *vp = (const Tin *)a.v.p + bi * a.v.sB + hi * a.v.sH;
    const float *ep = a.eta + bi * a.eta_sB + hi * a.eta_sH;
    Tout *op = (Tout *)a.out.p + bi * a.out.sB + hi * a.out.sH;

    if (a.rope) {
        // angle p * base^(-2i/D) for the pair (i, i + 32) holding column c
        for (int e = tid; e < 16 * kD; e += 256) {
            const int p = e / kD, cc = e % kD;
            const double th = (double)p * pow((double)a.rope_base, -2.0 * (double)(cc & 31) / (double)kD);
            rcs[p][cc] = (float)cos(th);
            rsn[p][cc] = (cc < 32 ? -1.f : 1.f) * (float)sin(th);  // x*cos - x_pair*sin | x*cos + x_pair*sin
        }
        __syncthreads();
    }

    for (int t = 0; t < a.ntok; ++t) {
        const int buf = t & 1;
        const int tok = a.t0 + t;
        const int64_t pos = a.pos0 + t;
        if (rg == 0) {
            float qv = to_f32(qp[(int64_t)tok * a.q.sL + c]);
            float kv = to_f32(kp[(int64_t)tok * a.k.sL + c]);
            if (a.rope) {
                const float qo = to_f32(qp[(int64_t)tok * a.q.sL + (c ^ 32)]);
                const float ko = to_f32(kp[(int64_t)tok * a.k.sL + (c ^ 32)]);
                const int p = (int)(pos % a.K);
                const float cs = rcs[p][c], sg = rsn[p][c];
                qv = qv * cs + qo * sg;
                kv = kv * cs + ko * sg;
            }
            sq[buf][c] = qv;
            sk[buf][c] = kv;
            sv[buf][c] = to_f32(vp[(int64_t)tok * a.v.sL + c]);
        }
        const float e = ep[tok];
        __syncthreads();

        // Z1 = k W + b at the mini-batch-start state
        float zp = 0.f;
#pragma unroll
        for (int i = 0; i < 16; ++i) zp += sk[buf][16 * rg + i] * Ws[i];
        pz[buf][rg][c] = zp;
        __syncthreads();
        const float z = pz[buf][0][c] + pz[buf][1][c] + pz[buf][2][c] + pz[buf][3][c] + bs;

        // gradient of 1/2 ||LN(z) - (v - k)||^2 (every wave holds the whole row)
        const float mu = wave_sum(z) * (1.f / kD);
        const float d = z - mu;
        const float rs = rsqrtf(wave_sum(d * d) * (1.f / kD) + a.eps);
        const float xh = d * rs;
        const float u = gam * (gam * xh + bet - (sv[buf][c] - sk[buf][c]));
        const float su = wave_sum(u) * (1.f / kD);
        const float sux = wave_sum(u * xh) * (1.f / kD);
        const float g = (u - su - xh * sux) * rs;

        // accumulate the eta-weighted gradient; prediction with W - W_grad
        const float eg = e * g;
        float zbp = 0.f;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const float kr = sk[buf][16 * rg + i];
            Gs[i] += kr * eg;
            zbp += sq[buf][16 * rg + i] * (Ws[i] - Gs[i]);
        }
        gbs += eg;
        pzb[buf][rg][c] = zbp;
        __syncthreads();
        const float zb = pzb[buf][0][c] + pzb[buf][1][c] + pzb[buf][2][c] + pzb[buf][3][c] + bs - gbs;
        if (rg == 0) {
            const float mu2 = wave_sum(zb) * (1.f / kD);
            const float d2 = zb - mu2;
            const float rs2 = rsqrtf(wave_sum(d2 * d2) * (1.f / kD) + a.eps);
            op[(int64_t)tok * a.out.sL + c] = from_f32<Tout>(sq[buf][c] + gam * d2 * rs2 + bet);
        }
        if ((pos + 1) % a.K == 0) {
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                Ws[i] -= Gs[i];
                Gs[i] = 0.f;
            }
            bs -= gbs;
            gbs = 0.f;
            committed = true;
        }
    }
    // write back what changed: W_s, b_s after a commit; the gradients unless
    // they were clear in memory and are clear again
    const bool g_clear_out = (a.pos0 + a.ntok) % a.K == 0;
    if (committed) {
#pragma unroll
        for (int i = 0; i < 16; ++i) Wc[(16 * rg + i) * kD + c] = Ws[i];
        if (rg == 0) a.b[(int64_t)ch * kD + c] = bs;
    }
    if (!(g_clear && g_clear_out)) {
#pragma unroll
        for (int i = 0; i < 16; ++i) Gc[(16 * rg + i) * kD + c] = Gs[i];
        if (rg == 0) a.bg[(int64_t)ch * kD + c] = gbs;
    }
}

// dst[b, i] = src[i % per] for b < copies: tiles a per-head parameter over the
// batch; with src == nullptr it writes zeros.
__global__ void tile_kernel(float *dst, const float *src, int64_t per, int64_t total) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < total) dst[i] = src ? src[i % per] : 0.f;
}

hipError_t launch_linear_token(const LinearArgs &a, int in_bf16, int out_bf16, hipStream_t s) {
    dim3 grid(a.B * a.H), block(256);
    if (in_bf16 && out_bf16)
        hipLaunchKernelGGL((linear_token_kernel<__bf16, __bf16>), grid, block, 0, s, a);
    else if (in_bf16)
        hipLaunchKernelGGL((linear_token_kernel<__bf16, float>), grid, block, 0, s, a);
    else if (out_bf16)
        hipLaunchKernelGGL((linear_token_kernel<float, __bf16>), grid, block, 0, s, a);
    else
        hipLaunchKernelGGL((linear_token_kernel<float, float>), grid, block, 0, s, a);
    return hipGetLastError();
}

hipError_t launch_tile(float *dst, const float *src, int64_t per, int64_t total, hipStream_t s) {
    if (total <= 0) return hipSuccess;
    const int64_t nb = (total + 255) / 256;
    hipLaunchKernelGGL(tile_kernel, dim3((unsigned)nb), dim3(256), 0, s, dst, src, per, total);
    return hipGetLastError();
}

}  // namespace ttt
