/*
 * c_example.c -- libttt used from plain C through include/ttt.h: TTT-Linear
 * prefill of the first tokens of a sequence, then decode of the rest with the
 * carried state, on fp32 inputs from a fixed linear congruential generator.
 *
 *   ttt_c_example OUT.bin
 *
 * writes, as little-endian int32 B, H, L, D, Lp followed by float32 arrays:
 * XQ, XK, XV [B,H,L,D]; eta [H,L]; W0 [H,D,D]; b0, ln_w, ln_b [H,D];
 * out [B,H,L,D]; W [B,H,D,D]; b [B,H,D] (the state after all L tokens).
 * Exit status 0 on success; on a libttt or HIP error the message goes to
 * stderr and the status is 1.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "ttt.h"

enum { B = 2, H = 3, L = 40, D = 64, LP = 27 };

static uint64_t lcg = 0x2545F4914F6CDD1DULL;
static float uniform(void) { /* [-1, 1) */
    lcg = lcg * 6364136223846793005ULL + 1442695040888963407ULL;
    return (float)((lcg >> 40) * (1.0 / 8388608.0)) - 1.0f;
}

#define HIP_OK(x)                                                                  \
    do {                                                                           \
        hipError_t e_ = (x);                                                       \
        if (e_ != hipSuccess) {                                                    \
            fprintf(stderr, "HIP error %s at line %d\n", hipGetErrorString(e_), __LINE__); \
            return 1;                                                              \
        }                                                                          \
    } while (0)
#define TTT_OK_(x)                                                                 \
    do {                                                                           \
        ttt_status s_ = (x);                                                       \
        if (s_ != TTT_OK) {                                                        \
            fprintf(stderr, "libttt: %s (%s)\n", ttt_status_string(s_), ttt_last_error()); \
            return 1;                                                              \
        }                                                                          \
    } while (0)

static int upload(float **dev, const float *host, size_t n) {
    if (hipMalloc((void **)dev, n * sizeof(float)) != hipSuccess) return 1;
    return hipMemcpy(*dev, host, n * sizeof(float), hipMemcpyHostToDevice) != hipSuccess;
}

int main(int argc, char **argv) {
    if (argc != 2) {
        fprintf(stderr, "usage: %s OUT.bin\n", argv[0]);
        return 2;
    }
    const size_t nx = (size_t)B * H * L * D, neta = (size_t)H * L, nw = (size_t)H * D * D, nv = (size_t)H * D;
    float *x[3], *eta = malloc(neta * 4), *w0 = malloc(nw * 4), *b0 = calloc(nv, 4), *lw = malloc(nv * 4),
                 *lb = calloc(nv, 4);
    for (int i = 0; i < 3; ++i) {
        x[i] = malloc(nx * 4);
        for (size_t j = 0; j < nx; ++j) x[i][j] = uniform();
    }
    for (size_t j = 0; j < neta; ++j) eta[j] = (1.0f / 64.0f) * (0.75f + 0.25f * uniform());
    for (size_t j = 0; j < nw; ++j) w0[j] = 0.02f * uniform();
    for (size_t j = 0; j < nv; ++j) lw[j] = 1.0f + 0.1f * uniform();

    float *dx[3], *deta, *dw0, *db0, *dlw, *dlb, *dout, *dW, *db, *dWg, *dbg;
    for (int i = 0; i < 3; ++i)
        if (upload(&dx[i], x[i], nx)) return 1;
    if (upload(&deta, eta, neta) || upload(&dw0, w0, nw) || upload(&db0, b0, nv) || upload(&dlw, lw, nv) ||
        upload(&dlb, lb, nv))
        return 1;
    HIP_OK(hipMalloc((void **)&dout, nx * 4));
    HIP_OK(hipMalloc((void **)&dW, (size_t)B * nw * 4));
    HIP_OK(hipMalloc((void **)&db, (size_t)B * nv * 4));
    HIP_OK(hipMalloc((void **)&dWg, (size_t)B * nw * 4));
    HIP_OK(hipMalloc((void **)&dbg, (size_t)B * nv * 4));

    const ttt_linear_cfg cfg = {B, H, D, 16, TTT_F32, TTT_F32, 0, 10000.0f, 1e-6f, TTT_GRAD_DENSE};
    ttt_linear_state st = {dW, db, dWg, dbg, 0};
    TTT_OK_(ttt_linear_state_init(&cfg, dw0, db0, &st, NULL));

    /* [B, H, L, D] tensors; a call on tokens [t0, t1) starts t0 rows in */
    const int64_t sB = (int64_t)H * L * D, sH = (int64_t)L * D, sL = D;
    for (int piece = 0; piece < 2; ++piece) {
        const int t0 = piece == 0 ? 0 : LP, t1 = piece == 0 ? LP : L;
        ttt_tensor q = {dx[0] + (size_t)t0 * D, sB, sH, sL}, k = {dx[1] + (size_t)t0 * D, sB, sH, sL},
                   v = {dx[2] + (size_t)t0 * D, sB, sH, sL}, o = {dout + (size_t)t0 * D, sB, sH, sL};
        ttt_eta e = {deta + t0, 0, L, NULL};
        if (piece == 0)
            TTT_OK_(ttt_linear_prefill(&cfg, t1 - t0, q, k, v, e, dlw, dlb, &st, o, NULL));
        else
            TTT_OK_(ttt_linear_decode(&cfg, t1 - t0, q, k, v, e, dlw, dlb, &st, o, NULL));
    }
    HIP_OK(hipDeviceSynchronize());
    if (st.offset != L) {
        fprintf(stderr, "state offset %lld, expected %d\n", (long long)st.offset, L);
        return 1;
    }

    float *out = malloc(nx * 4), *W = malloc((size_t)B * nw * 4), *bb = malloc((size_t)B * nv * 4);
    HIP_OK(hipMemcpy(out, dout, nx * 4, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(W, dW, (size_t)B * nw * 4, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(bb, db, (size_t)B * nv * 4, hipMemcpyDeviceToHost));

    FILE *f = fopen(argv[1], "wb");
    if (!f) {
        fprintf(stderr, "cannot open %s\n", argv[1]);
        return 1;
    }
    const int32_t hdr[5] = {B, H, L, D, LP};
    fwrite(hdr, sizeof hdr, 1, f);
    for (int i = 0; i < 3; ++i) fwrite(x[i], 4, nx, f);
    fwrite(eta, 4, neta, f);
    fwrite(w0, 4, nw, f);
    fwrite(b0, 4, nv, f);
    fwrite(lw, 4, nv, f);
    fwrite(lb, 4, nv, f);
    fwrite(out, 4, nx, f);
    fwrite(W, 4, (size_t)B * nw, f);
    fwrite(bb, 4, (size_t)B * nv, f);
    fclose(f);
    return 0;
}
