// device_common.hpp -- small gfx950 helpers shared by the libttt kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ttt {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kD = 64;      // head_dim handled by every kernel
constexpr int kWave = 64;   // CDNA wavefront

// Strided activation [B, H, L, D] (element strides), D contiguous.
struct TDesc {
    const void *p;
    int64_t sB, sH, sL;
};
struct ODesc {
    void *p;
    int64_t sB, sH, sL;
};

// Everything a TTT-Linear launch needs; passed by value as the kernel argument.
struct LinearArgs {
    TDesc q, k, v;
    const float *eta;
    int64_t eta_sB, eta_sH;
    const float *ln_w, *ln_b;   // [H, D]
    float *W, *b, *Wg, *bg;     // state [B*H, D, D], [B*H, D]
    ODesc out;
    int32_t B, H, K;
    int32_t ntok;               // tokens (token kernel) or whole mini-batches (dual kernel)
    int32_t t0;                 // first token index inside q/k/v/eta/out
    int64_t pos0;               // absolute position of that token
    int32_t rope;
    float rope_base;
    float eps;
};

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(__bf16 x) { return (float)x; }

template <typename T> __device__ __forceinline__ T from_f32(float x);
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <> __device__ __forceinline__ __bf16 from_f32<__bf16>(float x) { return (__bf16)x; }

// Sum over the 64 lanes of a wavefront; every lane receives the total.
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) x += __shfl_xor(x, m, kWave);
    return x;
}

// Sum over the 16 lanes of a DPP row (lanes 16r .. 16r+15); every lane of the
// row receives its row's total.
__device__ __forceinline__ float row16_sum(float x) {
#pragma unroll
    for (int m = 8; m >= 1; m >>= 1) x += __shfl_xor(x, m, kWave);
    return x;
}

// 16x16x32 bf16 MFMA, fp32 accumulate.
// Lane l (g = l/16, n = l%16): A holds A[n][8g .. 8g+7], B holds B[8g .. 8g+7][n],
// C/D holds C[4g .. 4g+3][n].
__device__ __forceinline__ f32x4 mfma_k32(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
// 16x16x16 bf16 MFMA, fp32 accumulate.  A holds A[n][4g .. 4g+3],
// B holds B[4g .. 4g+3][n], C/D as above.
__device__ __forceinline__ f32x4 mfma_k16(bf16x4 a, bf16x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(i16x4, a),
                                                      __builtin_bit_cast(i16x4, b), c, 0, 0, 0);
}

// Split x into a bf16 pair with x ~= hi + lo (error ~2^-17 |x|).
__device__ __forceinline__ void split_bf16(float x, __bf16 &hi, __bf16 &lo) {
    hi = (__bf16)x;
    lo = (__bf16)(x - (float)hi);
}

}  // namespace ttt
