// device_common.hpp -- small gfx950 helpers shared by the libttt kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ttt {

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
    int32_t grad_rows;          // W_grad holds the open mini-batch's rows [k_j | eta_j g_j]
    const float *te;            // token_eta [K] or nullptr (all ones)
};

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(__bf16 x) { return (float)x; }

template <typename T> __device__ __forceinline__ T from_f32(float x);
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <> __device__ __forceinline__ __bf16 from_f32<__bf16>(float x) { return (__bf16)x; }

// Sums over the 64 lanes of a wavefront; every lane receives the totals.
// Each 16-lane row is summed with DPP lane moves (pairs, quads, half-row
// mirror, row mirror: every lane of the row then holds the row total), and
// the four row totals are read out through scalar registers and added in a
// fixed order.  No LDS round trips, unlike cross-lane shuffles.
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float x) {
    return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), CTRL, 0xF, 0xF, true));
}
// Orders a wave's LDS writes before its later LDS reads of values other lanes
// wrote.  The hardware executes one wave's LDS accesses in program order, but
// the compiler reasons per lane and may move a read above a write whose
// address it proves different for that lane; this memory clobber stops it.
__device__ __forceinline__ void wave_lds_order() { asm volatile("" ::: "memory"); }

__device__ __forceinline__ float lane_value(float x, int lane) {
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), lane));
}
__device__ __forceinline__ float rows_total(float x) {
    return ((lane_value(x, 0) + lane_value(x, 16)) + lane_value(x, 32)) + lane_value(x, 48);
}
// two independent sums, their DPP chains interleaved
__device__ __forceinline__ void wave_sum2(float &x, float &y) {
    x += dpp_mov<0xB1>(x);   // quad_perm [1,0,3,2]
    y += dpp_mov<0xB1>(y);
    x += dpp_mov<0x4E>(x);   // quad_perm [2,3,0,1]
    y += dpp_mov<0x4E>(y);
    x += dpp_mov<0x141>(x);  // row_half_mirror
    y += dpp_mov<0x141>(y);
    x += dpp_mov<0x140>(x);  // row_mirror
    y += dpp_mov<0x140>(y);
    x = rows_total(x);
    y = rows_total(y);
}

}  // namespace ttt
