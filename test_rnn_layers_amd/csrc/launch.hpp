// launch.hpp -- host-side launchers of the libttt kernels (library-private).
#pragma once

#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdint>

#include "device_common.hpp"

namespace ttt {

// Raises a kernel's dynamic LDS limit to `bytes` once per device (the limit
// is per device), safe under concurrent callers: `done` holds one bit per
// device ordinal < 64 (a concurrent first call may set it twice, which is
// harmless); devices past 63 set it on every launch.
inline hipError_t ensure_lds_limit(const void *fn, size_t bytes, std::atomic<uint64_t> &done) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    const uint64_t bit = dev < 64 ? (uint64_t)1 << dev : 0;
    if (bit && (done.load(std::memory_order_acquire) & bit)) return hipSuccess;
    e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
    if (e == hipSuccess && bit) done.fetch_or(bit, std::memory_order_release);
    return e;
}

// Everything a TTT-MLP launch needs (state [B*H, ...] fp32, F = 256).
struct MlpArgs {
    TDesc q, k, v;
    const float *eta;
    int64_t eta_sB, eta_sH;
    const float *ln_w, *ln_b;
    float *W1, *b1, *W2, *b2;
    float *W1g, *b1g, *W2g, *b2g;
    ODesc out;
    int32_t B, H;
    int32_t nblk;     // mini-batches, the last one possibly partial
    int32_t tail;     // tokens in the last mini-batch if partial, else 0
    int32_t t0;
    int64_t pos0;
    int32_t rope;
    float rope_base;
    float eps;
    const float *te;  // token_eta [K] or nullptr (all ones)
    int32_t K;        // mini-batch size (token kernel; the dual kernel takes 16)
    int32_t ntok;     // tokens (token kernel)
    int32_t grad_rows;  // W1_grad / W2_grad hold the open rows [k | eta g1], [x2 | eta g2]
};

hipError_t launch_linear_token(const LinearArgs &a, int in_bf16, int out_bf16, hipStream_t s);
hipError_t launch_linear_dual(const LinearArgs &a, int in_bf16, int out_bf16, hipStream_t s);
hipError_t launch_mlp_dual(const MlpArgs &a, int in_bf16, int out_bf16, hipStream_t s);
hipError_t launch_mlp_token(const MlpArgs &a, int in_bf16, int out_bf16, hipStream_t s);
// State initialisation: up to 8 segments filled by one launch.
struct TileSeg {
    float *dst;
    const float *src;  // [per] tiled over dst[total]; nullptr: zeros
    int64_t per, total;
};
struct TileList {
    TileSeg seg[8];
    int32_t n;
};
hipError_t launch_tiles(const TileList &t, hipStream_t s);

}  // namespace ttt
