// post_proj.hpp -- host-side launchers of the post-norm LayerNorm and output
// projection (post_proj.hip; library-private).
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace ttt {

// Post-norm LayerNorm and output projection of the layer output (post_proj.hip).
struct PostPrepArgs {
    const float *gamma, *beta;  // [K]
    const float *Wo;            // [K, N]
    const float *bias;          // [N] or nullptr
    __bf16 *Wt;                 // W' = diag(gamma) Wo, transposed: [N, K]
    float *c1, *c2;             // [N]
    int32_t K, N;
};
struct PostArgs {
    const __bf16 *y;  // [M, K] rows of stride ldy
    int64_t ldy;
    const __bf16 *Wt;
    const float *c1, *c2;
    void *out;        // [M, N] rows of stride ldo
    int64_t ldo;
    int32_t M, K, N;
    float eps;
};
hipError_t launch_post_proj_prepare(const PostPrepArgs &a, hipStream_t s);
hipError_t launch_post_proj(const PostArgs &a, int out_bf16, hipStream_t s);

}  // namespace ttt
