// Internal launcher interface between the C ABI (api.hip) and the kernel files.
#pragma once

#include "common.hpp"

namespace spark {

// Validated sizes of one call, shared by every launcher.
struct LaunchCtx {
    int B, H, BH, N, Nv, n_sink, d, block, M, K;
    int pool_mode, dtype;
    float scale;
    hipStream_t stream;
};

void launch_pool(const LaunchCtx& L, const void* Q, const void* K, const void* V, float* q_mean,
                 float* k_mean, float* k_sum, float* v_sum, float* bias, float* anchor);

void launch_select(const LaunchCtx& L, const float* q_mean, const float* k_mean, int32_t* idx,
                   float* scores);

void launch_attend(const LaunchCtx& L, const void* Q, const void* K, const void* V, const float* k_sum,
                   const float* v_sum, const float* bias, const int32_t* idx, const int32_t* perm,
                   void* O, float* lse);

void launch_gather_rows(const LaunchCtx& L, const void* X, const int32_t* perm, void* Y);

// Reblock workspace layout (bytes), and its launch sequence.
size_t reblock_workspace_bytes(const LaunchCtx& L);
void launch_reblock(const LaunchCtx& L, const void* Q, const void* K, int32_t* perm, void* ws);

}  // namespace spark
