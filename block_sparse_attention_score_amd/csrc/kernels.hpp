// Internal launcher interface between the C ABI (api.hip) and the kernel files.
#pragma once

#include "common.hpp"

namespace spark {

// Validated sizes of one call, shared by every launcher.
struct LaunchCtx {
    int B, H, BH, N, Nv, n_sink, d, block, M, K;
    int block_k, Mk;  // key block size and key blocks (the route's columns); K is over Mk
    int pool_mode, dtype;
    float scale;
    hipStream_t stream;
};

void launch_pool(const LaunchCtx& L, const void* Q, const void* K, const void* V, float* q_mean,
                 float* k_mean, float* k_sum, float* v_sum, float* bias, float* anchor);
// launch_pool followed by launch_pack, with K and V read once: the pooling kernel also writes the
// video key tiles.
void launch_pool_pack(const LaunchCtx& L, const void* Q, const void* K, const void* V, float* q_mean,
                      float* k_mean, float* k_sum, float* v_sum, float* bias, float* anchor, void* packed);

// Select writes the full score matrix S [BH, M, M_k] (fp32) to `scores`, then the route.
size_t select_workspace_bytes(const LaunchCtx& L);
void launch_select(const LaunchCtx& L, const float* q_mean, const float* k_mean, int32_t* idx,
                   float* scores);
// adaptive-tau routes: idx [B,H,M,M] (row I's kept blocks ascending), counts [B,H,M], stats
// [B,H,2] = (mu, sigma) or NULL; scores [B,H,M,M] and partials (tau_partials_bytes) are scratch
size_t tau_partials_bytes(const LaunchCtx& L);
void launch_select_tau(const LaunchCtx& L, float tau, const float* q_mean, const float* k_mean, int32_t* idx,
                       int32_t* counts, float* stats, float* scores, double* partials);

// Packed 64-key tiles read by the attention kernel (layout in pack.hip).
struct PackGeom {
    int Tv, Ts, Tc, Tall;  // video, sink, compressed and total tiles per (batch, head)
    int SQ, NQT;           // sink-query tiles (of `block` rows) and all query tiles (SQ + M) per (batch, head)
    size_t tile_elems;     // bf16 elements per tile (K rows + V^T)
    size_t kv_bytes;       // all tiles of all heads
    size_t bias_off;       // byte offset of the fp32 bias rows [BH][Tall][64]
    size_t tmax_off;       // per tile {max |k|^2, max additive term} over its valid keys, float2 [BH][Tall]
    size_t bnd_off;        // per head {max |k| exact keys, max |k| pseudo-keys, max pseudo-key term, 0}, float4 [BH]
    size_t flag_off;       // per query tile: 1 when the fixed-offset pass left it to the exact pass, int32 [BH][NQT]
    size_t queue_off;      // the fixed-offset pass's tile counters, one per XCD, int32 [8]
    size_t bytes;          // total
};
PackGeom pack_geom(const LaunchCtx& L);

void launch_pack(const LaunchCtx& L, const void* K, const void* V, const float* k_sum, const float* v_sum,
                 const float* bias, void* packed);
// launch_fp8_scales restricted to rows row0 .. N-1 (amax zeroed first), and pooling that also
// takes the amax of the video rows (launch_fp8_scales + launch_pool in one pass over Q, K, V)
void launch_fp8_amax_rows(const LaunchCtx& L, const void* Q, const void* K, const void* V, uint32_t* amax,
                          int row0);
void launch_pool_fp8_scales(const LaunchCtx& L, const void* Q, const void* K, const void* V, float* q_mean,
                            float* k_mean, float* k_sum, float* v_sum, float* bias, float* anchor, uint32_t* amax);

// the sink tiles and the compressed tiles only
void launch_pack_rest(const LaunchCtx& L, const void* K, const void* V, const float* k_sum, const float* v_sum,
                      const float* bias, void* packed);
// the per-head logit-bound constants from the per-tile maxima (after every tile is written)
void launch_bounds(const LaunchCtx& L, void* packed);

// idx [B,H,M,K] with counts == NULL, or a variable route: idx [B,H,M,M] with counts [B,H,M]
void launch_attend(const LaunchCtx& L, const void* Q, const void* packed, const int32_t* idx,
                   const int32_t* counts, const int32_t* perm, void* O, float* lse);

void launch_gather_rows(const LaunchCtx& L, const void* X, const int32_t* perm, void* Y);

// FP8 (E4M3) carriers: per-head amax [BH][3] (Q, K, V; float bits), packed fp8 tiles (layout in
// attn_fwd_fp8.hip; same tile list and bias rows as pack_geom), and the attention on them.
PackGeom pack_geom_fp8(const LaunchCtx& L);
void launch_fp8_scales(const LaunchCtx& L, const void* Q, const void* K, const void* V, uint32_t* amax);
void launch_pack_fp8(const LaunchCtx& L, const void* K, const void* V, const float* k_sum, const float* v_sum,
                     const float* bias, const uint32_t* amax, void* packed);
void launch_attend_fp8(const LaunchCtx& L, const void* Q, const void* packed, const int32_t* idx,
                       const int32_t* perm, const uint32_t* amax, void* O, float* lse);

// Reblock workspace layout (bytes), and its launch sequence.
size_t reblock_workspace_bytes(const LaunchCtx& L);
void launch_reblock(const LaunchCtx& L, const void* Q, const void* K, int32_t* perm, void* ws);

}  // namespace spark
