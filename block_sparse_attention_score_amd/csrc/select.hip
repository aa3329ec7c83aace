// Top-K key-block selection per query block (core sparse-attention node page, section
// "ブロックスパースアテンション": each query block is routed to a subset of key blocks; the top-k
// mode keeps a fixed fraction of them; Spark-H3 page, "ワークフロー": topk_mode=topk_ratio).
//
// One workgroup scores R query-block rows of one (batch, head) against every key block:
// S_IJ = s * q_mean_I . k_mean_J in fp32 (the fp32 means are staged through LDS 64 key rows at a
// time, so each k_mean row is read once per workgroup).  The R score rows stay in LDS; one wave
// then finds each row's K-th largest score by a 32-step bisection on order-preserving integer
// keys (wave ballots and sums), resolves ties toward lower block indices, and writes the chosen
// blocks in ascending order with a ballot/popcount compaction.
#include "kernels.hpp"

namespace spark {

constexpr int kSelChunk = 64;  // key rows staged per step

// Order-preserving map float -> uint32 (larger float, larger key); -0 is folded onto +0.
__device__ __forceinline__ uint32_t score_key(float f) {
    f = f + 0.0f;
    const uint32_t u = __float_as_uint(f);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

template <int D>
__global__ __launch_bounds__(256) void select_kernel(const float* __restrict__ q_mean,
                                                     const float* __restrict__ k_mean, int M, int K,
                                                     int R, float scale, int32_t* __restrict__ idx,
                                                     float* __restrict__ scores) {
    extern __shared__ float smem[];
    constexpr int KS = D + 4;  // padded stride of staged key rows
    const int rowblocks = (M + R - 1) / R;
    const int bh = blockIdx.x / rowblocks, I0 = (blockIdx.x % rowblocks) * R;
    const int nr = min(R, M - I0);
    float* qs = smem;                 // [R][D]
    float* kc = qs + R * D;           // [kSelChunk][KS]
    float* S = kc + kSelChunk * KS;   // [R][M]

    const float* qsrc = q_mean + ((size_t)bh * M + I0) * D;
    for (int e = threadIdx.x; e < nr * D; e += 256) qs[e] = qsrc[e];

    const int jl = threadIdx.x & 63, rw = threadIdx.x >> 6;
    const float* ksrc = k_mean + (size_t)bh * M * D;
    for (int J0 = 0; J0 < M; J0 += kSelChunk) {
        const int nj = min(kSelChunk, M - J0);
        __syncthreads();
        for (int e = threadIdx.x; e < kSelChunk * (D / 4); e += 256) {
            const int r = e / (D / 4), c4 = (e % (D / 4)) * 4;
            f32x4 v = {0.f, 0.f, 0.f, 0.f};
            if (r < nj) v = *reinterpret_cast<const f32x4*>(ksrc + (size_t)(J0 + r) * D + c4);
            *reinterpret_cast<f32x4*>(kc + r * KS + c4) = v;
        }
        __syncthreads();
        if (jl < nj) {
            const float* kr = kc + jl * KS;
            for (int r = rw; r < nr; r += 4) {
                const float* qr = qs + r * D;
                float acc = 0.f;
#pragma unroll 8
                for (int c = 0; c < D; c += 4) {
                    const f32x4 kv = *reinterpret_cast<const f32x4*>(kr + c);
                    const f32x4 qv = *reinterpret_cast<const f32x4*>(qr + c);
                    acc = fmaf(qv[0], kv[0], acc);
                    acc = fmaf(qv[1], kv[1], acc);
                    acc = fmaf(qv[2], kv[2], acc);
                    acc = fmaf(qv[3], kv[3], acc);
                }
                S[r * M + J0 + jl] = scale * acc;
            }
        }
    }
    __syncthreads();

    if (scores) {
        float* dst = scores + ((size_t)bh * M + I0) * M;
        for (int e = threadIdx.x; e < nr * M; e += 256) dst[e] = S[e];
    }

    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const uint64_t below = lanemask_lt();
    for (int r = w; r < nr; r += 4) {
        const float* Sr = S + r * M;
        // largest T with #{J : key_J >= T} >= K, i.e. the K-th largest key, bit by bit from the top
        uint32_t T = 0;
        for (int bit = 31; bit >= 0; --bit) {
            const uint32_t cand = T | (1u << bit);
            int cnt = 0;
            for (int J = lane; J < M; J += 64) cnt += score_key(Sr[J]) >= cand;
            if (wave_sum_int(cnt) >= K) T = cand;
        }
        int gt = 0;
        for (int J = lane; J < M; J += 64) gt += score_key(Sr[J]) > T;
        const int need = K - wave_sum_int(gt);  // keys equal to T still to take, lowest J first
        int32_t* out = idx + ((size_t)bh * M + I0 + r) * K;
        int pos = 0, eq_seen = 0;
        for (int J0 = 0; J0 < M; J0 += 64) {
            const int J = J0 + lane;
            const uint32_t kk = J < M ? score_key(Sr[J]) : 0u;
            const bool eq = J < M && kk == T;
            const uint64_t eqb = __ballot(eq);
            const int eq_rank = eq_seen + __popcll(eqb & below);
            const bool sel = J < M && (kk > T || (eq && eq_rank < need));
            const uint64_t sb = __ballot(sel);
            if (sel) out[pos + __popcll(sb & below)] = J;
            pos += __popcll(sb);
            eq_seen += __popcll(eqb);
        }
    }
}

static int max_lds_bytes() {
    static int cached = 0;
    if (!cached) {
        int dev = 0, v = 0;
        if (hipGetDevice(&dev) == hipSuccess &&
            hipDeviceGetAttribute(&v, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) == hipSuccess && v > 0)
            cached = v;
        else
            cached = 65536;
    }
    return cached;
}

template <int D>
static void launch_select_t(const LaunchCtx& L, const float* q_mean, const float* k_mean, int32_t* idx,
                            float* scores) {
    const int budget = max_lds_bytes();
    const int fixed = kSelChunk * (D + 4) * 4;
    int R = (budget - fixed) / (4 * (D + L.M));
    R = R > 16 ? 16 : (R < 1 ? 1 : R);
    const size_t lds = (size_t)4 * (R * D + kSelChunk * (D + 4) + (size_t)R * L.M);
    if (lds > 65536)
        (void)hipFuncSetAttribute((const void*)select_kernel<D>,
                                  hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    const int rowblocks = (L.M + R - 1) / R;
    hipLaunchKernelGGL((select_kernel<D>), dim3(L.BH * rowblocks), dim3(256), lds, L.stream, q_mean, k_mean,
                       L.M, L.K, R, L.scale, idx, scores);
}

void launch_select(const LaunchCtx& L, const float* q_mean, const float* k_mean, int32_t* idx,
                   float* scores) {
    if (L.d == 64) launch_select_t<64>(L, q_mean, k_mean, idx, scores);
    else launch_select_t<128>(L, q_mean, k_mean, idx, scores);
}

}  // namespace spark
