// Block pooling: per-block means of Q and K, the per-head anchor, and the compressed K/V summary
// with its log-mass bias (Spark-H3 page, section "Spark-Attnが変えるもの", Spark-Reweight bullet).
//
// HBM-bound: Q is read once by pool_q, K and V once by pool_kv.  One workgroup per (batch,
// head, block) reads the block's rows with 16-byte loads (row-contiguous, fully coalesced);
// every reduction runs in a fixed order, so results are deterministic.
#include <type_traits>

#include "kernels.hpp"

namespace spark {

// Rows of a block handled by one thread: thread (c, rg) owns the 8-element column chunk c of rows
// rg, rg + RG, ... (RG row groups of CH chunk-threads).
template <int D> struct PoolGeom {
    static constexpr int CH = D / 8;
    static constexpr int RG = 256 / CH;
};

// Element j of eight loaded consecutive elements, as fp32; and the eight set to zero.
__device__ __forceinline__ float raw_elem(const Raw8<__bf16>& r, int j) {
    return bf16_bits_to_f32((j & 1) ? r.u[j >> 1] >> 16 : r.u[j >> 1] & 0xffffu);
}
__device__ __forceinline__ float raw_elem(const Raw8<float>& r, int j) { return j < 4 ? r.a[j] : r.b[j - 4]; }
__device__ __forceinline__ void raw_zero(Raw8<__bf16>& r) { r.u = u32x4{0u, 0u, 0u, 0u}; }
__device__ __forceinline__ void raw_zero(Raw8<float>& r) {
    r.a = f32x4{0.f, 0.f, 0.f, 0.f};
    r.b = f32x4{0.f, 0.f, 0.f, 0.f};
}

// AMAX: also raise amax_q (float bits; non-negative floats order as unsigned integers) to the
// largest |q| of the block, for the E4M3 scales.
template <typename T, int D, int BLK, bool AMAX>
__global__ __launch_bounds__(256) void pool_q_kernel(const T* __restrict__ Q, int N, int Nv, int M,
                                                     float* __restrict__ q_mean, uint32_t* __restrict__ amax) {
    using G = PoolGeom<D>;
    constexpr int RPT = (BLK + G::RG - 1) / G::RG;  // rows per thread
    const int bh = blockIdx.x / M, J = blockIdx.x % M;
    const int c = threadIdx.x % G::CH, rg = threadIdx.x / G::CH;
    const int lo = J * BLK, n = min(BLK, Nv - lo);
    const T* base = Q + ((size_t)bh * N + lo) * D + c * 8;

    // every row load is issued first (rows past the block end read its last row and are dropped)
    Raw8<T> raw[RPT];
#pragma unroll
    for (int k = 0; k < RPT; ++k) raw[k].load(base + (size_t)min(rg + k * G::RG, n - 1) * D);
    float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    float am = 0.f;
#pragma unroll
    for (int k = 0; k < RPT; ++k) {
        if (rg + k * G::RG < n) {
            float v[8];
            raw[k].widen(v);
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                acc[j] += v[j];
                if (AMAX) am = fmaxf(am, fabsf(v[j]));
            }
        }
    }
    __shared__ float wmax[4];
    if constexpr (AMAX) {
        am = wave_max(am);
        if ((threadIdx.x & 63) == 0) wmax[threadIdx.x >> 6] = am;
    }
    __shared__ float red[G::RG][D];
#pragma unroll
    for (int j = 0; j < 8; ++j) red[rg][c * 8 + j] = acc[j];
    __syncthreads();
    if (AMAX && threadIdx.x == 0)
        raise_max_bits(&amax[(size_t)bh * 3], fmaxf(fmaxf(wmax[0], wmax[1]), fmaxf(wmax[2], wmax[3])));
    for (int col = threadIdx.x; col < D; col += 256) {
        float s = 0.f;
        for (int g = 0; g < G::RG; ++g) s += red[g][col];
        q_mean[((size_t)bh * M + J) * D + col] = s / (float)n;
    }
}

// anchor = mean of all video queries = sum_J n_J * q_mean_J / N_v, binary64 accumulation in a
// fixed order: 1024 threads per (batch, head), P = 1024 / D interleaved partial sums per column,
// combined in part order.
constexpr int kAnchorThreads = 1024;

template <int D>
__global__ __launch_bounds__(kAnchorThreads) void anchor_kernel(const float* __restrict__ q_mean, int Nv, int M,
                                                                int BLK, float* __restrict__ anchor) {
    constexpr int P = kAnchorThreads / D;
    __shared__ double red[P][D];
    const int bh = blockIdx.x, col = threadIdx.x % D, part = threadIdx.x / D;
    const float* qm = q_mean + (size_t)bh * M * D + col;
    double s = 0.0;
#pragma unroll 8
    for (int J = part; J < M; J += P) s += (double)min(BLK, Nv - J * BLK) * (double)qm[(size_t)J * D];
    red[part][col] = s;
    __syncthreads();
    if (threadIdx.x < D) {
        double t = 0.0;
        for (int q = 0; q < P; ++q) t += red[q][col];
        anchor[(size_t)bh * D + col] = (float)(t / (double)Nv);
    }
}

// Key/value block summaries.  REWEIGHT: x_i = s * a.k_i, m = max x, e_i = exp(x_i - m),
// Z = sum e, k~ = sum e_i k_i / Z, v~ = sum e_i v_i / Z, bias = m + ln Z - s * a.k~.
// MEAN: k~ = mean k, v~ = mean v, bias = ln n.  Both write the plain key mean for ranking.
//
// MODE 1 (pack): the same kernel also writes the block's keys and values into their packed 64-key
// tiles (the layout of pack.hip: K rows as they are, bf16; V^T through LDS; additive term 0 for
// real keys, -inf for padding), so that K and V are read from HBM once for both.
// MODE 2 (amax): it also raises amax_k and amax_v to the block's largest |k| and |v| (E4M3 scales).
template <typename T, int D, int BLK, bool REWEIGHT, int MODE>
__global__ __launch_bounds__(256, 3) void pool_kv_kernel(const T* __restrict__ K, const T* __restrict__ V,
                                                      const float* __restrict__ anchor, int N, int Nv,
                                                      int M, float scale, float* __restrict__ k_mean,
                                                      float* __restrict__ k_sum, float* __restrict__ v_sum,
                                                      float* __restrict__ bias, __bf16* __restrict__ packed,
                                                      float* __restrict__ bias2, float2* __restrict__ tmax, int Tall,
                                                      uint32_t* __restrict__ amax) {
    constexpr bool PACK = MODE == 1;
    using G = PoolGeom<D>;
    constexpr int RPT = (BLK + G::RG - 1) / G::RG;
    const int bh = blockIdx.x / M, J = blockIdx.x % M;
    const int c = threadIdx.x % G::CH, rg = threadIdx.x / G::CH;
    const int lo = J * BLK, n = min(BLK, Nv - lo);
    const size_t off = ((size_t)bh * N + lo) * D + c * 8;

    // every row load is issued first (rows past the block end read its last row, then read as 0)
    Raw8<T> kraw[RPT], vraw[RPT];
#pragma unroll
    for (int k = 0; k < RPT; ++k) {
        const size_t ro = (size_t)min(rg + k * G::RG, n - 1) * D;
        kraw[k].load(K + off + ro);
        vraw[k].load(V + off + ro);
    }
    // rows past the block end are zero from here on; element j of a row is widened where it is used
    // (a shift or a mask for bf16), so the rows stay in registers at their loaded width
#pragma unroll
    for (int k = 0; k < RPT; ++k)
        if (rg + k * G::RG >= n) {
            raw_zero(kraw[k]);
            raw_zero(vraw[k]);
        }
    auto kr = [&](int k, int j) __attribute__((always_inline)) { return raw_elem(kraw[k], j); };
    auto vr = [&](int k, int j) __attribute__((always_inline)) { return raw_elem(vraw[k], j); };

    if constexpr (MODE == 2) {
        float ak = 0.f, av = 0.f;  // rows past the block end are zero here
#pragma unroll
        for (int k = 0; k < RPT; ++k)
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                ak = fmaxf(ak, fabsf(kr(k, j)));
                av = fmaxf(av, fabsf(vr(k, j)));
            }
        ak = wave_max(ak);
        av = wave_max(av);
        __shared__ float wmax[2][4];
        if ((threadIdx.x & 63) == 0) {
            wmax[0][threadIdx.x >> 6] = ak;
            wmax[1][threadIdx.x >> 6] = av;
        }
        __syncthreads();
        if (threadIdx.x < 2) {
            const float* w = wmax[threadIdx.x];
            raise_max_bits(&amax[(size_t)bh * 3 + 1 + threadIdx.x], fmaxf(fmaxf(w[0], w[1]), fmaxf(w[2], w[3])));
        }
    }

    // packed tiles of this key block: K rows straight from the registers, V rows into LDS; per tile
    // the largest squared norm of its keys as stored (bf16), for the attention stage's logit bound
    constexpr int TPB = BLK / 64;  // tiles per key block
    __shared__ __attribute__((aligned(16))) __bf16 vs[PACK ? BLK : 1][D + 8];
    __shared__ float tn2[PACK ? 4 : 1][TPB];
    const size_t tile0 = (size_t)bh * Tall + (size_t)J * TPB;
    if constexpr (PACK) {
        const u32x4 zero = {0u, 0u, 0u, 0u};
        float n2[TPB];
#pragma unroll
        for (int tt = 0; tt < TPB; ++tt) n2[tt] = 0.f;
#pragma unroll
        for (int k = 0; k < RPT; ++k) {
            const int r = rg + k * G::RG;
            if (r < BLK) {
                u32x4 kb = zero, vb = zero;
                if (r < n) {
                    if constexpr (std::is_same<T, __bf16>::value) {
                        kb = kraw[k].u;  // the input bits, unchanged
                        vb = vraw[k].u;
                    } else {
                        float kf[8], vf[8];
                        kraw[k].widen(kf);
                        vraw[k].widen(vf);
                        kb = pack8_bf16(kf);
                        vb = pack8_bf16(vf);
                    }
                }
                *reinterpret_cast<u32x4*>(packed + (tile0 + (r >> 6)) * (2 * 64 * D) + (r & 63) * D + c * 8) = kb;
                *reinterpret_cast<u32x4*>(&vs[r][c * 8]) = vb;
                float s2 = 0.f;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const float lo = bf16_bits_to_f32(kb[j] & 0xffffu), hi = bf16_bits_to_f32(kb[j] >> 16);
                    s2 = fmaf(lo, lo, s2);
                    s2 = fmaf(hi, hi, s2);
                }
                // the CH threads of a row are consecutive lanes of one wave
#pragma unroll
                for (int o = 1; o < G::CH; o <<= 1) s2 += __shfl_xor(s2, o);
                // RG divides 64, so the tile of row rg + k*RG depends on k alone
                n2[(k * G::RG) >> 6] = fmaxf(n2[(k * G::RG) >> 6], s2);
            }
        }
#pragma unroll
        for (int tt = 0; tt < TPB; ++tt) {
            const float v = wave_max(n2[tt]);
            if ((threadIdx.x & 63) == 0) tn2[threadIdx.x >> 6][tt] = v;
        }
    }

    // column sums: first over the row groups of a wave (shuffles), then over the 4 waves (LDS)
    __shared__ float red_k[4][D];
    __shared__ float red_w[4][D];
    __shared__ float red_v[4][D];
    __shared__ float red_s[G::RG];
    __shared__ float bcast[2];

    float ks[8], wk[8], wv[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        ks[j] = 0.f;
#pragma unroll
        for (int k = 0; k < RPT; ++k) ks[j] += kr(k, j);
    }

    float m = 0.f, Z = (float)n;
    if (REWEIGHT) {
        float a[8];
        In<float>::load8(anchor + (size_t)bh * D + c * 8, a);
        float x[RPT];
        float mloc = -INFINITY;
#pragma unroll
        for (int k = 0; k < RPT; ++k) {
            float pd = 0.f;
#pragma unroll
            for (int j = 0; j < 8; ++j) pd += a[j] * kr(k, j);
            // the CH threads of one row group are consecutive lanes of one wave
#pragma unroll
            for (int o = 1; o < G::CH; o <<= 1) pd += __shfl_xor(pd, o);
            const int r = rg + k * G::RG;
            x[k] = r < n ? scale * pd : -INFINITY;
            mloc = fmaxf(mloc, x[k]);
        }
        if (c == 0) red_s[rg] = mloc;
        __syncthreads();
        if (threadIdx.x == 0) {
            float mm = red_s[0];
            for (int g = 1; g < G::RG; ++g) mm = fmaxf(mm, red_s[g]);
            bcast[0] = mm;
        }
        __syncthreads();
        m = bcast[0];
        float zloc = 0.f;
#pragma unroll
        for (int j = 0; j < 8; ++j) { wk[j] = 0.f; wv[j] = 0.f; }
#pragma unroll
        for (int k = 0; k < RPT; ++k) {
            const float e = rg + k * G::RG < n ? expf(x[k] - m) : 0.f;
            zloc += e;
#pragma unroll
            for (int j = 0; j < 8; ++j) { wk[j] += e * kr(k, j); wv[j] += e * vr(k, j); }
        }
        __syncthreads();  // red_s reuse
        if (c == 0) red_s[rg] = zloc;
    } else {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            wk[j] = ks[j];
            wv[j] = 0.f;
#pragma unroll
            for (int k = 0; k < RPT; ++k) wv[j] += vr(k, j);
        }
    }
#pragma unroll
    for (int o = G::CH; o < 64; o <<= 1)  // lanes c + CH * r of a wave hold chunk c of its row groups
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            ks[j] += __shfl_xor(ks[j], o);
            wk[j] += __shfl_xor(wk[j], o);
            wv[j] += __shfl_xor(wv[j], o);
        }
    if ((threadIdx.x & 63) < G::CH) {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            red_k[threadIdx.x >> 6][c * 8 + j] = ks[j];
            red_w[threadIdx.x >> 6][c * 8 + j] = wk[j];
            red_v[threadIdx.x >> 6][c * 8 + j] = wv[j];
        }
    }
    __syncthreads();
    if (REWEIGHT) {
        if (threadIdx.x == 0) {
            float z = 0.f;
            for (int g = 0; g < G::RG; ++g) z += red_s[g];
            bcast[1] = z;
        }
        __syncthreads();
        Z = bcast[1];
    }
    const size_t o = ((size_t)bh * M + J) * D;
    float dot = 0.f;  // a . k~ partial over this thread's columns
    for (int col = threadIdx.x; col < D; col += 256) {
        float sk = 0.f, sw = 0.f, sv = 0.f;
        for (int g = 0; g < 4; ++g) { sk += red_k[g][col]; sw += red_w[g][col]; sv += red_v[g][col]; }
        const float kt = sw / Z;
        k_mean[o + col] = sk / (float)n;
        k_sum[o + col] = kt;
        v_sum[o + col] = sv / Z;
        if (REWEIGHT) dot += anchor[(size_t)bh * D + col] * kt;
    }
    if (REWEIGHT) {
        // D <= 256 columns live in the first D threads: waves 0 (and 1 for D = 128)
        dot = wave_sum(dot);
        __syncthreads();
        if ((threadIdx.x & 63) == 0) red_s[threadIdx.x >> 6] = dot;
        __syncthreads();
        if (threadIdx.x == 0) {
            float t = 0.f;
            for (int w = 0; w < 4; ++w) t += red_s[w];
            bias[(size_t)bh * M + J] = m + logf(Z) - scale * t;
        }
    } else if (threadIdx.x == 0) {
        bias[(size_t)bh * M + J] = logf((float)n);
    }
    if constexpr (PACK) {
        __syncthreads();  // every V row is in LDS
        // V^T row dr of tile tt = keys 0..63 of dimension dr: 8 chunks of 8 keys
#pragma unroll
        for (int tt = 0; tt < TPB; ++tt) {
            __bf16* vdst = packed + (tile0 + tt) * (2 * 64 * D) + 64 * D;
            for (int e = threadIdx.x; e < D * 8; e += 256) {
                const int dr = e / 8, kc = e % 8;
                u32x4 o;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const uint32_t lo = __builtin_bit_cast(uint16_t, vs[tt * 64 + kc * 8 + 2 * j][dr]);
                    const uint32_t hi = __builtin_bit_cast(uint16_t, vs[tt * 64 + kc * 8 + 2 * j + 1][dr]);
                    o[j] = lo | (hi << 16);
                }
                *reinterpret_cast<u32x4*>(vdst + dr * 64 + kc * 8) = o;
            }
            if (threadIdx.x < 64) bias2[(tile0 + tt) * 64 + threadIdx.x] = tt * 64 + (int)threadIdx.x < n ? 0.f : -INFINITY;
            if (threadIdx.x == 0)
                tmax[tile0 + tt] = make_float2(fmaxf(fmaxf(tn2[0][tt], tn2[1][tt]), fmaxf(tn2[2][tt], tn2[3][tt])),
                                               tt * 64 < n ? 0.f : -INFINITY);
        }
    }
}

// Query means (and the anchor) over the L.M query blocks of L.block rows; key summaries over the
// L.Mk key blocks of L.block_k keys.
template <typename T, int D, int BLK>
static void launch_pool_q_t(const LaunchCtx& L, const void* Q, float* q_mean, float* anchor, uint32_t* amax) {
    if (amax)
        hipLaunchKernelGGL((pool_q_kernel<T, D, BLK, true>), dim3(L.BH * L.M), dim3(256), 0, L.stream, (const T*)Q,
                           L.N, L.Nv, L.M, q_mean, amax);
    else
        hipLaunchKernelGGL((pool_q_kernel<T, D, BLK, false>), dim3(L.BH * L.M), dim3(256), 0, L.stream,
                           (const T*)Q, L.N, L.Nv, L.M, q_mean, nullptr);
    hipLaunchKernelGGL((anchor_kernel<D>), dim3(L.BH), dim3(kAnchorThreads), 0, L.stream, q_mean, L.Nv, L.M,
                       BLK, anchor);
}

template <typename T, int D, int BLK, int MODE>
static void launch_pool_kv_t(const LaunchCtx& L, const void* K, const void* V, const float* anchor,
                             float* k_mean, float* k_sum, float* v_sum, float* bias, void* packed,
                             uint32_t* amax) {
    const dim3 grid(L.BH * L.Mk);
    __bf16* kv = nullptr;
    float* b2 = nullptr;
    float2* tm = nullptr;
    int Tall = 0;
    if (MODE == 1) {
        const PackGeom g = pack_geom(L);
        kv = (__bf16*)packed;
        b2 = (float*)((char*)packed + g.bias_off);
        tm = (float2*)((char*)packed + g.tmax_off);
        Tall = g.Tall;
    }
    if (L.pool_mode == SPARK_ATTN_POOL_REWEIGHT)
        hipLaunchKernelGGL((pool_kv_kernel<T, D, BLK, true, MODE>), grid, dim3(256), 0, L.stream, (const T*)K,
                           (const T*)V, anchor, L.N, L.Nv, L.Mk, L.scale, k_mean, k_sum, v_sum, bias, kv, b2, tm,
                           Tall, amax);
    else
        hipLaunchKernelGGL((pool_kv_kernel<T, D, BLK, false, MODE>), grid, dim3(256), 0, L.stream, (const T*)K,
                           (const T*)V, anchor, L.N, L.Nv, L.Mk, L.scale, k_mean, k_sum, v_sum, bias, kv, b2, tm,
                           Tall, amax);
}

template <typename T, int D>
static void launch_pool_t(const LaunchCtx& L, const void* Q, const void* K, const void* V, float* q_mean,
                          float* k_mean, float* k_sum, float* v_sum, float* bias, float* anchor, void* packed,
                          uint32_t* amax) {
    if (L.block == 64) launch_pool_q_t<T, D, 64>(L, Q, q_mean, anchor, amax);
    else launch_pool_q_t<T, D, 128>(L, Q, q_mean, anchor, amax);
#define SPARK_POOL_KV(MODE)                                                                                    \
    if (L.block_k == 64) launch_pool_kv_t<T, D, 64, MODE>(L, K, V, anchor, k_mean, k_sum, v_sum, bias, packed, amax); \
    else launch_pool_kv_t<T, D, 128, MODE>(L, K, V, anchor, k_mean, k_sum, v_sum, bias, packed, amax);
    if (packed) { SPARK_POOL_KV(1) }
    else if (amax) { SPARK_POOL_KV(2) }
    else { SPARK_POOL_KV(0) }
#undef SPARK_POOL_KV
}

static void launch_pool_any(const LaunchCtx& L, const void* Q, const void* K, const void* V, float* q_mean,
                            float* k_mean, float* k_sum, float* v_sum, float* bias, float* anchor, void* packed,
                            uint32_t* amax) {
    if (L.dtype == SPARK_ATTN_BF16) {
        if (L.d == 64) launch_pool_t<__bf16, 64>(L, Q, K, V, q_mean, k_mean, k_sum, v_sum, bias, anchor, packed, amax);
        else launch_pool_t<__bf16, 128>(L, Q, K, V, q_mean, k_mean, k_sum, v_sum, bias, anchor, packed, amax);
    } else {
        if (L.d == 64) launch_pool_t<float, 64>(L, Q, K, V, q_mean, k_mean, k_sum, v_sum, bias, anchor, packed, amax);
        else launch_pool_t<float, 128>(L, Q, K, V, q_mean, k_mean, k_sum, v_sum, bias, anchor, packed, amax);
    }
}

void launch_pool(const LaunchCtx& L, const void* Q, const void* K, const void* V, float* q_mean,
                 float* k_mean, float* k_sum, float* v_sum, float* bias, float* anchor) {
    launch_pool_any(L, Q, K, V, q_mean, k_mean, k_sum, v_sum, bias, anchor, nullptr, nullptr);
}

// Pooling and the per-head E4M3 amax of Q, K and V in one pass over the video rows (the sink rows,
// which pooling does not read, by the amax kernel).
void launch_pool_fp8_scales(const LaunchCtx& L, const void* Q, const void* K, const void* V, float* q_mean,
                            float* k_mean, float* k_sum, float* v_sum, float* bias, float* anchor, uint32_t* amax) {
    launch_fp8_amax_rows(L, Q, K, V, amax, L.Nv);  // zeroes amax, then the rows Nv .. N-1
    launch_pool_any(L, Q, K, V, q_mean, k_mean, k_sum, v_sum, bias, anchor, nullptr, amax);
}

// Pool and pack in one pass over K and V: the video key tiles are written by the pooling kernel,
// then the sink tiles and the compressed tiles (which need the summaries) by the pack kernels.
void launch_pool_pack(const LaunchCtx& L, const void* Q, const void* K, const void* V, float* q_mean,
                      float* k_mean, float* k_sum, float* v_sum, float* bias, float* anchor, void* packed) {
    launch_pool_any(L, Q, K, V, q_mean, k_mean, k_sum, v_sum, bias, anchor, packed, nullptr);
    launch_pack_rest(L, K, V, k_sum, v_sum, bias, packed);
}

}  // namespace spark
