// Two-branch block-sparse attention forward on bf16 MFMA (gfx950).
//
// Spark-H3 page, section "Spark-Attnが変えるもの": the exact branch attends fully to the
// top-ranked key/value blocks and the compressed branch covers every other block cheaply; here the
// compressed branch is one pseudo-key per unselected block (logit s*q.k~_J + bias_J, value v~_J)
// folded into the SAME online-softmax state as the exact keys, so the branches merge exactly by
// log-sum-exp.  Core node page, section "ブロックスパースアテンション": sink_conditioning rows are
// attended exactly by every query.  H3 Optimizations README, "Nodes": non-video (sink) queries are
// dense over all keys.
//
// One workgroup = one query block (BLK rows) of one (batch, head); BLK/32 waves, each owning 32
// query rows.  For every KV tile of 64 keys (a half or whole selected block, a sink tile, or 64
// compressed pseudo-keys) the wave computes S^T = K_tile Q^T with v_mfma_f32_32x32x16_bf16, so
// each lane ends up holding one query's logits (lane % 32 = query, 32 keys per lane): the row max
// and row sum need only one cross-half shuffle, and P is already laid out as the B operand of
// O^T += V^T P^T.  K tiles are staged row-major in LDS, V tiles transposed (d-major) in LDS; the
// next tile's global loads are issued before the current tile's math (register prefetch).
#include "kernels.hpp"

namespace spark {

template <int D, int BLK> struct AttnGeom {
    static constexpr int NW = BLK / 32;       // waves per workgroup
    static constexpr int NT = NW * kWave;     // threads
    static constexpr int TK = 64;             // keys per tile
    static constexpr int NC = TK / 32;        // 32-key chunks per tile (one MFMA output tile each)
    static constexpr int KST = D + 8;         // row stride of the K tile in LDS (bf16 elements)
    static constexpr int VST = TK + 4;        // row stride of the V^T tile in LDS (bf16 elements)
    static constexpr int KCHUNKS = TK * D / 8;           // 16-byte chunks of a K tile
    static constexpr int VGROUPS = (TK / 4) * (D / 8);   // 4-key x 8-dim groups of a V tile
    static constexpr int KCH = (KCHUNKS + NT - 1) / NT;  // per thread
    static constexpr int VGR = (VGROUPS + NT - 1) / NT;  // per thread
    static_assert(NT >= TK, "bias staging needs one thread per key");
};

enum TileKind { kTileKV = 0, kTileCompressed = 1 };

struct TileDesc {
    int kind;
    int row0;    // first key row (K/V rows) or first pseudo-key (compressed)
    int nvalid;  // valid keys in the tile (<= 0: fully masked)
};

template <typename T, int D, int BLK>
struct TileRegs {
    using G = AttnGeom<D, BLK>;
    u32x4 k[G::KCH];
    u32x4 v[G::VGR][4];
    float bias;  // per-key additive logit term (log2 units) for thread t < TK
};

template <typename T, int D, int BLK>
__device__ __forceinline__ void load_tile(TileRegs<T, D, BLK>& R, const TileDesc& td, const T* Kh,
                                          const T* Vh, const float* ksum_h, const float* vsum_h,
                                          const float* bias_h, const uint32_t* sel_bits, int M) {
    using G = AttnGeom<D, BLK>;
    const int t = threadIdx.x;
    constexpr int CPR = D / 8;  // 16-byte chunks per row
    const u32x4 zero = {0u, 0u, 0u, 0u};
    if (td.kind == kTileKV) {
#pragma unroll
        for (int i = 0; i < G::KCH; ++i) {
            const int e = t + i * G::NT, r = e / CPR, c = e % CPR;
            if (e >= G::KCHUNKS) break;
            R.k[i] = r < td.nvalid ? load8_as_bf16<T>(Kh + (size_t)(td.row0 + r) * D + c * 8) : zero;
        }
#pragma unroll
        for (int i = 0; i < G::VGR; ++i) {
            const int g = t + i * G::NT, c = g % CPR, kg = g / CPR;
            if (g >= G::VGROUPS) break;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int r = kg * 4 + j;
                R.v[i][j] = r < td.nvalid ? load8_as_bf16<T>(Vh + (size_t)(td.row0 + r) * D + c * 8) : zero;
            }
        }
        if (t < G::TK) R.bias = t < td.nvalid ? 0.f : -INFINITY;
    } else {
#pragma unroll
        for (int i = 0; i < G::KCH; ++i) {
            const int e = t + i * G::NT, r = e / CPR, c = e % CPR;
            if (e >= G::KCHUNKS) break;
            R.k[i] = r < td.nvalid ? load8_as_bf16<float>(ksum_h + (size_t)(td.row0 + r) * D + c * 8) : zero;
        }
#pragma unroll
        for (int i = 0; i < G::VGR; ++i) {
            const int g = t + i * G::NT, c = g % CPR, kg = g / CPR;
            if (g >= G::VGROUPS) break;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int r = kg * 4 + j;
                R.v[i][j] = r < td.nvalid ? load8_as_bf16<float>(vsum_h + (size_t)(td.row0 + r) * D + c * 8) : zero;
            }
        }
        if (t < G::TK) {
            const int J = td.row0 + t;
            const bool live = t < td.nvalid && !((sel_bits[J >> 5] >> (J & 31)) & 1u);
            R.bias = live ? bias_h[J] * 1.4426950408889634f : -INFINITY;
        }
    }
}

template <typename T, int D, int BLK>
__device__ __forceinline__ void store_tile(const TileRegs<T, D, BLK>& R, __bf16* Ks, __bf16* Vt, float* bias_s) {
    using G = AttnGeom<D, BLK>;
    const int t = threadIdx.x;
    constexpr int CPR = D / 8;
#pragma unroll
    for (int i = 0; i < G::KCH; ++i) {
        const int e = t + i * G::NT, r = e / CPR, c = e % CPR;
        if (e >= G::KCHUNKS) break;
        *reinterpret_cast<u32x4*>(Ks + r * G::KST + c * 8) = R.k[i];
    }
#pragma unroll
    for (int i = 0; i < G::VGR; ++i) {
        const int g = t + i * G::NT, c = g % CPR, kg = g / CPR;
        if (g >= G::VGROUPS) break;
        // rows kg*4 .. kg*4+3 of V, dims c*8 .. c*8+7  ->  V^T rows c*8+e, keys kg*4 .. kg*4+3
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int w = e >> 1, sh = (e & 1) * 16;
            const uint32_t x0 = (R.v[i][0][w] >> sh) & 0xffffu, x1 = (R.v[i][1][w] >> sh) & 0xffffu;
            const uint32_t x2 = (R.v[i][2][w] >> sh) & 0xffffu, x3 = (R.v[i][3][w] >> sh) & 0xffffu;
            u32x2 pk;
            pk[0] = x0 | (x1 << 16);
            pk[1] = x2 | (x3 << 16);
            *reinterpret_cast<u32x2*>(Vt + (c * 8 + e) * G::VST + kg * 4) = pk;
        }
    }
    if (t < G::TK) bias_s[t] = R.bias;
}

template <typename T, int D, int BLK>
__global__ __launch_bounds__(BLK * 2, 2) void attn_fwd_kernel(
    const T* __restrict__ Q, const T* __restrict__ K, const T* __restrict__ V, const float* __restrict__ k_sum,
    const float* __restrict__ v_sum, const float* __restrict__ bias, const int32_t* __restrict__ idx,
    const int32_t* __restrict__ perm, T* __restrict__ O, float* __restrict__ lse, int N, int Nv, int M,
    int Ksel, int SQ, int BH, float c_log2) {
    using G = AttnGeom<D, BLK>;
    __shared__ __attribute__((aligned(16))) __bf16 Ks[G::TK * G::KST];
    __shared__ __attribute__((aligned(16))) __bf16 Vt[D * G::VST];
    __shared__ __attribute__((aligned(16))) float bias_s[G::TK];
    __shared__ uint32_t sel_bits[kMaxBlocks / 32];

    // --- which query tile: sink-query tiles (dense, longest) come first in the grid
    int bh, qrow0, nq, ntiles;
    bool dense;
    {
        const int wg = blockIdx.x;
        if (wg < BH * SQ) {
            dense = true;
            bh = wg / SQ;
            qrow0 = Nv + (wg % SQ) * BLK;
            nq = min(BLK, N - qrow0);
            ntiles = (N + G::TK - 1) / G::TK;
        } else {
            dense = false;
            const int v = wg - BH * SQ;
            bh = v / M;
            const int I = v % M;
            qrow0 = I * BLK;
            nq = min(BLK, Nv - qrow0);
            ntiles = Ksel * (BLK / G::TK) + (N - Nv + G::TK - 1) / G::TK + (M + G::TK - 1) / G::TK;
        }
    }
    const size_t head = (size_t)bh * N * D;
    const T* Qh = Q + head;
    const T* Kh = K + head;
    const T* Vh = V + head;
    const float* ksum_h = k_sum + (size_t)bh * M * D;
    const float* vsum_h = v_sum + (size_t)bh * M * D;
    const float* bias_h = bias + (size_t)bh * M;
    const int32_t* sel = dense ? nullptr : idx + ((size_t)bh * M + qrow0 / BLK) * Ksel;

    if (!dense) {
        for (int w = threadIdx.x; w < (M + 31) / 32; w += G::NT) sel_bits[w] = 0u;
        __syncthreads();
        for (int k = threadIdx.x; k < Ksel; k += G::NT) {
            const int J = sel[k];
            atomicOr(&sel_bits[J >> 5], 1u << (J & 31));
        }
        __syncthreads();
    }

    const int nsub = BLK / G::TK;
    const int n_exact = dense ? 0 : Ksel * nsub;
    const int n_sinkt = dense ? 0 : (N - Nv + G::TK - 1) / G::TK;
    auto desc = [&](int t) -> TileDesc {
        TileDesc td;
        if (dense) {
            td.kind = kTileKV;
            td.row0 = t * G::TK;
            td.nvalid = min(G::TK, N - td.row0);
        } else if (t < n_exact) {
            const int J = sel[t / nsub], sub = t % nsub;
            const int nJ = min(BLK, Nv - J * BLK);
            td.kind = kTileKV;
            td.row0 = J * BLK + sub * G::TK;
            td.nvalid = min(G::TK, nJ - sub * G::TK);
        } else if (t < n_exact + n_sinkt) {
            td.kind = kTileKV;
            td.row0 = Nv + (t - n_exact) * G::TK;
            td.nvalid = min(G::TK, N - td.row0);
        } else {
            td.kind = kTileCompressed;
            td.row0 = (t - n_exact - n_sinkt) * G::TK;
            td.nvalid = min(G::TK, M - td.row0);
        }
        return td;
    };

    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int i32 = lane & 31, h = lane >> 5;

    // Q rows of this wave as the B operand of S^T = K Q^T: lane (i32, h) holds row w*32 + i32,
    // dims ds*16 + 8h .. +8 for each 16-wide k step ds.
    bf16x8 qreg[D / 16];
    {
        const int qr = w * 32 + i32;
        const T* src = Qh + (size_t)(qrow0 + qr) * D;
#pragma unroll
        for (int ds = 0; ds < D / 16; ++ds) {
            u32x4 u = {0u, 0u, 0u, 0u};
            if (qr < nq) u = load8_as_bf16<T>(src + ds * 16 + 8 * h);
            qreg[ds] = __builtin_bit_cast(bf16x8, u);
        }
    }

    f32x16 acc[D / 32];
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[dt][r] = 0.f;
    float m_run = -INFINITY, l_run = 0.f;

    TileRegs<T, D, BLK> R;
    load_tile<T, D, BLK>(R, desc(0), Kh, Vh, ksum_h, vsum_h, bias_h, sel_bits, M);

    for (int t = 0; t < ntiles; ++t) {
        __syncthreads();
        store_tile<T, D, BLK>(R, Ks, Vt, bias_s);
        __syncthreads();
        if (t + 1 < ntiles) load_tile<T, D, BLK>(R, desc(t + 1), Kh, Vh, ksum_h, vsum_h, bias_h, sel_bits, M);

        // ---- S^T = K_tile Q^T : G::NC chunks of 32 keys x 32 queries
        f32x16 st[G::NC];
#pragma unroll
        for (int c = 0; c < G::NC; ++c) {
            f32x16 s;
#pragma unroll
            for (int r = 0; r < 16; ++r) s[r] = 0.f;
#pragma unroll
            for (int ds = 0; ds < D / 16; ++ds) {
                const bf16x8 a = *reinterpret_cast<const bf16x8*>(Ks + (c * 32 + i32) * G::KST + ds * 16 + 8 * h);
                s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qreg[ds], s, 0, 0, 0);
            }
            st[c] = s;
        }
        // ---- logits in log2 units; lane holds keys c*32 + 8*(r/4) + 4*h + r%4 of query i32
        float mx = -INFINITY;
#pragma unroll
        for (int c = 0; c < G::NC; ++c)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const f32x4 bb = *reinterpret_cast<const f32x4*>(bias_s + c * 32 + 8 * g + 4 * h);
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const float z = fmaf(st[c][4 * g + j], c_log2, bb[j]);
                    st[c][4 * g + j] = z;
                    mx = fmaxf(mx, z);
                }
            }
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const float m_new = fmaxf(m_run, mx);
        const float m_use = m_new == -INFINITY ? 0.f : m_new;
        const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
        float ls = 0.f;
#pragma unroll
        for (int c = 0; c < G::NC; ++c)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const float p = __builtin_amdgcn_exp2f(st[c][r] - m_use);
                st[c][r] = p;
                ls += p;
            }
        l_run = l_run * alpha + ls;
        m_run = m_new;
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[dt][r] *= alpha;

        // ---- O^T += V^T P^T, 16 keys per MFMA step: P regs 8*(kt%2) .. +7 of chunk kt/2 hold keys
        // 16*kt + 8*(e/4) + 4*h + e%4 (e = 0..7); V^T is read for exactly those keys.
#pragma unroll
        for (int kt = 0; kt < G::TK / 16; ++kt) {
            bf16x8 b;
#pragma unroll
            for (int e = 0; e < 8; ++e) b[e] = (__bf16)st[kt >> 1][8 * (kt & 1) + e];
#pragma unroll
            for (int dt = 0; dt < D / 32; ++dt) {
                const __bf16* vrow = Vt + (dt * 32 + i32) * G::VST + 16 * kt + 4 * h;
                const bf16x4 lo = *reinterpret_cast<const bf16x4*>(vrow);
                const bf16x4 hi = *reinterpret_cast<const bf16x4*>(vrow + 8);
                const bf16x8 a = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
                acc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[dt], 0, 0, 0);
            }
        }
    }

    // ---- epilogue: lane (i32, h) holds query row w*32 + i32, dims dt*32 + 8*g + 4*h + (0..3)
    const float l_tot = l_run + __shfl_xor(l_run, 32);
    const float inv = 1.f / l_tot;
    const int qr = w * 32 + i32;
    if (qr < nq) {
        const int row = qrow0 + qr;
        const int orow = (!dense && perm) ? perm[(size_t)bh * Nv + row] : row;
        T* dst = O + head + (size_t)orow * D;
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int col = dt * 32 + 8 * g + 4 * h;
                if constexpr (sizeof(T) == 2) {
                    bf16x4 o;
#pragma unroll
                    for (int j = 0; j < 4; ++j) o[j] = (__bf16)(acc[dt][4 * g + j] * inv);
                    *reinterpret_cast<bf16x4*>(dst + col) = o;
                } else {
                    f32x4 o;
#pragma unroll
                    for (int j = 0; j < 4; ++j) o[j] = acc[dt][4 * g + j] * inv;
                    *reinterpret_cast<f32x4*>(dst + col) = o;
                }
            }
        if (lse && h == 0) lse[(size_t)bh * N + orow] = (m_run + log2f(l_tot)) * 0.6931471805599453f;
    }
}

template <typename T, int D, int BLK>
static void launch_attend_t(const LaunchCtx& L, const void* Q, const void* K, const void* V, const float* k_sum,
                            const float* v_sum, const float* bias, const int32_t* idx, const int32_t* perm,
                            void* O, float* lse) {
    using G = AttnGeom<D, BLK>;
    const int SQ = (L.n_sink + BLK - 1) / BLK;
    const dim3 grid(L.BH * (SQ + L.M));
    const float c_log2 = L.scale * 1.4426950408889634f;
    hipLaunchKernelGGL((attn_fwd_kernel<T, D, BLK>), grid, dim3(G::NT), 0, L.stream, (const T*)Q, (const T*)K,
                       (const T*)V, k_sum, v_sum, bias, idx, perm, (T*)O, lse, L.N, L.Nv, L.M, L.K, SQ, L.BH,
                       c_log2);
}

void launch_attend(const LaunchCtx& L, const void* Q, const void* K, const void* V, const float* k_sum,
                   const float* v_sum, const float* bias, const int32_t* idx, const int32_t* perm, void* O,
                   float* lse) {
#define SPARK_ATTN_CASE(T, D, B)                                                                  \
    if (L.d == D && L.block == B) {                                                               \
        launch_attend_t<T, D, B>(L, Q, K, V, k_sum, v_sum, bias, idx, perm, O, lse);              \
        return;                                                                                   \
    }
    if (L.dtype == SPARK_ATTN_BF16) {
        SPARK_ATTN_CASE(__bf16, 64, 64) SPARK_ATTN_CASE(__bf16, 64, 128)
        SPARK_ATTN_CASE(__bf16, 128, 64) SPARK_ATTN_CASE(__bf16, 128, 128)
    } else {
        SPARK_ATTN_CASE(float, 64, 64) SPARK_ATTN_CASE(float, 64, 128)
        SPARK_ATTN_CASE(float, 128, 64) SPARK_ATTN_CASE(float, 128, 128)
    }
#undef SPARK_ATTN_CASE
}

}  // namespace spark
