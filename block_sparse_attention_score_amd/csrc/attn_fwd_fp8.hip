// Two-branch block-sparse attention forward on E4M3 (FP8) carriers, gfx950 FP8 MFMA.
//
// H3 Optimizations README, section "Manual Sparse Sage recovery" (the FP8 FlexAttention fallback):
// queries, keys and values are carried as E4M3 with one scale per head, the Q/K scale is restored
// before the softmax, the output returns in the original floating type, and the route is the one
// the bf16 path uses.  Per (batch, head) and tensor, amax = max |x| over all N rows; in binary32
// r = 448 / amax and s = amax / 448 (1 and 1 when amax = 0); the carrier of x is e4m3(x * r) (the
// product rounded to binary32, then to the nearest E4M3 value, ties to even: v_cvt_pk_fp8_f32).
// The compressed pseudo-keys ride on the keys' and values' scales.  Every logit is
// scale * s_Q * s_K * (q8 . k8) (+ the pseudo-key's bias) and every value s_V * v8.
//
// The kernel follows the bf16 kernel's design (one workgroup per query block, tiles streamed
// HBM -> LDS with buffer_load ... lds into two stages, K one tile ahead of V, scores of tile t+1
// computed while tile t is applied) with these differences:
//  * A packed tile is [K rows: 64 x d bytes | V^T: d x 64 bytes] (half the bf16 bytes) plus the
//    same fp32 bias row.
//  * S^T = K Q^T and O^T += V^T P^T both run on v_mfma_f32_32x32x64_f8f6f4 (E4M3 x E4M3).  Lane
//    (i32, h) of either operand holds row i32 and the 32 bytes 32h .. 32h+31 of its 64-deep k
//    range.  The S^T accumulator of lane (i32, h) holds, for query i32, keys 32c + 8g + 4h + j
//    in register 4g + j of chunk c; the V^T columns of a tile are stored in the order that makes
//    byte 16c + 4g + j of the P^T operand of that lane exactly that key, so the probabilities
//    feed the PV product straight from registers.
//  * Probabilities are bounded by 2^8 (the running max is raised once a tile exceeds it by more
//    than 8 in log2 units), inside the E4M3 range; they are rounded to E4M3 for the PV product,
//    while the normaliser sums them before rounding.
#include <type_traits>

#include <algorithm>

#include "kernels.hpp"

namespace spark {

typedef int i32x8 __attribute__((ext_vector_type(8)));

constexpr int kTK8 = 64;               // keys per tile
constexpr float kRescaleSlack8 = 8.f;  // log2-domain slack before the running max is raised

// ---------------------------------------------------------------------------------------------
// Per-head scales.

__global__ __launch_bounds__(256) void fp8_zero_kernel(uint32_t* __restrict__ p, int n) {
    const int i = blockIdx.x * 256 + threadIdx.x;
    if (i < n) p[i] = 0u;
}

// amax[bh][t] (float bits; non-negative floats order as unsigned integers) of tensor t = Q, K, V
// raised to the largest |x| over rows row0 .. N-1 of (batch, head) bh.
template <typename T>
__global__ __launch_bounds__(256) void fp8_amax_kernel(const T* __restrict__ Q, const T* __restrict__ K,
                                                       const T* __restrict__ V, int N, int row0, int d,
                                                       uint32_t* __restrict__ amax) {
    const int bh = blockIdx.y, t = blockIdx.z;
    const T* x = (t == 0 ? Q : t == 1 ? K : V) + ((size_t)bh * N + row0) * d;
    const size_t n8 = (size_t)(N - row0) * d / 8;
    float m = 0.f;
    for (size_t e = (size_t)blockIdx.x * 256 + threadIdx.x; e < n8; e += (size_t)gridDim.x * 256) {
        Raw8<T> r;
        r.load(x + 8 * e);
        float v[8];
        r.widen(v);
#pragma unroll
        for (int j = 0; j < 8; ++j) m = fmaxf(m, fabsf(v[j]));
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
    if ((threadIdx.x & 63) == 0) atomicMax(&amax[bh * 3 + t], __float_as_uint(m));
}

// r = 448 / amax and s = amax / 448, both correctly rounded binary32 (1 and 1 when amax = 0).
__device__ __forceinline__ float fp8_r(uint32_t amax_bits) {
    const float a = __uint_as_float(amax_bits);
    return a > 0.f ? __fdiv_rn(448.f, a) : 1.f;
}
__device__ __forceinline__ float fp8_s(uint32_t amax_bits) {
    const float a = __uint_as_float(amax_bits);
    return a > 0.f ? __fdiv_rn(a, 448.f) : 1.f;
}

// Four binary32 values to four E4M3 bytes (round to nearest even), in order.  The first
// conversion writes the low half of the word and keeps the high half of its third operand, which
// the second conversion then replaces: any value serves there, and passing a's own bits (rather
// than a literal 0) lets the result take a's register instead of a freshly cleared one.
__device__ __forceinline__ uint32_t fp8x4(float a, float b, float c, float e) {
    const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, __builtin_bit_cast(int, a), false);
    return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(c, e, lo, true);
}

// ---------------------------------------------------------------------------------------------
// Packing.  V^T column kap = 32h + 16c + 4g + j of a tile holds key 32c + 8g + 4h + j.
__device__ __forceinline__ int fp8_vt_key(int kap) {
    const int h = kap >> 5, c = (kap >> 4) & 1, g = (kap >> 2) & 3, j = kap & 3;
    return 32 * c + 8 * g + 4 * h + j;
}

PackGeom pack_geom_fp8(const LaunchCtx& L) {
    PackGeom g = pack_geom(L);
    g.tile_elems = (size_t)2 * 64 * L.d;  // bytes of a tile (one byte per element)
    g.kv_bytes = (size_t)L.BH * g.Tall * g.tile_elems;
    g.bias_off = (g.kv_bytes + 255) & ~(size_t)255;
    g.queue_off = (g.bias_off + (size_t)L.BH * g.Tall * 64 * 4 + 255) & ~(size_t)255;
    g.bytes = g.queue_off + 8 * 4;
    return g;
}

// One workgroup per tile of 64 source rows (real keys of type S, or the fp32 summaries).
template <typename S, int D>
__device__ __forceinline__ void pack_tile_fp8(const S* __restrict__ Ksrc, const S* __restrict__ Vsrc, int nvalid,
                                              float rk, float rv, uint8_t* __restrict__ tile,
                                              float* __restrict__ bias2, const float* __restrict__ bias_src,
                                              float bias_scale) {
    __shared__ __attribute__((aligned(16))) uint8_t vs[64][D + 4];
    constexpr int C8 = D / 8;  // eight-element groups per row
    const int t = threadIdx.x;
    for (int e = t; e < 64 * C8; e += 256) {
        const int r = e / C8, c8 = (e % C8) * 8;
        float kv[8] = {}, vv[8] = {};
        if (r < nvalid) {
            Raw8<S> a, b;
            a.load(Ksrc + (size_t)r * D + c8);
            b.load(Vsrc + (size_t)r * D + c8);
            a.widen(kv);
            b.widen(vv);
        }
        uint2 ko, vo;
        ko.x = fp8x4(kv[0] * rk, kv[1] * rk, kv[2] * rk, kv[3] * rk);
        ko.y = fp8x4(kv[4] * rk, kv[5] * rk, kv[6] * rk, kv[7] * rk);
        vo.x = fp8x4(vv[0] * rv, vv[1] * rv, vv[2] * rv, vv[3] * rv);
        vo.y = fp8x4(vv[4] * rv, vv[5] * rv, vv[6] * rv, vv[7] * rv);
        *reinterpret_cast<uint2*>(tile + r * D + c8) = ko;
        *reinterpret_cast<uint32_t*>(&vs[r][c8]) = vo.x;
        *reinterpret_cast<uint32_t*>(&vs[r][c8 + 4]) = vo.y;
    }
    __syncthreads();
    // V^T row dr: 64 bytes, column kap from key fp8_vt_key(kap); 16 bytes per thread and step
    uint8_t* vdst = tile + 64 * D;
    for (int e = t; e < D * 4; e += 256) {
        const int dr = e / 4, k16 = (e % 4) * 16;
        uint32_t w[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            uint32_t x = 0;
#pragma unroll
            for (int b = 0; b < 4; ++b) x |= (uint32_t)vs[fp8_vt_key(k16 + 4 * q + b)][dr] << (8 * b);
            w[q] = x;
        }
        *reinterpret_cast<u32x4*>(vdst + dr * 64 + k16) = u32x4{w[0], w[1], w[2], w[3]};
    }
    if (t < 64) {
        float b = -INFINITY;
        if (t < nvalid) b = bias_src ? bias_src[t] * bias_scale : 0.f;
        bias2[t] = b;
    }
}

template <typename T, int D>
__global__ __launch_bounds__(256) void pack_keys_fp8_kernel(const T* __restrict__ K, const T* __restrict__ V, int N,
                                                            int Nv, int Tv, int Ts, int Tall,
                                                            const uint32_t* __restrict__ amax,
                                                            uint8_t* __restrict__ packed, float* __restrict__ bias2) {
    const int per = Tv + Ts;
    const int bh = blockIdx.x / per, t = blockIdx.x % per;
    int row0, nvalid;
    if (t < Tv) {
        row0 = t * 64;
        nvalid = min(64, Nv - row0);
    } else {
        row0 = Nv + (t - Tv) * 64;
        nvalid = min(64, N - row0);
    }
    const size_t src = ((size_t)bh * N + row0) * D;
    const size_t tile = (size_t)bh * Tall + t;
    pack_tile_fp8<T, D>(K + src, V + src, nvalid, fp8_r(amax[bh * 3 + 1]), fp8_r(amax[bh * 3 + 2]),
                        packed + tile * (2 * 64 * D), bias2 + tile * 64, nullptr, 0.f);
}

template <int D>
__global__ __launch_bounds__(256) void pack_compressed_fp8_kernel(const float* __restrict__ k_sum,
                                                                  const float* __restrict__ v_sum,
                                                                  const float* __restrict__ bias, int M, int Tv,
                                                                  int Ts, int Tc, int Tall,
                                                                  const uint32_t* __restrict__ amax,
                                                                  uint8_t* __restrict__ packed,
                                                                  float* __restrict__ bias2) {
    const int bh = blockIdx.x / Tc, c = blockIdx.x % Tc;
    const int J0 = c * 64, nvalid = min(64, M - J0);
    const size_t src = ((size_t)bh * M + J0) * D;
    const size_t tile = (size_t)bh * Tall + Tv + Ts + c;
    pack_tile_fp8<float, D>(k_sum + src, v_sum + src, nvalid, fp8_r(amax[bh * 3 + 1]), fp8_r(amax[bh * 3 + 2]),
                            packed + tile * (2 * 64 * D), bias2 + tile * 64, bias + (size_t)bh * M + J0,
                            1.4426950408889634f);
}

// ---------------------------------------------------------------------------------------------
// Attention.

template <int D> struct TileGeom8 {
    static constexpr int CK = D / 16;            // 16-byte chunks per K row
    static constexpr int BYTES = 2 * kTK8 * D;   // bytes of a packed tile
    static constexpr int K_CHUNKS = kTK8 * CK;   // chunks of the K part (= chunks of the V part)
    static constexpr int V_CPR = kTK8 / 16;      // chunks per V^T row (4)
};

// Chunk swizzle of an LDS row: rows of 8 chunks use (row / 2) % 8, rows of 4 chunks (row / 4) % 4,
// so 16 consecutive rows read at one logical chunk hit 16 distinct bank groups.
template <int CPR>
__device__ __forceinline__ int swz8(int row) {
    return CPR == 8 ? ((row >> 1) & 7) : ((row >> 2) & 3);
}

typedef __attribute__((address_space(3))) void* lds_ptr8;

// HBM -> LDS copy of one half (K rows, or V^T rows) of a packed tile: lane tid moves the chunks
// i*NT + tid (i < 4D/NT).  The swizzle repeats every 16 rows and NT spans a multiple of 16 rows of
// either half, so source chunk(i*NT + tid) = chunk(tid) + i*NT: one byte offset per lane and half,
// the chunk term in the scalar offset.
template <int D, int NT, typename RS>
__device__ __forceinline__ void issue_half8(RS rs, uint32_t tile_byte, uint32_t off, uint8_t* l, int wv) {
    constexpr int NCH = TileGeom8<D>::K_CHUNKS / NT;
#pragma unroll
    for (int i = 0; i < NCH; ++i)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_ptr8)(l + (size_t)(i * NT + wv * 64) * 16), 16, off,
                                                 tile_byte + (uint32_t)(i * NT * 16), 0, 0);
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t byte_rsrc8(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

// 32 bytes of an LDS row at two 16-byte chunks as one MFMA operand.
__device__ __forceinline__ i32x8 lds32(const char* p0, const char* p1) {
    const u32x4 a = *reinterpret_cast<const u32x4*>(p0);
    const u32x4 b = *reinterpret_cast<const u32x4*>(p1);
    return i32x8{(int)a[0], (int)a[1], (int)a[2], (int)a[3], (int)b[0], (int)b[1], (int)b[2], (int)b[3]};
}

__device__ __forceinline__ f32x16 mfma8(i32x8 a, i32x8 b, f32x16 c) {
    // formats 0, 0: E4M3 x E4M3; unit scales
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

// S^T = K_tile Q^T for two chunks of 32 keys x this wave's 32 queries.  kboff[ds][u]: byte offset of
// lane (i32, h)'s chunk u (of 2) of k step ds in row i32 (row 32 + i32 is 32*D bytes further).
template <int D>
__device__ __forceinline__ void scores8(const uint8_t* Kl, const uint32_t (&kboff)[D / 64][2],
                                        const i32x8 (&qreg)[D / 64], f32x16 (&st)[2]) {
    const char* Kb = reinterpret_cast<const char*>(Kl);
#pragma unroll
    for (int c = 0; c < 2; ++c) {
        f32x16 a16;
#pragma unroll
        for (int r = 0; r < 16; ++r) a16[r] = 0.f;
#pragma unroll
        for (int ds = 0; ds < D / 64; ++ds) {
            const i32x8 a = lds32(Kb + c * 32 * D + kboff[ds][0], Kb + c * 32 * D + kboff[ds][1]);
            a16 = mfma8(a, qreg[ds], a16);
        }
        st[c] = a16;
    }
}

template <int V> using IC8 = std::integral_constant<int, V>;

template <typename T, int D, int BLK>
__global__ __launch_bounds__(BLK * 2, 2) void attn_fwd_fp8_kernel(
    const T* __restrict__ Q, const uint8_t* __restrict__ packed, const float* __restrict__ bias2,
    const int32_t* __restrict__ idx, const int32_t* __restrict__ perm, const uint32_t* __restrict__ amax,
    int32_t* __restrict__ queue,
    T* __restrict__ O, float* __restrict__ lse, int N, int Nv, int M, int Mk, int nsh, int Ksel, int SQ, int BH, int C,
    int Tv,
    int Ts, int Tc, float c_log2) {
#if defined(__HIP_DEVICE_COMPILE__)
    using G = TileGeom8<D>;
    constexpr int NT = BLK * 2;
    __shared__ __attribute__((aligned(16))) uint8_t kbuf0[kTK8 * D];
    __shared__ __attribute__((aligned(16))) uint8_t kbuf1[kTK8 * D];
    __shared__ __attribute__((aligned(16))) uint8_t vbuf0[kTK8 * D];
    __shared__ __attribute__((aligned(16))) uint8_t vbuf1[kTK8 * D];
    __shared__ __attribute__((aligned(16))) float lbias0[kTK8];
    __shared__ __attribute__((aligned(16))) float lbias1[kTK8];
    __shared__ uint32_t sel_bits[kMaxBlocks / 32 + 2];
    auto kbuf = [&](auto s) __attribute__((always_inline)) -> uint8_t* { if constexpr (decltype(s)::value == 0) return kbuf0; else return kbuf1; };
    auto vbuf = [&](auto s) __attribute__((always_inline)) -> uint8_t* { if constexpr (decltype(s)::value == 0) return vbuf0; else return vbuf1; };
    auto lbias = [&](auto s) __attribute__((always_inline)) -> float* { if constexpr (decltype(s)::value == 0) return lbias0; else return lbias1; };

    // which query tile: sink-query tiles first; video query blocks laid out per XCD as in the bf16
    // kernel (each XCD walks a contiguous run of one head's query blocks), claimed from the XCD's
    // counter and, once its run is spent, from another XCD's (the grid holds one workgroup per
    // item, so each claims exactly one)
    int bh, qrow0, nq, ntiles;
    bool dense;
    {
        const int wg = blockIdx.x;
        if (wg < BH * SQ) {
            dense = true;
            bh = wg / SQ;
            qrow0 = Nv + (wg % SQ) * BLK;
            nq = min(BLK, N - qrow0);
            ntiles = Tv + Ts;
        } else {
            dense = false;
            const int v = wg - BH * SQ;
            int xcd = wg & 7, slot = v >> 3;
            __shared__ int s_claim;
            if (threadIdx.x == 0) {
                int c = -1;
                for (int k = 0; k < 8 && c < 0; ++k) {
                    const int x2 = (xcd + k) & 7;
                    const int j = atomicAdd(&queue[x2], 1);
                    if (j < BH * C) c = x2 * BH * C + j;
                }
                s_claim = c;
            }
            __syncthreads();
            const int c = s_claim;
            if (c < 0) return;  // none left (not reached: items = workgroups); uniform
            xcd = c / (BH * C);
            slot = c % (BH * C);
            bh = slot / C;
            const int I = xcd * C + slot % C;
            if (I >= M) return;
            qrow0 = I * BLK;
            nq = min(BLK, Nv - qrow0);
            ntiles = (Ksel << nsh) + Ts + Tc;
        }
    }
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int i32 = lane & 31, h = lane >> 5;
    const int Tall = Tv + Ts + Tc;
    const uint8_t* ptile = packed + (size_t)bh * Tall * G::BYTES;
    const float* pbias = bias2 + (size_t)bh * Tall * kTK8;
    const int32_t* sel = dense ? nullptr : idx + ((size_t)bh * M + qrow0 / BLK) * Ksel;
    // a selected key block is 1 << nsh tiles (key blocks of 64 or 128 keys)
    const int n_exact = dense ? 0 : Ksel << nsh;
    const int first_cmp = dense ? ntiles : n_exact + Ts;

    // selected block ids, 64 per register window (lane l holds entry base + l), the next window
    // loaded one ahead so that moving to it never waits for memory
    int win_base = 0, selw = 0, selw_next = 0;
    if (!dense) {
        selw = lane < Ksel ? clamp_block(sel[lane], Mk) : 0;
        selw_next = 64 + lane < Ksel ? clamp_block(sel[64 + lane], Mk) : 0;
    }
    auto tile_of = [&](int t) __attribute__((always_inline)) -> int {
        if (dense) return t;
        if (t >= n_exact) return Tv + (t - n_exact);
        const int k = t >> nsh;
        if (k >= win_base + 64) {  // k grows by at most one per call: this is the next window
            win_base += 64;
            selw = selw_next;
            selw_next = win_base + 64 + lane < Ksel ? clamp_block(sel[win_base + 64 + lane], Mk) : 0;
        }
        return (__builtin_amdgcn_readlane(selw, k - win_base) << nsh) + (t & ((1 << nsh) - 1));
    };

    if (!dense) {
        for (int j = threadIdx.x; j < (Mk + 63) / 32 + 1; j += NT) sel_bits[j] = 0u;
        __syncthreads();
        for (int k = threadIdx.x; k < Ksel; k += NT) {
            const int J = clamp_block(sel[k], Mk);
            atomicOr(&sel_bits[J >> 5], 1u << (J & 31));
        }
    }
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    uint32_t off_k, off_v;  // byte offsets of this lane's first chunk inside a packed tile
    {
        const int q = threadIdx.x;
        const int m = q / G::CK, pc = q % G::CK;
        off_k = (uint32_t)(m * G::CK + (pc ^ swz8<G::CK>(m))) * 16u;
        const int dr = q / G::V_CPR, pv = q % G::V_CPR;
        off_v = (uint32_t)(G::K_CHUNKS + dr * G::V_CPR + (pv ^ swz8<G::V_CPR>(dr))) * 16u;
    }
    const __amdgpu_buffer_rsrc_t rs_tiles = byte_rsrc8(ptile, (uint32_t)Tall * G::BYTES);
    const __amdgpu_buffer_rsrc_t rs_bias = byte_rsrc8(pbias, (uint32_t)Tall * (kTK8 * 4));
    auto load_k = [&](int tl, auto s) __attribute__((always_inline)) {
        issue_half8<D, NT>(rs_tiles, (uint32_t)tl * G::BYTES, off_k, kbuf(s), wv);
    };
    auto load_v = [&](int tl, auto s) __attribute__((always_inline)) {
        issue_half8<D, NT>(rs_tiles, (uint32_t)tl * G::BYTES, off_v, vbuf(s), wv);
        if (wv == 0)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rs_bias, (lds_ptr8)lbias(s), 4, (uint32_t)lane * 4u,
                                                     (uint32_t)tl * (kTK8 * 4), 0, 0);
    };
    int tl_v;
    {
        const int tl0 = tile_of(0);
        load_k(tl0, IC8<0>{});
        tl_v = ntiles > 1 ? tile_of(1) : 0;
        if (ntiles > 1) load_k(tl_v, IC8<1>{});
        load_v(tl0, IC8<0>{});
    }

    // Q rows of this wave on their E4M3 carrier, as the B operand of S^T = K Q^T: lane (i32, h)
    // holds row w*32 + i32, dims 64 ds + 32h .. +32.
    const float rq = fp8_r(amax[bh * 3 + 0]);
    const float sq = fp8_s(amax[bh * 3 + 0]), sk = fp8_s(amax[bh * 3 + 1]), sv = fp8_s(amax[bh * 3 + 2]);
    i32x8 qreg[D / 64];
    {
        const int qr = w * 32 + i32;
        const T* src = Q + ((size_t)bh * N + qrow0 + min(qr, nq - 1)) * D;
#pragma unroll
        for (int ds = 0; ds < D / 64; ++ds) {
            Raw8<T> raw[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) raw[u].load(src + 64 * ds + 32 * h + 8 * u);
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                float v[8];
                raw[u].widen(v);
                if (qr >= nq)
#pragma unroll
                    for (int j = 0; j < 8; ++j) v[j] = 0.f;
                qreg[ds][2 * u] = (int)fp8x4(v[0] * rq, v[1] * rq, v[2] * rq, v[3] * rq);
                qreg[ds][2 * u + 1] = (int)fp8x4(v[4] * rq, v[5] * rq, v[6] * rq, v[7] * rq);
            }
        }
    }
    // logits in log2 units: raw * (scale * log2 e) * s_Q * s_K
    const float cl = c_log2 * sq * sk;

    uint32_t kboff[D / 64][2], vboff[2];
#pragma unroll
    for (int ds = 0; ds < D / 64; ++ds)
#pragma unroll
        for (int u = 0; u < 2; ++u)
            kboff[ds][u] = (i32 * G::CK + ((4 * ds + 2 * h + u) ^ swz8<G::CK>(i32))) * 16;
#pragma unroll
    for (int u = 0; u < 2; ++u) vboff[u] = (i32 * G::V_CPR + ((2 * h + u) ^ swz8<G::V_CPR>(i32))) * 16;
    const int Ns = N - Nv;
    auto clean_of = [&](int tl) __attribute__((always_inline)) -> bool {
        return tl < Tv ? (tl + 1) * kTK8 <= Nv : (tl - Tv + 1) * kTK8 <= Ns;
    };

    f32x16 acc[D / 32];
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[dt][r] = 0.f;
    float m_run = -INFINITY, l_run = 0.f;

    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    f32x16 sc[2][2];
    scores8<D>(kbuf(IC8<0>{}), kboff, qreg, sc[0]);
    bool clean_t = clean_of(tile_of(0)), clean_v = ntiles > 1 && clean_of(tl_v);

    auto step = [&](int t, auto masked, auto par, auto known_clean) __attribute__((always_inline)) {
        constexpr bool MASKED = decltype(masked)::value;
        constexpr int P = decltype(par)::value;
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        const int tl_k = t + 2 < ntiles ? tile_of(t + 2) : 0;
        if (t + 2 < ntiles) load_k(tl_k, IC8<P>{});
        if (t + 1 < ntiles) load_v(tl_v, IC8<P ^ 1>{});
        const bool clean = decltype(known_clean)::value || (!MASKED && clean_t);
        clean_t = clean_v;
        clean_v = t + 2 < ntiles && clean_of(tl_k);
        tl_v = tl_k;
        scores8<D>(kbuf(IC8<P ^ 1>{}), kboff, qreg, sc[P ^ 1]);

        // probabilities of tile t; register 4g+j of chunk c holds key 32c + 8g + 4h + j
        f32x16 (&st)[2] = sc[P];
        float mx = -INFINITY, cc;
        if (clean) {
#pragma unroll
            for (int c = 0; c < 2; ++c)
#pragma unroll
                for (int r = 0; r < 16; ++r) mx = fmaxf(mx, st[c][r]);
            mx = half_max(mx) * cl;  // cl > 0: the max commutes with it
            cc = cl;
        } else {
            const int cbase = (t - first_cmp) * kTK8;
            const float* lb = lbias(IC8<P>{});
#pragma unroll
            for (int c = 0; c < 2; ++c)
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const int key = 32 * c + 8 * g + 4 * h;
                    f32x4 bb = *reinterpret_cast<const f32x4*>(lb + key);
                    if constexpr (MASKED) {
                        const uint32_t selw_ = sel_bits[(cbase + key) >> 5] >> ((cbase + key) & 31);
#pragma unroll
                        for (int j = 0; j < 4; ++j) bb[j] = ((selw_ >> j) & 1u) ? -INFINITY : bb[j];
                    }
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        st[c][4 * g + j] = fmaf(st[c][4 * g + j], cl, bb[j]);
                        mx = fmaxf(mx, st[c][4 * g + j]);
                    }
                }
            mx = half_max(mx);
            cc = 1.f;
        }
        const bool raise = mx > m_run + kRescaleSlack8;
        if (__ballot(raise)) {
            const float m_new = raise ? mx : m_run;
            const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
            l_run *= alpha;
#pragma unroll
            for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
                for (int r = 0; r < 16; ++r) acc[dt][r] *= alpha;
            m_run = m_new;
        }
        const float neg_m = m_run == -INFINITY ? 0.f : -m_run;
        // P^T operand: byte 16c + r of lane (i32, h) is the probability of S^T register r of chunk c
        i32x8 pf;
#pragma unroll
        for (int c = 0; c < 2; ++c)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                float p4[4];
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    p4[j] = __builtin_amdgcn_exp2f(fmaf(st[c][4 * q + j], cc, neg_m));
                    l_run += p4[j];
                }
                pf[4 * c + q] = (int)fp8x4(p4[0], p4[1], p4[2], p4[3]);
            }
        const char* Vb = reinterpret_cast<const char*>(vbuf(IC8<P>{}));
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt) {  // V^T row dt*32 + i32 is 32*64 bytes past row i32
            const i32x8 a = lds32(Vb + dt * 32 * kTK8 + vboff[0], Vb + dt * 32 * kTK8 + vboff[1]);
            acc[dt] = mfma8(a, pf, acc[dt]);
        }
    };
    auto run = [&](int t, int end, auto masked) __attribute__((always_inline)) {
        constexpr std::false_type any{};
        if (t < end && (t & 1)) step(t++, masked, IC8<1>{}, any);
        if constexpr (!decltype(masked)::value) {
            // leading pairs of tiles known to need no additive term (all but ragged edge tiles)
            for (; t + 1 < end && clean_t && clean_v; t += 2) {
                step(t, masked, IC8<0>{}, std::true_type{});
                step(t + 1, masked, IC8<1>{}, std::true_type{});
            }
        }
        for (; t + 1 < end; t += 2) {
            step(t, masked, IC8<0>{}, any);
            step(t + 1, masked, IC8<1>{}, any);
        }
        if (t < end) step(t++, masked, IC8<0>{}, any);
        return t;
    };
    run(run(0, first_cmp, std::false_type{}), ntiles, std::true_type{});

    // epilogue: lane (i32, h) holds query row w*32 + i32, dims dt*32 + 8g + 4h + (0..3); values
    // restored by s_V
    const float l_tot = l_run + __shfl_xor(l_run, 32);
    const float inv = sv / l_tot;
    const int qr = w * 32 + i32;
    if (qr < nq) {
        const int row = qrow0 + qr;
        const int orow = (!dense && perm) ? perm[(size_t)bh * Nv + row] : row;
        if (!dense && perm && (unsigned)orow >= (unsigned)Nv) return;  // a permutation entry out of range: row not written
        T* dst = O + ((size_t)bh * N + orow) * D;
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
#endif
}

// ---------------------------------------------------------------------------------------------
// Launchers.

// zero amax, then raise it over rows row0 .. N-1 (all rows: row0 = 0)
void launch_fp8_amax_rows(const LaunchCtx& L, const void* Q, const void* K, const void* V, uint32_t* amax,
                          int row0) {
    hipLaunchKernelGGL(fp8_zero_kernel, dim3((L.BH * 3 + 255) / 256), dim3(256), 0, L.stream, amax, L.BH * 3);
    if (row0 >= L.N) return;
    // workgroups per (batch, head, tensor): enough for the full tensor, fewer for a few sink rows
    const int wg = (int)std::min<long long>(64, ((long long)(L.N - row0) * L.d / 8 + 255) / 256);
    if (L.dtype == SPARK_ATTN_BF16)
        hipLaunchKernelGGL((fp8_amax_kernel<__bf16>), dim3(wg, L.BH, 3), dim3(256), 0, L.stream, (const __bf16*)Q,
                           (const __bf16*)K, (const __bf16*)V, L.N, row0, L.d, amax);
    else
        hipLaunchKernelGGL((fp8_amax_kernel<float>), dim3(wg, L.BH, 3), dim3(256), 0, L.stream, (const float*)Q,
                           (const float*)K, (const float*)V, L.N, row0, L.d, amax);
}

void launch_fp8_scales(const LaunchCtx& L, const void* Q, const void* K, const void* V, uint32_t* amax) {
    launch_fp8_amax_rows(L, Q, K, V, amax, 0);
}

template <typename T, int D>
static void launch_pack_fp8_t(const LaunchCtx& L, const void* K, const void* V, const float* k_sum,
                              const float* v_sum, const float* bias, const uint32_t* amax, void* packed) {
    const PackGeom g = pack_geom_fp8(L);
    uint8_t* kv = (uint8_t*)packed;
    float* b2 = (float*)((char*)packed + g.bias_off);
    hipLaunchKernelGGL((pack_keys_fp8_kernel<T, D>), dim3(L.BH * (g.Tv + g.Ts)), dim3(256), 0, L.stream, (const T*)K,
                       (const T*)V, L.N, L.Nv, g.Tv, g.Ts, g.Tall, amax, kv, b2);
    hipLaunchKernelGGL((pack_compressed_fp8_kernel<D>), dim3(L.BH * g.Tc), dim3(256), 0, L.stream, k_sum, v_sum, bias,
                       L.Mk, g.Tv, g.Ts, g.Tc, g.Tall, amax, kv, b2);
}

void launch_pack_fp8(const LaunchCtx& L, const void* K, const void* V, const float* k_sum, const float* v_sum,
                     const float* bias, const uint32_t* amax, void* packed) {
    if (L.dtype == SPARK_ATTN_BF16) {
        if (L.d == 64) launch_pack_fp8_t<__bf16, 64>(L, K, V, k_sum, v_sum, bias, amax, packed);
        else launch_pack_fp8_t<__bf16, 128>(L, K, V, k_sum, v_sum, bias, amax, packed);
    } else {
        if (L.d == 64) launch_pack_fp8_t<float, 64>(L, K, V, k_sum, v_sum, bias, amax, packed);
        else launch_pack_fp8_t<float, 128>(L, K, V, k_sum, v_sum, bias, amax, packed);
    }
}

template <typename T, int D, int BLK>
static void launch_attend_fp8_t(const LaunchCtx& L, const void* Q, const void* packed, const int32_t* idx,
                                const int32_t* perm, const uint32_t* amax, void* O, float* lse) {
    const PackGeom g = pack_geom_fp8(L);
    const int SQ = (L.n_sink + BLK - 1) / BLK;
    const int C = (L.M + 7) / 8;
    const dim3 grid(L.BH * SQ + L.BH * 8 * C);
    const float c_log2 = L.scale * 1.4426950408889634f;
    // the tile counters start at zero on every call (a kernel, so that a captured graph replays it)
    int32_t* queue = (int32_t*)((char*)packed + g.queue_off);  // workspace the library owns inside the packed buffer
    hipLaunchKernelGGL(fp8_zero_kernel, dim3(1), dim3(256), 0, L.stream, (uint32_t*)queue, 8);
    hipLaunchKernelGGL((attn_fwd_fp8_kernel<T, D, BLK>), grid, dim3(BLK * 2), 0, L.stream, (const T*)Q,
                       (const uint8_t*)packed, (const float*)((const char*)packed + g.bias_off), idx, perm, amax,
                       queue, (T*)O, lse, L.N, L.Nv, L.M, L.Mk, L.block_k == 128 ? 1 : 0, L.K, SQ, L.BH, C, g.Tv, g.Ts,
                       g.Tc, c_log2);
}

void launch_attend_fp8(const LaunchCtx& L, const void* Q, const void* packed, const int32_t* idx,
                       const int32_t* perm, const uint32_t* amax, void* O, float* lse) {
#define SPARK_ATTN_CASE8(T, D, B)                                                \
    if (L.d == D && L.block == B) {                                              \
        launch_attend_fp8_t<T, D, B>(L, Q, packed, idx, perm, amax, O, lse);     \
        return;                                                                  \
    }
    if (L.dtype == SPARK_ATTN_BF16) {
        SPARK_ATTN_CASE8(__bf16, 64, 64) SPARK_ATTN_CASE8(__bf16, 64, 128)
        SPARK_ATTN_CASE8(__bf16, 128, 64) SPARK_ATTN_CASE8(__bf16, 128, 128)
    } else {
        SPARK_ATTN_CASE8(float, 64, 64) SPARK_ATTN_CASE8(float, 64, 128)
        SPARK_ATTN_CASE8(float, 128, 64) SPARK_ATTN_CASE8(float, 128, 128)
    }
#undef SPARK_ATTN_CASE8
}

}  // namespace spark
