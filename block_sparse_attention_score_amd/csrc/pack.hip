// Packing of the keys and values the attention stage reads, once per call, into 64-key tiles:
//
//   tile t of (batch, head) = [ K rows: 64 x d bf16, row-major | V^T: d x 64 bf16 ]  (contiguous)
//   bias2[t][64] fp32: additive logit term in log2 units (0 or -inf for real keys, log2(e) * bias
//                      for compressed pseudo-keys, -inf for padding)
//
// Tiles 0 .. Tv-1 hold the video keys (row r of the video part is tile r/64, slot r%64; Tv covers
// M whole blocks, so a short last block ends in padding), tiles
// Tv .. Tv+Ts-1 the sink keys, tiles Tv+Ts .. Tall-1 the compressed pseudo-keys (the per-block
// summaries, Spark-H3 page, "Spark-Attnが変えるもの", Spark-Reweight bullet).  A selected block J
// is the tiles J*block_k/64 .. (J+1)*block_k/64 - 1 (block_k: the key block size).  Padding rows
// are zero with bias -inf, so the attention kernel reads whole tiles with no bounds logic.
//
// Every value tile is stored transposed: each selected block is used by ~K of the M query blocks,
// so transposing once here replaces a transposition at every use inside the attention loop.
//
// Each tile writer also records, for its tile, the largest squared norm of its keys as stored
// (bf16) and the largest additive term of its valid keys.  Per (batch, head) these give the
// constants of a Cauchy-Schwarz bound on every logit a query can meet, which the attention stage
// uses as its softmax offset (launch_bounds).
#include "kernels.hpp"

namespace spark {

PackGeom pack_geom(const LaunchCtx& L) {
    PackGeom g;
    g.Tv = L.Mk * (L.block_k / 64);  // every key block owns whole tiles (a short last block is padded)
    g.Ts = (L.n_sink + 63) / 64;
    g.Tc = (L.Mk + 63) / 64;
    g.Tall = g.Tv + g.Ts + g.Tc;
    g.SQ = (L.n_sink + L.block - 1) / L.block;
    g.NQT = g.SQ + L.M;
    g.tile_elems = (size_t)2 * 64 * L.d;
    g.kv_bytes = (size_t)L.BH * g.Tall * g.tile_elems * 2;
    auto a256 = [](size_t x) { return (x + 255) & ~(size_t)255; };
    g.bias_off = a256(g.kv_bytes);
    g.tmax_off = a256(g.bias_off + (size_t)L.BH * g.Tall * 64 * 4);
    g.bnd_off = a256(g.tmax_off + (size_t)L.BH * g.Tall * 8);
    g.flag_off = a256(g.bnd_off + (size_t)L.BH * 16);
    g.queue_off = a256(g.flag_off + (size_t)L.BH * g.NQT * 4);
    g.bytes = a256(g.queue_off + 8 * 4);
    return g;
}

// Sum of squares of eight packed bf16 values (the key as the matrix cores see it).
__device__ __forceinline__ float sumsq8_bf16(const u32x4 u) {
    float s = 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const float lo = bf16_bits_to_f32(u[j] & 0xffffu), hi = bf16_bits_to_f32(u[j] >> 16);
        s = fmaf(lo, lo, s);
        s = fmaf(hi, hi, s);
    }
    return s;
}

// One workgroup per tile of 64 source rows: rows of X (real keys, type T) or of the fp32
// summaries (compressed).  K rows are re-packed as bf16 rows; V rows go through LDS to be
// written transposed with 16-byte stores.
template <typename T, typename S, int D>
__device__ __forceinline__ void pack_tile(const T* __restrict__ Ksrc, const T* __restrict__ Vsrc, int nvalid,
                                          __bf16* __restrict__ tile, float* __restrict__ bias2,
                                          const float* __restrict__ bias_src, float bias_scale,
                                          float2* __restrict__ tmax) {
    constexpr int CPR = D / 8;                 // 16-byte bf16 chunks per row
    constexpr int ROWS_PER_PASS = 256 / CPR;   // rows covered by the 256 threads in one pass
    __shared__ __attribute__((aligned(16))) __bf16 vs[64][D + 8];
    __shared__ float wmax[4];
    const int t = threadIdx.x, c = t % CPR;
    __bf16* kdst = tile;
    __bf16* vdst = tile + 64 * D;
    const u32x4 zero = {0u, 0u, 0u, 0u};
    float n2 = 0.f;  // largest squared key norm among this thread's rows (padding rows are zero)
#pragma unroll
    for (int r0 = 0; r0 < 64; r0 += ROWS_PER_PASS) {
        const int r = r0 + t / CPR;
        u32x4 kv = zero, vv = zero;
        if (r < nvalid) {
            kv = load8_as_bf16<S>(reinterpret_cast<const S*>(Ksrc) + (size_t)r * D + c * 8);
            vv = load8_as_bf16<S>(reinterpret_cast<const S*>(Vsrc) + (size_t)r * D + c * 8);
        }
        *reinterpret_cast<u32x4*>(kdst + r * D + c * 8) = kv;
        *reinterpret_cast<u32x4*>(&vs[r][c * 8]) = vv;
        float s2 = sumsq8_bf16(kv);
        // the CPR threads of a row are consecutive lanes of one wave
#pragma unroll
        for (int o = 1; o < CPR; o <<= 1) s2 += __shfl_xor(s2, o);
        n2 = fmaxf(n2, s2);
    }
    n2 = wave_max(n2);
    if ((t & 63) == 0) wmax[t >> 6] = n2;
    __syncthreads();
    // V^T row dr = keys 0..63 of dimension dr: 8 chunks of 8 keys
    for (int e = t; e < D * 8; e += 256) {
        const int dr = e / 8, kc = e % 8;
        u32x4 o;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const uint32_t lo = __builtin_bit_cast(uint16_t, vs[kc * 8 + 2 * j][dr]);
            const uint32_t hi = __builtin_bit_cast(uint16_t, vs[kc * 8 + 2 * j + 1][dr]);
            o[j] = lo | (hi << 16);
        }
        *reinterpret_cast<u32x4*>(vdst + dr * 64 + kc * 8) = o;
    }
    if (t < 64) {
        float b = -INFINITY;
        if (t < nvalid) b = bias_src ? bias_src[t] * bias_scale : 0.f;
        bias2[t] = b;
        b = wave_max(b);
        if (t == 0) *tmax = make_float2(fmaxf(fmaxf(wmax[0], wmax[1]), fmaxf(wmax[2], wmax[3])), b);
    }
}

// grid: BH * cnt tiles of real keys, tiles t0 .. t0+cnt-1 of each (batch, head)
template <typename T, int D>
__global__ __launch_bounds__(256) void pack_keys_kernel(const T* __restrict__ K, const T* __restrict__ V, int N,
                                                        int Nv, int Tv, int Tall, int t0, int cnt,
                                                        __bf16* __restrict__ packed, float* __restrict__ bias2,
                                                        float2* __restrict__ tmax) {
    const int bh = blockIdx.x / cnt, t = t0 + blockIdx.x % cnt;
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
    pack_tile<T, T, D>(K + src, V + src, nvalid, packed + tile * (2 * 64 * D), bias2 + tile * 64, nullptr, 0.f,
                       tmax + tile);
}

// grid: BH * Tc tiles of compressed pseudo-keys (fp32 summaries)
template <int D>
__global__ __launch_bounds__(256) void pack_compressed_kernel(const float* __restrict__ k_sum,
                                                              const float* __restrict__ v_sum,
                                                              const float* __restrict__ bias, int M, int Tv,
                                                              int Ts, int Tc, int Tall,
                                                              __bf16* __restrict__ packed, float* __restrict__ bias2,
                                                              float2* __restrict__ tmax) {
    const int bh = blockIdx.x / Tc, c = blockIdx.x % Tc;
    const int J0 = c * 64, nvalid = min(64, M - J0);
    const size_t src = ((size_t)bh * M + J0) * D;
    const size_t tile = (size_t)bh * Tall + Tv + Ts + c;
    pack_tile<float, float, D>(k_sum + src, v_sum + src, nvalid, packed + tile * (2 * 64 * D), bias2 + tile * 64,
                               bias + (size_t)bh * M + J0, 1.4426950408889634f, tmax + tile);
}

// Per (batch, head): the largest key norm over the video and sink tiles, and over the compressed
// tiles the largest pseudo-key norm and additive term.  A query q' (already scaled into log2
// units) then meets no logit above max(|q'| * kx, |q'| * kc + bc) (Cauchy-Schwarz).
__global__ __launch_bounds__(256) void bounds_kernel(const float2* __restrict__ tmax, int Tv, int Ts, int Tc,
                                                     int Tall, float4* __restrict__ bnd) {
    const int bh = blockIdx.x;
    const float2* tm = tmax + (size_t)bh * Tall;
    float kx = 0.f, kc = 0.f, bc = -INFINITY;
    for (int t = threadIdx.x; t < Tv + Ts; t += 256) kx = fmaxf(kx, tm[t].x);
    for (int t = threadIdx.x; t < Tc; t += 256) {
        const float2 v = tm[Tv + Ts + t];
        kc = fmaxf(kc, v.x);
        bc = fmaxf(bc, v.y);
    }
    __shared__ float red[3][4];
    kx = wave_max(kx);
    kc = wave_max(kc);
    bc = wave_max(bc);
    if ((threadIdx.x & 63) == 0) {
        red[0][threadIdx.x >> 6] = kx;
        red[1][threadIdx.x >> 6] = kc;
        red[2][threadIdx.x >> 6] = bc;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        float r[3];
#pragma unroll
        for (int i = 0; i < 3; ++i) r[i] = fmaxf(fmaxf(red[i][0], red[i][1]), fmaxf(red[i][2], red[i][3]));
        bnd[bh] = make_float4(sqrtf(r[0]), sqrtf(r[1]), r[2], 0.f);
    }
}

void launch_bounds(const LaunchCtx& L, void* packed) {
    const PackGeom g = pack_geom(L);
    hipLaunchKernelGGL(bounds_kernel, dim3(L.BH), dim3(256), 0, L.stream,
                       (const float2*)((const char*)packed + g.tmax_off), g.Tv, g.Ts, g.Tc, g.Tall,
                       (float4*)((char*)packed + g.bnd_off));
}

template <typename T, int D>
static void launch_pack_t(const LaunchCtx& L, const void* K, const void* V, const float* k_sum, const float* v_sum,
                          const float* bias, void* packed, bool sinks_only) {
    const PackGeom g = pack_geom(L);
    __bf16* kv = (__bf16*)packed;
    float* b2 = (float*)((char*)packed + g.bias_off);
    float2* tm = (float2*)((char*)packed + g.tmax_off);
    const int t0 = sinks_only ? g.Tv : 0, cnt = g.Tv + g.Ts - t0;
    if (cnt > 0)
        hipLaunchKernelGGL((pack_keys_kernel<T, D>), dim3(L.BH * cnt), dim3(256), 0, L.stream, (const T*)K,
                           (const T*)V, L.N, L.Nv, g.Tv, g.Tall, t0, cnt, kv, b2, tm);
    hipLaunchKernelGGL((pack_compressed_kernel<D>), dim3(L.BH * g.Tc), dim3(256), 0, L.stream, k_sum, v_sum,
                       bias, L.Mk, g.Tv, g.Ts, g.Tc, g.Tall, kv, b2, tm);
    launch_bounds(L, packed);
}

static void launch_pack_any(const LaunchCtx& L, const void* K, const void* V, const float* k_sum,
                            const float* v_sum, const float* bias, void* packed, bool sinks_only) {
    if (L.dtype == SPARK_ATTN_BF16) {
        if (L.d == 64) launch_pack_t<__bf16, 64>(L, K, V, k_sum, v_sum, bias, packed, sinks_only);
        else launch_pack_t<__bf16, 128>(L, K, V, k_sum, v_sum, bias, packed, sinks_only);
    } else {
        if (L.d == 64) launch_pack_t<float, 64>(L, K, V, k_sum, v_sum, bias, packed, sinks_only);
        else launch_pack_t<float, 128>(L, K, V, k_sum, v_sum, bias, packed, sinks_only);
    }
}

void launch_pack(const LaunchCtx& L, const void* K, const void* V, const float* k_sum, const float* v_sum,
                 const float* bias, void* packed) {
    launch_pack_any(L, K, V, k_sum, v_sum, bias, packed, false);
}

// the sink tiles and the compressed tiles (the video tiles come from the pooling kernel)
void launch_pack_rest(const LaunchCtx& L, const void* K, const void* V, const float* k_sum, const float* v_sum,
                      const float* bias, void* packed) {
    launch_pack_any(L, K, V, k_sum, v_sum, bias, packed, true);
}

}  // namespace spark
