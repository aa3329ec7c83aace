// Spark-Reblock partition (Spark-H3 page, section "Spark-Attnが変えるもの", Spark-Reblock bullet):
// queries are alike when their score patterns against the keys are alike, measured by the cosine
// in the metric of the keys' second moment; a hierarchical partitioner keeps splitting groups
// until every leaf holds the block size, in O(N log N); keys reuse the query partition
// (section "ワークフロー": reblock_layout=q_reuse_k).
//
// Every decision is taken in binary64 with one fixed operation order, so the permutation is
// exact and reproducible (this file is compiled with -ffp-contract=off and every multiply-add
// below is an explicit fma):
//   Sigma  = K^T K / N_v in fixed point: k^ = rint(k 2^s) (s = 21 - E, max|k| < 2^E), exact int64
//            sums of k^_a k^_b (exact integer products of base-256 digits on int8 MFMA), scaled back;
//   n_i    = sqrt(q_i^T Sigma q_i): t_a = fma(Sigma_ab, q_b, t_a) over b, r = fma(q_a, t_a, r) over a;
//   g(P)   = t(P) / n_P;  cos(i, P) = (fma chain over a of q_ia g_a(P)) / n_i  (0 when a norm is 0);
//   split  : P0 = lowest index, A = argmin cos(., P0), B = argmin cos(., A) (ties: lower index),
//            key = cos(., A) - cos(., B); the ceil(c/2)*block tokens first in (key desc, index asc)
//            form the left child;
//   perm   : leaves left to right, ascending token index inside each leaf.
// Argmins are lexicographic (order-preserving key, index) reductions and the balanced split is a
// radix select on (key, index), so nothing depends on thread timing.
//
// Kernels: max|k|, the fixed-point Sigma and the norms are wide (all CUs).  The partition keeps
// an order array in which every group's tokens are contiguous, at the positions its leaves will
// occupy in the permutation (leaves L0 .. L0+c-1 of a group own positions L0*block ..).  Levels
// whose groups are large run the three cos passes over (group, chunk) workgroups, with a small
// pivot launch between passes, then one workgroup per group selects and partitions; levels of
// mid-sized groups run one fused workgroup per group; the last levels, once a group fits one
// workgroup with a token per thread, run in one launch that keeps every token on chip.  A stable
// partition writes each next order, so inside every leaf the tokens stay in ascending index.
#include <limits.h>

#include <algorithm>
#include <type_traits>

#include "kernels.hpp"

#pragma clang fp contract(off)

namespace spark {

typedef double f64x2 __attribute__((ext_vector_type(2)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x16 __attribute__((ext_vector_type(16)));

constexpr int kRbMaxRows = 1 << 20; // int64 sums of <= 2^20 products of magnitude <= 2^42
constexpr int kRbChunk = 2048;      // most order positions per workgroup of a chunked cos pass
constexpr int kRbChunkThreads = 256;

static int rb_levels(int M) {
    int l = 0;
    while ((1 << l) < M) ++l;
    return l;
}

// Chunks per group at level lev (groups hold at most ceil(M / 2^lev) leaves); the level runs
// chunked when this is 2 or more.
static int rb_chunks(const LaunchCtx& L, int lev) {
    const long long cmax = ((long long)L.M + (1ll << lev) - 1) >> lev;
    const long long nmax = std::min(cmax * L.block, (long long)L.Nv);
    return (int)((nmax + kRbChunk - 1) / kRbChunk);
}

struct RbLayout {
    size_t kmax, sint, subq, sigma, nrm, ord0, ord1, cbuf, dk, c0, gbuf, pkey, pidx, total;
};

static RbLayout rb_layout(const LaunchCtx& L) {
    RbLayout r;
    const size_t BH = L.BH, Nv = L.Nv, d = L.d;
    size_t gmax = 1, pmax = 1;
    for (int lev = 0, levels = rb_levels(L.M); lev < levels; ++lev) {
        const int nch = rb_chunks(L, lev);
        if (nch < 2) continue;
        gmax = std::max(gmax, (size_t)1 << lev);
        pmax = std::max(pmax, ((size_t)1 << lev) * nch);
    }
    size_t o = 0;
    auto take = [&](size_t bytes) {
        const size_t at = o;
        o = (o + bytes + 255) & ~(size_t)255;
        return at;
    };
    r.kmax = take(BH * 4);
    r.sint = take(BH * d * d * 8);
    r.subq = take(BH * 4);  // the subtree kernel's per-head group counters
    r.sigma = take(BH * d * d * 8);
    r.nrm = take(BH * Nv * 8);
    r.ord0 = take(BH * Nv * 4);
    r.ord1 = take(BH * Nv * 4);
    r.cbuf = take(BH * Nv * 8);
    r.dk = take(BH * Nv * 8);
    r.c0 = take(BH * Nv * 8);  // per token: cos(., P0) of its group at the last chunked level
    r.gbuf = take(BH * gmax * d * 8);
    r.pkey = take(BH * pmax * 8);
    r.pidx = take(BH * pmax * 4);
    r.total = o;
    return r;
}

size_t reblock_workspace_bytes(const LaunchCtx& L) {
    if (L.Nv > kRbMaxRows) return 0;  // outside the exact fixed-point range: unsupported
    return rb_layout(L).total;
}

template <typename T> __device__ __forceinline__ float elem_f(const T* p);
template <> __device__ __forceinline__ float elem_f<__bf16>(const __bf16* p) { return (float)*p; }
template <> __device__ __forceinline__ float elem_f<float>(const float* p) { return *p; }

// Order-preserving map of a binary64 (-0 folded onto +0) to uint64: larger value, larger key.
__device__ __forceinline__ uint64_t asc_key(double x) {
    x = x + 0.0;
    const uint64_t u = (uint64_t)__double_as_longlong(x);
    return (u >> 63) ? ~u : (u | (1ull << 63));
}

__global__ __launch_bounds__(256) void rb_zero_kernel(uint64_t* __restrict__ p, size_t n) {
    for (size_t e = (size_t)blockIdx.x * 256 + threadIdx.x; e < n; e += (size_t)gridDim.x * 256) p[e] = 0;
}

// max |k| over the video keys of each (batch, head), as float bits (non-negative floats order as
// unsigned integers).  The video rows of a head are one contiguous span of Nv*d elements (a
// multiple of 8), read eight at a time.
template <typename T>
__global__ __launch_bounds__(256) void rb_kmax_kernel(const T* __restrict__ K, int N, int Nv, int d,
                                                      uint32_t* __restrict__ kmax) {
    const int bh = blockIdx.y;
    const T* kh = K + (size_t)bh * N * d;
    const size_t n8 = (size_t)Nv * d / 8;
    float m = 0.f;
    const size_t stride = (size_t)gridDim.x * 256;
    size_t e = (size_t)blockIdx.x * 256 + threadIdx.x;
    // four loads in flight per thread, then the remainder one at a time
    for (; e + 3 * stride < n8; e += 4 * stride) {
        Raw8<T> r[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) r[u].load(kh + 8 * (e + u * stride));
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            float v[8];
            r[u].widen(v);
#pragma unroll
            for (int j = 0; j < 8; ++j) m = fmaxf(m, fabsf(v[j]));
        }
    }
    for (; e < n8; e += stride) {
        Raw8<T> r;
        r.load(kh + 8 * e);
        float v[8];
        r.widen(v);
#pragma unroll
        for (int j = 0; j < 8; ++j) m = fmaxf(m, fabsf(v[j]));
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
    if ((threadIdx.x & 63) == 0) atomicMax(&kmax[bh], __float_as_uint(m));
}

__device__ __forceinline__ int fixed_point_shift(uint32_t kmax_bits) {
    int E = 0;
    (void)frexp((double)__uint_as_float(kmax_bits), &E);
    return 21 - E;
}

// Exact fixed-point K^T K on int8 MFMA.  Every key entry k^ = rint(k 2^s) (|k^| <= 2^21) is
// written as three balanced base-256 digits, k^ = d0 + 256 d1 + 65536 d2 with d0, d1 in [-128, 127]
// and d2 in [-32, 32]; then sum_i k^_ia k^_ib = sum_{p,q} 256^(p+q) sum_i d_p(i,a) d_q(i,b), whose
// inner sums are exact integer products (v_mfma_i32_32x32x32_i8).  Digit pairs with the same p + q
// share one int32 accumulator: at most three products of magnitude <= 2^14 per row and entry, so
// the sums stay exact for the kRbSigRows rows of a workgroup; they are combined in int64 at the end
// and added to the int64 sums of the (batch, head).  Workgroup (bh, row chunk): each wave owns one
// 32 x 32 tile of Sigma on or above the diagonal.  Rows are converted 64 at a time into digit
// planes in LDS (plane p: feature rows of 64 bytes, one byte per row of K), which give both MFMA
// operands: lane l reads 16 bytes of feature 32t + l % 32, rows 16 (l / 32) .. of a 32-row step,
// the same rows for the A and the B side, so the products pair the digits of one row.
template <int D> struct RbSig {
    static constexpr int TB = D / 32;               // 32-feature blocks
    static constexpr int NTL = TB * (TB + 1) / 2;   // tiles on or above the diagonal: one per wave
    static constexpr int NT = 64 * NTL;
    static constexpr int FPI = D == 128 ? 4 : 8;    // features per conversion item (4 rows each)
    static constexpr int ITEMS = 16 * (D / FPI);    // conversion items per step of 64 rows
    static_assert(ITEMS <= NT, "one conversion item per thread and step");
};
constexpr int kRbSigRows = 4096;  // rows per workgroup: 3 * 2^14 * 4096 < 2^31
constexpr int kRbSigStep = 64;    // rows per LDS step (two MFMA k-steps of 32)
static_assert(3 * (1 << 14) * (long long)kRbSigRows < (1ll << 31), "int32 digit sums must stay exact");

// dword of digit-plane row f (16 dwords: 64 rows of K, one byte each) holding rows 16c + 4w ..
// 16c + 4w + 3; the 16-byte chunks are rotated by (f / 4) % 4 so that lanes reading one chunk of
// 32 consecutive feature rows spread over the banks
__device__ __forceinline__ int rb_plane_dw(int f, int c, int w) { return f * 16 + 4 * (c ^ ((f >> 2) & 3)) + w; }

// W consecutive elements of a row of K, kept raw until converted.
template <typename T, int W> struct RbRaw;
template <typename T> struct RbRaw<T, 8> : Raw8<T> {};
template <> struct RbRaw<__bf16, 4> {
    uint2 u;
    __device__ __forceinline__ void load(const __bf16* p) { u = *reinterpret_cast<const uint2*>(p); }
    __device__ __forceinline__ void widen(float (&v)[4]) const {
        v[0] = __uint_as_float(u.x << 16);
        v[1] = __uint_as_float(u.x & 0xffff0000u);
        v[2] = __uint_as_float(u.y << 16);
        v[3] = __uint_as_float(u.y & 0xffff0000u);
    }
};
template <> struct RbRaw<float, 4> {
    f32x4 a;
    __device__ __forceinline__ void load(const float* p) { a = *reinterpret_cast<const f32x4*>(p); }
    __device__ __forceinline__ void widen(float (&v)[4]) const {
#pragma unroll
        for (int j = 0; j < 4; ++j) v[j] = a[j];
    }
};

// k^ = rint(k 2^s) as the three balanced base-256 digits in bytes 0..2: with x = k^, the bytes of
// x + 0x808080 are d_i + 128 (each in [0, 255]: |x| <= 2^21), and flipping their top bits leaves
// d_i as a signed byte.  In binary32 when s <= 100 (k 2^s is then exact, or below 2^-26 in
// magnitude and rounds to 0 whether or not a subnormal k is kept), else in binary64.
template <bool F32>
__device__ __forceinline__ uint32_t rb_digits(float v, int sh) {
    const int x = F32 ? (int)rintf(ldexpf(v, sh)) : (int)rint(ldexp((double)v, sh));
    return (uint32_t)(x + 0x808080) ^ 0x808080u;
}

// Two buffers of digit planes: while the waves multiply one step's planes, the next step's rows
// (loaded a step earlier) are converted into the other.
template <typename T, int D>
__global__ __launch_bounds__(RbSig<D>::NT) void rb_sigma_kernel(const T* __restrict__ K, int N, int Nv,
                                                               const uint32_t* __restrict__ kmax,
                                                               long long* __restrict__ sint) {
    using S = RbSig<D>;
    constexpr int PL = 3 * D * 16;  // dwords of one buffer's three planes
    __shared__ __attribute__((aligned(16))) uint32_t pl[2 * PL];
    const int bh = blockIdx.y;
    const int r0 = blockIdx.x * kRbSigRows, r1 = min(Nv, r0 + kRbSigRows);
    const int sh = fixed_point_shift(kmax[bh]);
    const int lane = threadIdx.x & 63, wv = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
    const T* kh = K + (size_t)bh * N * D;

    // this wave's tile of the upper triangle (rows of blocks one after another)
    int ta = 0, tb;
    {
        int rest = wv;
        while (rest >= S::TB - ta) {
            rest -= S::TB - ta;
            ++ta;
        }
        tb = ta + rest;
    }
    i32x16 acc[5];
#pragma unroll
    for (int q = 0; q < 5; ++q)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[q][r] = 0;

    // conversion item of this thread: rows 4*tk4 .. +3, features FPI*fc .. of a step
    constexpr int FPI = S::FPI;
    const bool conv = (int)threadIdx.x < S::ITEMS;
    const int tk4 = (int)threadIdx.x / (D / FPI), fc = (int)threadIdx.x % (D / FPI);
    const bool f32 = sh <= 100;
    RbRaw<T, FPI> nx[4];  // rows of the next step to convert
    auto fetch = [&](int rs) __attribute__((always_inline)) {
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int r = rs + 4 * tk4 + u;
            if (conv && r < r1) nx[u].load(kh + (size_t)r * D + FPI * fc);
        }
    };
    auto convert = [&](int rs, uint32_t* buf) __attribute__((always_inline)) {
        if (!conv) return;
        uint32_t z[4][FPI];  // digits of row u, feature j
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            float v[FPI] = {};
            if (rs + 4 * tk4 + u < r1) nx[u].widen(v);
#pragma unroll
            for (int j = 0; j < FPI; ++j) z[u][j] = f32 ? rb_digits<true>(v[j], sh) : rb_digits<false>(v[j], sh);
        }
        // per feature, byte p of the four rows' digit words into one dword of plane p
#pragma unroll
        for (int j = 0; j < FPI; ++j) {
            const uint32_t a = __builtin_amdgcn_perm(z[1][j], z[0][j], 0x05010400u);  // r0.d0 r1.d0 r0.d1 r1.d1
            const uint32_t b = __builtin_amdgcn_perm(z[3][j], z[2][j], 0x05010400u);  // r2.d0 r3.d0 r2.d1 r3.d1
            const uint32_t c = __builtin_amdgcn_perm(z[1][j], z[0][j], 0x0c0c0602u);  // r0.d2 r1.d2
            const uint32_t e = __builtin_amdgcn_perm(z[3][j], z[2][j], 0x0c0c0602u);  // r2.d2 r3.d2
            const int dw = rb_plane_dw(FPI * fc + j, tk4 >> 2, tk4 & 3);
            buf[dw] = __builtin_amdgcn_perm(b, a, 0x05040100u);
            buf[D * 16 + dw] = __builtin_amdgcn_perm(b, a, 0x07060302u);
            buf[2 * D * 16 + dw] = __builtin_amdgcn_perm(e, c, 0x05040100u);
        }
    };
    fetch(r0);
    convert(r0, pl);
    if (r0 + kRbSigStep < r1) fetch(r0 + kRbSigStep);
    __syncthreads();
    for (int rs = r0, cur = 0; rs < r1; rs += kRbSigStep, cur ^= 1) {
        const uint32_t* bp = pl + cur * PL;
        if (rs + kRbSigStep < r1) {
            convert(rs + kRbSigStep, pl + (cur ^ 1) * PL);
            if (rs + 2 * kRbSigStep < r1) fetch(rs + 2 * kRbSigStep);
        }
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            i32x4 A[3], B[3];
#pragma unroll
            for (int p = 0; p < 3; ++p) {
                A[p] = *reinterpret_cast<const i32x4*>(bp + p * D * 16 + rb_plane_dw(32 * ta + (lane & 31), 2 * ks + (lane >> 5), 0));
                B[p] = *reinterpret_cast<const i32x4*>(bp + p * D * 16 + rb_plane_dw(32 * tb + (lane & 31), 2 * ks + (lane >> 5), 0));
            }
#pragma unroll
            for (int p = 0; p < 3; ++p)
#pragma unroll
                for (int q = 0; q < 3; ++q)
                    acc[p + q] = __builtin_amdgcn_mfma_i32_32x32x32_i8(A[p], B[q], acc[p + q], 0, 0, 0);
        }
        __syncthreads();
    }
    // accumulator register r of lane l: Sigma row 32 ta + 8 (r / 4) + 4 (l / 32) + r % 4, column
    // 32 tb + l % 32; the entries on or above the diagonal are added
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        const int a = 32 * ta + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3), c = 32 * tb + (lane & 31);
        if (a > c) continue;
        long long v = 0;
#pragma unroll
        for (int q = 0; q < 5; ++q) v += (long long)acc[q][r] << (8 * q);
        atomicAdd((unsigned long long*)&sint[((size_t)bh * D + a) * D + c], (unsigned long long)v);
    }
}

// Sigma_ab = ((double)sum * 2^(-2s)) / N_v, mirrored from the upper triangle (exactly symmetric).
__global__ __launch_bounds__(256) void rb_sigma_finalize_kernel(const long long* __restrict__ sint,
                                                                const uint32_t* __restrict__ kmax, int D, int Nv,
                                                                double* __restrict__ sigma) {
    const int bh = blockIdx.y, e = blockIdx.x * 256 + threadIdx.x;
    if (e >= D * D) return;
    const int a = e / D, c = e % D;
    const int lo = min(a, c), hi = max(a, c);
    const int sh = fixed_point_shift(kmax[bh]);
    const long long v = sint[((size_t)bh * D + lo) * D + hi];
    sigma[((size_t)bh * D + a) * D + c] = ldexp((double)v, -2 * sh) / (double)Nv;
}

// A zero the compiler cannot see through: added to an LDS address inside a loop, it keeps the
// loads of a loop-invariant vector in the loop instead of hoisted into registers.
__device__ __forceinline__ uint32_t rb_opaque_zero() {
    uint32_t z;
    asm volatile("s_mov_b32 %0, 0" : "=s"(z));
    return z;
}

// A token row of D elements kept as raw bits (D/8 sixteen-byte loads issued back to back).
template <typename T, int D>
struct RbRow {
    Raw8<T> p[D / 8];
    __device__ __forceinline__ void load(const T* __restrict__ q) {
#pragma unroll
        for (int k = 0; k < D / 8; ++k) p[k].load(q + 8 * k);
    }
};

// An empty asm that claims to change a row's bits: a row reused across passes is then widened
// again in each pass instead of kept widened in twice the registers.
__device__ __forceinline__ void rb_launder(Raw8<__bf16>& r) { asm volatile("" : "+v"(r.u)); }
__device__ __forceinline__ void rb_launder(Raw8<float>& r) { asm volatile("" : "+v"(r.a), "+v"(r.b)); }

// fma chain over a = 0..D-1 of q_a g_a.
template <typename T, int D>
__device__ __forceinline__ double rb_dot(const RbRow<T, D>& r, const double* gv) {
    double acc = 0.0;
#pragma unroll
    for (int k = 0; k < D / 8; ++k) {
        float v[8];
        r.p[k].widen(v);
#pragma unroll
        for (int e = 0; e < 8; ++e) acc = fma((double)v[e], gv[8 * k + e], acc);
    }
    return acc;
}

// One element of a token row as raw bits (bf16 in the low half, or fp32), and its binary64 value.
template <typename T> __device__ __forceinline__ uint32_t rb_elem_bits(const T* p);
template <> __device__ __forceinline__ uint32_t rb_elem_bits<__bf16>(const __bf16* p) {
    return *reinterpret_cast<const uint16_t*>(p);
}
template <> __device__ __forceinline__ uint32_t rb_elem_bits<float>(const float* p) {
    return *reinterpret_cast<const uint32_t*>(p);
}
template <typename T> __device__ __forceinline__ double rb_bits_f64(uint32_t v) {
    return (double)__uint_as_float(sizeof(T) == 2 ? v << 16 : v);
}

typedef double f64x4 __attribute__((ext_vector_type(4)));

// n_i for every video query on the binary64 matrix cores.  v_mfma_f64_16x16x4f64 accumulates its
// four products into C one fused multiply-add at a time, in k order (a probe on the device matched
// the chain fma(a3 b3, fma(a2 b2, fma(a1 b1, fma(a0 b0, c)))) on 131,072 of 131,072 outputs of
// random operands spanning 20 binades, and no other order), so a chain of these instructions over
// k-steps 0, 1, ... is the fixed binary64 order of the norm bit for bit:
//  * t_a = fma(Sigma_ab, q_b, t_a) over b ascending: D1 = A1 B1 with A1[i][k] = Sigma[4s+k][16c+i] (c the
//    16-column tile of a) and B1[k][j] = q_j[4s+k], s = 0 .. D/4-1, so D1[i][j] = t_{16c+i} of row j;
//  * r = fma(q_a, t_a, r) over a ascending: D2 = A2 B2 with A2[i][k] = q_i[4s+k] and B2[k][j] =
//    t_{4s+k} of row j; its diagonal D2[j][j] is r of row j (the rest is not used).
// Operand layouts (lane l, one fp64 each): A[l % 16][l / 16], B[l / 16][l % 16]; accumulator register
// r of lane l is D[4r + l / 16][l % 16].  So B2 of step s is D1 register s % 4 of tile s / 4 in the
// same lane, and A2 is B1: no data moves between lanes.  A wave takes 16 rows at a time (lane l:
// row l % 16, its elements b = l / 16 mod 4); Sigma of the (batch, head) sits in LDS (128 KB at
// d = 128), staged once per head; the resident workgroups split the (head, 16-row block) items
// evenly.
constexpr int kRbNrmWaves = 8;

template <typename T, int D>
__global__ __launch_bounds__(64 * kRbNrmWaves) void rb_norms_kernel(const T* __restrict__ Q, int N, int Nv, int BH,
                                                                    const double* __restrict__ sigma,
                                                                    double* __restrict__ nrm) {
    __shared__ __attribute__((aligned(16))) double sS[D * D];
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, jr = lane & 15, kq = lane >> 4;
    const long long nb = (Nv + 15) / 16, items = nb * BH;
    const long long i0 = items * blockIdx.x / gridDim.x, i1 = items * (blockIdx.x + 1) / gridDim.x;
    for (long long seg = i0; seg < i1;) {
        const int bh = (int)(seg / nb);
        const long long seg_end = min(i1, (long long)(bh + 1) * nb);
        __syncthreads();  // the previous head's Sigma is no longer read
        const f64x2* src = reinterpret_cast<const f64x2*>(sigma + (size_t)bh * D * D);
        for (int e = threadIdx.x; e < D * D / 2; e += 64 * kRbNrmWaves) reinterpret_cast<f64x2*>(sS)[e] = src[e];
        __syncthreads();
        // lane l needs only the elements b = 4s + l / 16 of its row: D / 4 loads per block, and the
        // next block's are in flight while this block's products run
        uint32_t qc[D / 4], qn[D / 4];
        auto load_q = [&](uint32_t (&dst)[D / 4], long long item) __attribute__((always_inline)) {
            const int rw = min((int)(item - (long long)bh * nb) * 16 + jr, Nv - 1);
            const T* src = Q + ((size_t)bh * N + rw) * D + kq;
#pragma unroll
            for (int s = 0; s < D / 4; ++s) dst[s] = rb_elem_bits<T>(src + 4 * s);
        };
        if (seg + w < seg_end) load_q(qc, seg + w);
        for (long long it = seg + w; it < seg_end; it += kRbNrmWaves) {
            const int row = (int)(it - (long long)bh * nb) * 16 + jr;
            if (it + kRbNrmWaves < seg_end) load_q(qn, it + kRbNrmWaves);
            f64x4 t[D / 16];
#pragma unroll
            for (int c = 0; c < D / 16; ++c) t[c] = f64x4{0.0, 0.0, 0.0, 0.0};
#pragma unroll
            for (int s = 0; s < D / 4; ++s) {
                // keeps the compiler from hoisting the LDS reads of every step to the top (they
                // would need 2 * D * D / 64 registers)
                __builtin_amdgcn_sched_barrier(0);
                const double qb = rb_bits_f64<T>(qc[s]);
#pragma unroll
                for (int c = 0; c < D / 16; ++c)
                    t[c] = __builtin_amdgcn_mfma_f64_16x16x4f64(sS[(4 * s + kq) * D + 16 * c + jr], qb, t[c], 0, 0, 0);
            }
            f64x4 r = {0.0, 0.0, 0.0, 0.0};
#pragma unroll
            for (int s = 0; s < D / 4; ++s)
                r = __builtin_amdgcn_mfma_f64_16x16x4f64(rb_bits_f64<T>(qc[s]), t[s >> 2][s & 3], r, 0, 0, 0);
            // the diagonal: row jr's r is register jr / 4 of the lane with l / 16 = jr % 4
            if ((jr & 3) == kq && row < Nv) {
                const double v = r[jr >> 2];
                nrm[(size_t)bh * Nv + row] = v > 0.0 ? sqrt(v) : 0.0;
            }
#pragma unroll
            for (int s = 0; s < D / 4; ++s) qc[s] = qn[s];
        }
        seg = seg_end;
    }
}

// g(P) = t(P) / n_P into gv[0..D): thread a computes t_a = fma chain over b of Sigma_ab q_Pb.
// Sigma is exactly symmetric, so Sigma_ab is read as Sigma[b][a]: at each b the lanes read one
// contiguous row segment.
template <typename T, int D, int NT>
__device__ __forceinline__ void rb_pivot(const double* __restrict__ sigma, const double* __restrict__ nrm,
                                         const T* __restrict__ Qh, int P, double* gv) {
    for (int a = threadIdx.x; a < D; a += NT) {
        const double nP = nrm[P];
        double g = 0.0;
        if (nP != 0.0) {
            const T* qp = Qh + (size_t)P * D;
            double t = 0.0;
#pragma unroll 16
            for (int b = 0; b < D; ++b) t = fma(sigma[(size_t)b * D + a], (double)elem_f<T>(qp + b), t);
            g = t / nP;
        }
        gv[a] = g;
    }
}

// cos(i, P) = (fma chain over a of q_ia g_a(P)) / n_i (0 when n_i = 0) for the positions
// jb + tid, jb + tid + NT, ... below je of an order segment; f(j, i, cos) sees each one.  One row
// per thread is live (no row loaded ahead), so the kernels that use this fit 4-5 waves per SIMD;
// loading the next row ahead instead, at 3 waves, took the same time.
template <typename T, int D, int NT, typename F>
__device__ __forceinline__ void rb_cos_range(const T* __restrict__ Qh, const double* __restrict__ nrm,
                                             const int32_t* __restrict__ seg, int jb, int je, const double* gv,
                                             F&& f) {
    int j = jb + (int)threadIdx.x;
    if (j >= je) return;
    int i = seg[j];
    for (;;) {
        const int jn = j + NT;
        const bool more = jn < je;
        RbRow<T, D> r;
        r.load(Qh + (size_t)i * D);
        const double ni = nrm[i];
        const int i1 = more ? seg[jn] : 0;
        const double acc = rb_dot<T, D>(r, gv + rb_opaque_zero());
        f(j, i, ni == 0.0 ? 0.0 : acc / ni);
        if (!more) break;
        j = jn;
        i = i1;
    }
}

// rb_cos_range with the rows gathered cooperatively: a wave takes 64 consecutive positions (lane l:
// position j0 + l, the same position-to-thread map as rb_cos_range's) and loads their rows straight
// into a wave-private LDS buffer (buffer_load ... lds), each load instruction covering whole rows
// (16 lanes per 256-byte row).  Chunk c of row r sits at chunk slot c ^ (r mod 16) (the lane loading
// slot s of row r fetches source chunk s ^ (r mod 16)), so each lane then reads its own row
// conflict-free and runs the same fma chain.  A timing probe of the gather on the box (75,600 x 24
// rows of 256 bytes, 2048 positions per workgroup) took 0.103-0.105 ms with whole-row loads staged
// through LDS against 0.121-0.124 ms with one row per thread.  bf16 rows only (16 chunks of 16
// bytes at d = 128, 8 at d = 64); stage holds 64 rows per wave.
// 16-byte words of the staging buffer of a workgroup of NT threads: 64 rows per wave for bf16 rows,
// none (one word) for fp32 rows, which are read one per thread.
template <typename T, int D, int NT>
constexpr int kRbStageWords = std::is_same<T, __bf16>::value ? NT / 64 * 64 * (D / 8) : 1;

template <int D, int NT, typename F>
__device__ __forceinline__ void rb_cos_range_staged(const __bf16* __restrict__ Qh, uint32_t q_bytes,
                                                    const double* __restrict__ nrm,
                                                    const int32_t* __restrict__ seg, int jb, int je,
                                                    const double* gv, u32x4* __restrict__ stage, F&& f) {
    constexpr int CPR = D / 8;     // 16-byte chunks per row
    constexpr int RPI = 64 / CPR;  // rows per load instruction
    const int lane = threadIdx.x & 63, w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    u32x4* B = stage + (size_t)w * 64 * CPR;
    int j0 = jb + 64 * w;
    if (j0 >= je) return;  // uniform for the wave
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(const_cast<__bf16*>(Qh), (short)0,
                                                                        (int)q_bytes, 0x00020000);
    int inext = seg[min(j0 + lane, je - 1)];
    for (; j0 < je; j0 += NT) {
        const int j = j0 + lane, iown = inext;
        if (j0 + NT < je) inext = seg[min(j0 + NT + lane, je - 1)];
#pragma unroll
        for (int u = 0; u < CPR; ++u) {
            const int r = u * RPI + lane / CPR;
            const int i = __shfl(iown, r);
            const uint32_t src = (uint32_t)i * (D * 2) + (uint32_t)(((lane % CPR) ^ (r % CPR)) * 16);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                rs, (__attribute__((address_space(3))) void*)(B + u * 64), 16, src, 0, 0, 0);
        }
        const double ni = nrm[iown];
        __builtin_amdgcn_s_waitcnt(0);  // the staged rows have landed (vector memory count 0)
        __builtin_amdgcn_wave_barrier();
        // the chain reads its row chunk and the eight g values of chunk c + 1 while it runs chunk c:
        // their addresses carry a zero that depends on the chain's value after chunk c - 1, so the
        // compiler cannot hoist every LDS read to the top (their values would need ~300 registers)
        const double* gp = gv;
        Raw8<__bf16> cur, nxt;
        double gc[8], gn[8];
        cur.u = B[lane * CPR + (0 ^ (lane % CPR))];
#pragma unroll
        for (int e = 0; e < 8; ++e) gc[e] = gp[e];
        double acc = 0.0;
#pragma unroll
        for (int c = 0; c < CPR; ++c) {
            if (c + 1 < CPR) {
                uint32_t z;
                asm volatile("v_mov_b32 %0, 0" : "=v"(z) : "v"(acc));
                nxt.u = B[lane * CPR + ((c + 1) ^ (lane % CPR)) + z];
#pragma unroll
                for (int e = 0; e < 8; ++e) gn[e] = gp[8 * (c + 1) + e + z];
            }
            float v[8];
            cur.widen(v);
#pragma unroll
            for (int e = 0; e < 8; ++e) acc = fma((double)v[e], gc[e], acc);
            cur = nxt;
#pragma unroll
            for (int e = 0; e < 8; ++e) gc[e] = gn[e];
        }
        if (j < je) f(j, iown, ni == 0.0 ? 0.0 : acc / ni);
        __builtin_amdgcn_s_waitcnt(0);  // this wave's reads of the stage precede its next loads into it
        __builtin_amdgcn_wave_barrier();
    }
}

// (k2, i2) before (k, i) in the lexicographic order.
__device__ __forceinline__ bool rb_before(uint64_t k2, int i2, uint64_t k, int i) {
    return k2 < k || (k2 == k && i2 < i);
}

// Lexicographic minimum of (key, idx) over the workgroup (result in every thread).
template <int NT>
__device__ __forceinline__ void rb_argmin(uint64_t& key, int& idx, uint64_t* skey, int* sidx) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
        const uint64_t k2 = __shfl_xor(key, o);
        const int i2 = __shfl_xor(idx, o);
        if (rb_before(k2, i2, key, idx)) {
            key = k2;
            idx = i2;
        }
    }
    if (lane == 0) {
        skey[w] = key;
        sidx[w] = idx;
    }
    __syncthreads();
    key = skey[0];
    idx = sidx[0];
    for (int v = 1; v < NT / 64; ++v) {
        const uint64_t k2 = skey[v];
        const int i2 = sidx[v];
        if (rb_before(k2, i2, key, idx)) {
            key = k2;
            idx = i2;
        }
    }
    __syncthreads();
}

// Leaves [L0, L0 + c) of group g of level lev: g's bits, most significant first, choose the
// child (0 = left, which takes ceil(c/2) leaves).
__device__ __forceinline__ void rb_group(int g, int lev, int M, int& L0, int& c) {
    L0 = 0;
    c = M;
    for (int b = lev - 1; b >= 0; --b) {
        const int cl = (c + 1) / 2;
        if ((g >> b) & 1) {
            L0 += cl;
            c -= cl;
        } else {
            c = cl;
        }
    }
}

constexpr int kRbU = 4;  // elements per thread in flight in the select and partition loops

template <int NT>
struct RbSplitShared {
    unsigned hist[NT / 64][256];
    int wc[2][kRbU * (NT / 64)];
    int tot[2];
    int sel_digit, sel_rem, sel_cnt;
    uint64_t thr_key;
    uint32_t thr_idx;
};

// Split a group of n order entries with keys dk (order (dk, index) ascending = (cos(., A) -
// cos(., B)) descending, index ascending): a radix select finds the nl-th smallest (dk, index)
// (8 digits of dk, then 3 of the index, which is below 2^24); a stable partition writes the nl
// smallest, in their current order, to out[0 .. nl) and the rest to out[nl .. n).  Once the
// chosen digit's bin holds a single entry, that entry is the nl-th smallest: one more sweep
// reads its key and index and the remaining digits are skipped.
template <int NT>
__device__ void rb_split(const uint64_t* __restrict__ dk, const int32_t* __restrict__ seg, int n, int nl,
                         int32_t* __restrict__ out, RbSplitShared<NT>& sh) {
    constexpr int NW = NT / 64, U = kRbU;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    uint64_t pre_hi = 0;
    uint32_t pre_lo = 0;
    int rem = nl;
    for (int pass = 0; pass < 11; ++pass) {
        for (int b = lane; b < 256; b += 64) sh.hist[w][b] = 0u;
        __syncthreads();
        for (int j0 = tid; j0 < n; j0 += U * NT) {
            uint64_t kk[U];
            uint32_t ii[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int j = j0 + u * NT;
                kk[u] = 0;
                ii[u] = 0;
                if (j < n) {
                    kk[u] = dk[j];
                    ii[u] = (uint32_t)seg[j];
                }
            }
#pragma unroll
            for (int u = 0; u < U; ++u) {
                if (j0 + u * NT >= n) continue;
                const uint64_t k = kk[u];
                const uint32_t i = ii[u];
                bool match;
                unsigned digit;
                if (pass < 8) {
                    match = pass == 0 || (k >> (64 - 8 * pass)) == pre_hi;
                    digit = (unsigned)(k >> (56 - 8 * pass)) & 255u;
                } else {
                    const int p = pass - 8;
                    match = k == pre_hi && (p == 0 || (i >> (24 - 8 * p)) == pre_lo);
                    digit = (i >> (16 - 8 * p)) & 255u;
                }
                if (match) atomicAdd(&sh.hist[w][digit], 1u);
            }
        }
        __syncthreads();
        if (w == 0) {
            // lane l owns bins 4l .. 4l+3
            unsigned cnt[4], tot = 0;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                unsigned v = 0;
                for (int u = 0; u < NW; ++u) v += sh.hist[u][4 * lane + q];
                cnt[q] = v;
                tot += v;
            }
            unsigned inc = tot;
#pragma unroll
            for (int o = 1; o < 64; o <<= 1) {
                const unsigned y = __shfl_up(inc, o);
                if (lane >= o) inc += y;
            }
            const unsigned before = inc - tot;  // count of bins below 4*lane
            // the lane whose range holds the rem-th element picks the bin
            if ((int)before < rem && rem <= (int)inc) {
                unsigned cum = before, csel = cnt[3];
                int dsel = 4 * lane + 3;
                for (int q = 0; q < 4; ++q) {
                    if ((int)(cum + cnt[q]) >= rem) {
                        dsel = 4 * lane + q;
                        csel = cnt[q];
                        break;
                    }
                    cum += cnt[q];
                }
                sh.sel_digit = dsel;
                sh.sel_rem = rem - (int)cum;
                sh.sel_cnt = (int)csel;
            }
        }
        __syncthreads();
        const unsigned dsel = (unsigned)sh.sel_digit;
        const int csel = sh.sel_cnt;
        rem = sh.sel_rem;
        if (pass < 8) pre_hi = (pre_hi << 8) | dsel;
        else pre_lo = (pre_lo << 8) | dsel;
        __syncthreads();
        if (csel == 1 && pass < 10) {
            // the one entry with this prefix is the threshold: take its whole key and index
            for (int j = tid; j < n; j += NT) {
                const uint64_t k = dk[j];
                const uint32_t i = (uint32_t)seg[j];
                const bool match = pass < 8 ? (k >> (56 - 8 * pass)) == pre_hi
                                            : k == pre_hi && (i >> (16 - 8 * (pass - 8))) == pre_lo;
                if (match) {
                    sh.thr_key = k;
                    sh.thr_idx = i;
                }
            }
            __syncthreads();
            pre_hi = sh.thr_key;
            pre_lo = sh.thr_idx;
            break;
        }
    }
    // stable partition, U*NT positions per tile: position t0 + u*NT + tid is the (u, wave, lane)-th
    const uint64_t below = lane == 0 ? 0ull : (~0ull >> (64 - lane));
    int lbase = 0, rbase = 0;
    for (int t0 = 0; t0 < n; t0 += U * NT) {
        bool valid[U], left[U];
        int ii[U];
        uint64_t bl[U], br[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int j = t0 + u * NT + tid;
            valid[u] = j < n;
            uint64_t k = 0;
            ii[u] = 0;
            if (valid[u]) {
                k = dk[j];
                ii[u] = seg[j];
            }
            left[u] = k < pre_hi || (k == pre_hi && (uint32_t)ii[u] <= pre_lo);
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            bl[u] = __ballot(valid[u] && left[u]);
            br[u] = __ballot(valid[u] && !left[u]);
            if (lane == 0) {
                sh.wc[0][u * NW + w] = __popcll(bl[u]);
                sh.wc[1][u * NW + w] = __popcll(br[u]);
            }
        }
        __syncthreads();
        if (w == 0) {
            // exclusive prefix over (u, wave) in position order, per side; totals for the tile
#pragma unroll
            for (int side = 0; side < 2; ++side) {
                const int v = lane < U * NW ? sh.wc[side][lane] : 0;
                int inc = v;
#pragma unroll
                for (int o = 1; o < 64; o <<= 1) {
                    const int y = __shfl_up(inc, o);
                    if (lane >= o) inc += y;
                }
                if (lane < U * NW) sh.wc[side][lane] = inc - v;
                if (lane == 63) sh.tot[side] = inc;
            }
        }
        __syncthreads();
#pragma unroll
        for (int u = 0; u < U; ++u) {
            if (!valid[u]) continue;
            if (left[u]) out[lbase + sh.wc[0][u * NW + w] + __popcll(bl[u] & below)] = ii[u];
            else out[nl + rbase + sh.wc[1][u * NW + w] + __popcll(br[u] & below)] = ii[u];
        }
        lbase += sh.tot[0];
        rbase += sh.tot[1];
        __syncthreads();
    }
}

// Whether group g of level lev has its parent's P0 (never at level 0).  The parent's segment is
// the two children's segments one after the other, each in ascending index, so the parent's P0 (its
// lowest index) is the lower of the two children's first entries; the child whose first entry that
// is keeps it as its own P0, and cos(., P0) of its members is in c0 already.  It reads this level's
// order only, which no pass of the level writes.
__device__ __forceinline__ bool rb_keeps_p0(const int32_t* ord, int g, int lev, int M, int BLK, int first) {
    if (lev == 0) return false;
    int L0s, cs;
    rb_group(g ^ 1, lev, M, L0s, cs);  // the sibling: not empty, since the parent was split
    return first < ord[(size_t)L0s * BLK];
}

// One level for groups that fit one workgroup: workgroup (group g of this level, (batch, head)).
// A group of one leaf is copied; a group of more leaves is split.  Every group's order segment
// is in ascending token index (the start is the identity and every partition is stable), so
// P0, its lowest index, is its first entry.
template <typename T, int D, int NT>
__global__ __launch_bounds__(NT) void rb_level_kernel(const T* __restrict__ Q, int N, int Nv, int BLK, int M, int lev,
                                                      const double* __restrict__ sigma_all,
                                                      const double* __restrict__ nrm_all,
                                                      const int32_t* __restrict__ ord_in_all,
                                                      int32_t* __restrict__ ord_out_all, double* __restrict__ cbuf_all,
                                                      uint64_t* __restrict__ dk_all) {
    constexpr int NW = NT / 64;
    __shared__ double gv[D];
    __shared__ uint64_t skey[NW];
    __shared__ int sidx[NW];
    __shared__ RbSplitShared<NT> sh;
    __shared__ __attribute__((aligned(16))) u32x4 stage[kRbStageWords<T, D, NT>];

    const int bh = blockIdx.y, g = blockIdx.x, tid = threadIdx.x;
    int L0, c;
    rb_group(g, lev, M, L0, c);
    if (c <= 0) return;
    const int s0 = L0 * BLK, n = min(s0 + c * BLK, Nv) - s0;
    const int32_t* seg = ord_in_all + (size_t)bh * Nv + s0;
    int32_t* out = ord_out_all + (size_t)bh * Nv + s0;
    if (c == 1) {
        for (int j = tid; j < n; j += NT) out[j] = seg[j];
        return;
    }
    const T* Qh = Q + (size_t)bh * N * D;
    const double* sigma = sigma_all + (size_t)bh * D * D;
    const double* nrm = nrm_all + (size_t)bh * Nv;
    double* cb = cbuf_all + (size_t)bh * Nv + s0;
    uint64_t* dk = dk_all + (size_t)bh * Nv + s0;

    // bf16 rows are gathered by whole-row loads staged through LDS, fp32 rows one per thread
    auto cos_range = [&](auto&& f) __attribute__((always_inline)) {
        if constexpr (std::is_same<T, __bf16>::value)
            rb_cos_range_staged<D, NT>(Qh, (uint32_t)((size_t)N * D * sizeof(T)), nrm, seg, 0, n, gv, stage, f);
        else
            rb_cos_range<T, D, NT>(Qh, nrm, seg, 0, n, gv, f);
    };
    rb_pivot<T, D, NT>(sigma, nrm, Qh, seg[0], gv);
    __syncthreads();
    // A = argmin cos(., P0), ties to the lower index
    uint64_t kmin = ~0ull;
    int A = INT_MAX;
    cos_range([&](int, int i, double cs) {
        const uint64_t k = asc_key(cs);
        if (rb_before(k, i, kmin, A)) {
            kmin = k;
            A = i;
        }
    });
    rb_argmin<NT>(kmin, A, skey, sidx);
    rb_pivot<T, D, NT>(sigma, nrm, Qh, A, gv);
    __syncthreads();
    // B = argmin cos(., A); cos(., A) is kept for the key
    kmin = ~0ull;
    int B = INT_MAX;
    cos_range([&](int j, int i, double cs) {
        cb[j] = cs;
        const uint64_t k = asc_key(cs);
        if (rb_before(k, i, kmin, B)) {
            kmin = k;
            B = i;
        }
    });
    rb_argmin<NT>(kmin, B, skey, sidx);
    rb_pivot<T, D, NT>(sigma, nrm, Qh, B, gv);
    __syncthreads();
    // key = cos(., A) - cos(., B); order (key desc, index asc) = (~asc_key(key), index) asc.
    // Each position is revisited by the thread that wrote its cos(., A).
    cos_range([&](int j, int, double cs) { dk[j] = ~asc_key(cb[j] - cs); });
    __syncthreads();
    rb_split<NT>(dk, seg, n, ((c + 1) / 2) * BLK, out, sh);
}

// Levels whose groups span several chunks of kRbChunk order positions run the three cos passes
// over (group, chunk) workgroups.  Partials of an argmin are stored per (group, chunk); a pivot
// launch, one workgroup of D threads per group, reduces them (or takes P0 = the segment's first
// entry) and writes g(P) for the next pass.
template <typename T, int D>
__global__ __launch_bounds__(D) void rb_chunk_pivot_kernel(const T* __restrict__ Q, int N, int Nv, int BLK, int M,
                                                           int lev, int nch, const double* __restrict__ sigma_all,
                                                           const double* __restrict__ nrm_all,
                                                           const int32_t* __restrict__ ord_in_all,
                                                           const uint64_t* __restrict__ pkey,
                                                           const int* __restrict__ pidx, double* __restrict__ gbuf,
                                                           int first) {
    __shared__ uint64_t skey[D / 64];
    __shared__ int sidx[D / 64];
    const int bh = blockIdx.y, g = blockIdx.x, G = gridDim.x;
    int L0, c;
    rb_group(g, lev, M, L0, c);
    if (c <= 1) return;
    const int s0 = L0 * BLK;
    int P;
    if (first) {
        P = ord_in_all[(size_t)bh * Nv + s0];
    } else {
        const size_t base = ((size_t)bh * G + g) * nch;
        uint64_t k = ~0ull;
        P = INT_MAX;
        for (int ch = threadIdx.x; ch < nch; ch += D) {
            const uint64_t k2 = pkey[base + ch];
            const int i2 = pidx[base + ch];
            if (rb_before(k2, i2, k, P)) {
                k = k2;
                P = i2;
            }
        }
        rb_argmin<D>(k, P, skey, sidx);
    }
    rb_pivot<T, D, D>(sigma_all + (size_t)bh * D * D, nrm_all + (size_t)bh * Nv, Q + (size_t)bh * N * D, P,
                      gbuf + ((size_t)bh * G + g) * D);
}

// MODE 0: argmin partial of cos(., P0); 1: cos(., A) kept and argmin partial; 2: the key dk.
// MODE 0 also keeps cos(., P0) per token in c0 (see rb_keeps_p0).
template <typename T, int D, int MODE>
__global__ __launch_bounds__(kRbChunkThreads, 2) void rb_chunk_cos_kernel(
    const T* __restrict__ Q, int N, int Nv, int BLK, int M, int lev, int nch, const double* __restrict__ nrm_all,
    const int32_t* __restrict__ ord_in_all, const double* __restrict__ gbuf, double* __restrict__ cbuf_all,
    uint64_t* __restrict__ dk_all, uint64_t* __restrict__ pkey, int* __restrict__ pidx,
    double* __restrict__ c0_all) {
    constexpr int NT = kRbChunkThreads;
    __shared__ double gv[D];
    __shared__ uint64_t skey[NT / 64];
    __shared__ int sidx[NT / 64];
    __shared__ __attribute__((aligned(16))) u32x4 stage[kRbStageWords<T, D, NT>];
    const int bh = blockIdx.y, g = blockIdx.x / nch, ch = blockIdx.x % nch, G = gridDim.x / nch;
    int L0, c;
    rb_group(g, lev, M, L0, c);
    if (c <= 1) return;
    const int s0 = L0 * BLK, n = min(s0 + c * BLK, Nv) - s0;
    // the group's positions split evenly over its nch chunks (at most kRbChunk each), so that no
    // workgroup of the pass holds many more positions than the others
    const int jb = (int)((long long)ch * n / nch), je = (int)((long long)(ch + 1) * n / nch);
    if (jb >= je) {  // no positions (not met at the sizes that run chunked): a neutral partial
        if (MODE != 2 && threadIdx.x == 0) {
            const size_t at = ((size_t)bh * G + g) * nch + ch;
            pkey[at] = ~0ull;
            pidx[at] = INT_MAX;
        }
        return;
    }
    const double* gsrc = gbuf + ((size_t)bh * G + g) * D;
    for (int a = threadIdx.x; a < D; a += NT) gv[a] = gsrc[a];
    __syncthreads();
    const T* Qh = Q + (size_t)bh * N * D;
    const double* nrm = nrm_all + (size_t)bh * Nv;
    const int32_t* seg = ord_in_all + (size_t)bh * Nv + s0;
    double* cb = cbuf_all + (size_t)bh * Nv + s0;
    uint64_t* dk = dk_all + (size_t)bh * Nv + s0;
    // bf16 rows are gathered by whole-row loads staged through LDS, fp32 rows one per thread
    auto cos_range = [&](auto&& f) __attribute__((always_inline)) {
        if constexpr (std::is_same<T, __bf16>::value)
            rb_cos_range_staged<D, NT>(Qh, (uint32_t)((size_t)N * D * sizeof(T)), nrm, seg, jb, je, gv, stage, f);
        else
            rb_cos_range<T, D, NT>(Qh, nrm, seg, jb, je, gv, f);
    };
    if (MODE == 2) {
        cos_range([&](int j, int, double cs) { dk[j] = ~asc_key(cb[j] - cs); });
        return;
    }
    uint64_t kmin = ~0ull;
    int P = INT_MAX;
    double* c0 = MODE == 0 ? c0_all + (size_t)bh * Nv : nullptr;
    if (MODE == 0 && rb_keeps_p0(ord_in_all + (size_t)bh * Nv, g, lev, M, BLK, seg[0])) {
        // the same P0 as the parent's: cos(., P0) of every member is in c0 already
        for (int j = jb + (int)threadIdx.x; j < je; j += NT) {
            const int i = seg[j];
            const uint64_t k = asc_key(c0[i]);
            if (rb_before(k, i, kmin, P)) {
                kmin = k;
                P = i;
            }
        }
    } else {
        cos_range([&](int j, int i, double cs) {
            if (MODE == 0) c0[i] = cs;
            if (MODE == 1) cb[j] = cs;
            const uint64_t k = asc_key(cs);
            if (rb_before(k, i, kmin, P)) {
                kmin = k;
                P = i;
            }
        });
    }
    rb_argmin<NT>(kmin, P, skey, sidx);
    if (threadIdx.x == 0) {
        const size_t at = ((size_t)bh * G + g) * nch + ch;
        pkey[at] = kmin;
        pidx[at] = P;
    }
}

// Select and partition of a chunked level: one workgroup per group.
template <int NT>
__global__ __launch_bounds__(NT) void rb_chunk_split_kernel(int Nv, int BLK, int M, int lev,
                                                            const int32_t* __restrict__ ord_in_all,
                                                            int32_t* __restrict__ ord_out_all,
                                                            const uint64_t* __restrict__ dk_all) {
    __shared__ RbSplitShared<NT> sh;
    const int bh = blockIdx.y, g = blockIdx.x;
    int L0, c;
    rb_group(g, lev, M, L0, c);
    if (c <= 0) return;
    const int s0 = L0 * BLK, n = min(s0 + c * BLK, Nv) - s0;
    const int32_t* seg = ord_in_all + (size_t)bh * Nv + s0;
    int32_t* out = ord_out_all + (size_t)bh * Nv + s0;
    if (c == 1) {
        for (int j = threadIdx.x; j < n; j += NT) out[j] = seg[j];
        return;
    }
    rb_split<NT>(dk_all + (size_t)bh * Nv + s0, seg, n, ((c + 1) / 2) * BLK, out, sh);
}

// The last levels of a group small enough for one token per thread (a subtree): each thread
// keeps its token's row, norm and current subgroup for the remaining levels, and the upper
// triangle of Sigma sits in LDS, so after the first loads everything stays on chip.  Per level
// and subgroup: P0 is the lowest member index; the thread holding a pivot publishes its row for
// g(P); the argmins are lexicographic minima in LDS (least key, then least index among that key);
// a member goes left when fewer than ceil(c/2)*block members precede it in (dk, index) order,
// exactly the membership the radix select and stable partition give.  That rank is the member's
// place in its subgroup's run after one bitonic sort of all (subgroup, dk, index) triples.  At the
// end a token's position is its leaf's start plus the number of members of the same leaf with a
// lower index.
// Members are in ascending index with the thread number, so thread numbers stand in for indexes
// in every tie-break.  The grid holds as many workgroups as stay resident; each claims (head,
// group) items from per-head counters, starting at head (id mod heads) so that with a multiple of 8
// heads an XCD (every eighth workgroup id) works on its own heads, and moves to any head with
// groups left once its own are spent.  The upper triangle of Sigma is staged once per head and
// workgroup.
constexpr int kRbSubThreads = 512;  // largest subtree: threads = tokens

// Lane l ^ J's value of v (J = 1 .. 32, a constant), by VALU cross-lane moves where one exists:
// DPP quad permutes for 1 and 2, v_permlane16/32_swap for 16 and 32 (the swap's outputs are told
// apart by swapping the lane numbers alongside, so the choice does not rest on their order), the
// swizzle's bit mode for 4 and 8.
struct RbXorLanes {
    bool first16, first32;
    __device__ __forceinline__ RbXorLanes() {
        const uint32_t l = threadIdx.x & 63;
        first16 = __builtin_amdgcn_permlane16_swap(l, l, false, false)[0] == (l ^ 16u);
        first32 = __builtin_amdgcn_permlane32_swap(l, l, false, false)[0] == (l ^ 32u);
    }
    template <int J>
    __device__ __forceinline__ uint32_t get(uint32_t v) const {
        if constexpr (J == 1) return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xF, 0xF, false);  // [1,0,3,2]
        else if constexpr (J == 2) return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x4E, 0xF, 0xF, false);  // [2,3,0,1]
        else if constexpr (J == 4 || J == 8) return (uint32_t)__builtin_amdgcn_ds_swizzle((int)v, (J << 10) | 0x1F);
        else if constexpr (J == 16) {
            const auto r = __builtin_amdgcn_permlane16_swap(v, v, false, false);
            return first16 ? r[0] : r[1];
        } else {
            static_assert(J == 32, "lane distance");
            const auto r = __builtin_amdgcn_permlane32_swap(v, v, false, false);
            return first32 ? r[0] : r[1];
        }
    }
};

// One compare-exchange of a bitonic network between thread t and t ^ j, given the partner's pair.
__device__ __forceinline__ void rb_bitonic_step(uint64_t& key, uint32_t& val, uint64_t kp, uint32_t vp, int t, int j,
                                                int k) {
    const uint32_t g = val >> 16, gp = vp >> 16;
    const bool after = g > gp || (g == gp && (key > kp || (key == kp && (val & 0xffffu) > (vp & 0xffffu))));
    // ascending runs where bit k of t is clear: there the lower partner keeps the smaller
    const bool keep_smaller = ((t & j) == 0) == ((t & k) == 0);
    if (after == keep_smaller) {
        key = kp;
        val = vp;
    }
}

template <int J>
__device__ __forceinline__ void rb_bitonic_lane_step(uint64_t& key, uint32_t& val, const RbXorLanes& xl, int t,
                                                     int k) {
    const uint64_t kp = ((uint64_t)xl.get<J>((uint32_t)(key >> 32)) << 32) | xl.get<J>((uint32_t)key);
    rb_bitonic_step(key, val, kp, xl.get<J>(val), t, J, k);
}

// Sort NT (key, val) pairs ascending by (val >> 16, key, val & 0xffff), thread t holding pair t in
// registers: a bitonic network.  Stages whose partners are lanes of one wave exchange through
// cross-lane moves; stages whose partners sit in other waves go through LDS (skey, sval), two
// barriers each.
template <int NT>
__device__ __forceinline__ void rb_bitonic_sort(uint64_t& key, uint32_t& val, uint64_t* skey, uint32_t* sval) {
    const int t = threadIdx.x;
    const RbXorLanes xl;
#pragma unroll 1
    for (int k = 2; k <= NT; k <<= 1) {
        int j = k >> 1;
#pragma unroll 1
        for (; j >= 64; j >>= 1) {
            skey[t] = key;
            sval[t] = val;
            __syncthreads();
            const uint64_t kp = skey[t ^ j];
            const uint32_t vp = sval[t ^ j];
            __syncthreads();
            rb_bitonic_step(key, val, kp, vp, t, j, k);
        }
        // j = min(k / 2, 32) down to 1
        if (j >= 32) rb_bitonic_lane_step<32>(key, val, xl, t, k);
        if (j >= 16) rb_bitonic_lane_step<16>(key, val, xl, t, k);
        if (j >= 8) rb_bitonic_lane_step<8>(key, val, xl, t, k);
        if (j >= 4) rb_bitonic_lane_step<4>(key, val, xl, t, k);
        if (j >= 2) rb_bitonic_lane_step<2>(key, val, xl, t, k);
        rb_bitonic_lane_step<1>(key, val, xl, t, k);
    }
}

__host__ __device__ constexpr int rb_tri(int a, int D) { return a * (2 * D - a + 1) / 2; }

// After head bh's groups are all claimed: the next head, in rotation from bh, with groups left
// (one read of every head's counter), or -1 when none has.  Every thread gets the same answer.
template <int NT>
__device__ int rb_next_head(const int32_t* hq, int BH, int G, int bh, int* s_pick) {
    if (threadIdx.x == 0) *s_pick = INT_MAX;
    __syncthreads();
    for (int j = 1 + (int)threadIdx.x; j < BH; j += NT)
        if (__hip_atomic_load(&hq[(bh + j) % BH], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < G)
            atomicMin(s_pick, j);
    __syncthreads();
    const int j = *s_pick;
    __syncthreads();  // read by every thread before it is written again
    return j == INT_MAX ? -1 : (bh + j) % BH;
}

template <typename T, int D, int NT>
__global__ __launch_bounds__(NT, sizeof(T) == 2 || D == 64 ? 4 : 1) void rb_subtree_kernel(const T* __restrict__ Q, int N, int Nv, int BLK,
                                                                   int M, int lev0, int nsub, int BH,
                                                                   const double* __restrict__ sigma_all,
                                                                   const double* __restrict__ nrm_all,
                                                                   const int32_t* __restrict__ ord_in_all,
                                                                   int32_t* __restrict__ perm_all,
                                                                   int32_t* __restrict__ hq) {
    // a subtree holds at most NT/64 leaves (block >= 64), so at most NT/128 subgroups split at
    // one sub-level
    constexpr int SG = NT / 128;
    __shared__ double stri[D * (D + 1) / 2];
    __shared__ double gvs[SG][D];
    __shared__ __attribute__((aligned(16))) float qpv[SG][D];
    __shared__ double spn[SG];
    __shared__ unsigned long long skey[SG];
    __shared__ int sown[SG], sarg[SG];
    __shared__ uint64_t tkey[NT];  // the sort's exchange of keys dk ...
    __shared__ uint32_t tval[NT];  // ... and of (subgroup << 16 | thread), members not splitting
                                   // last; then the sorted entries; then a member's rank in its
                                   // subgroup
    __shared__ int sstart[SG];
    __shared__ int lcnt[NT / 64][NT / 64];
    __shared__ int sany;  // some member splits at this sublevel (read from the second one on)
    __shared__ int s_claim;

    const int G = 1 << lev0;
    int staged = -1;  // the head whose Sigma triangle is in LDS
    for (int bh = (int)(blockIdx.x % BH); bh >= 0; bh = rb_next_head<NT>(hq, BH, G, bh, &s_claim)) {
        for (;;) {
            if (threadIdx.x == 0) s_claim = atomicAdd(&hq[bh], 1);
            __syncthreads();
            const int g = s_claim;
            __syncthreads();  // read by every thread before it is written again
            if (g >= G) break;
            int L0, c;
            rb_group(g, lev0, M, L0, c);
            if (c <= 0) continue;
            // the thread number, opaque to the compiler: what derives from it is computed per group
            // instead of being hoisted out of the loop and held in registers across it
            const int t = (int)(threadIdx.x + rb_opaque_zero());
            const int s0 = L0 * BLK, n = min(s0 + c * BLK, Nv) - s0;
            const bool act = t < n;
            const T* Qh = Q + (size_t)bh * N * D;
            const double* sigma = sigma_all + (size_t)bh * D * D;
            const int idx = act ? ord_in_all[(size_t)bh * Nv + s0 + t] : INT_MAX;
            RbRow<T, D> row;
            double ni = 0.0;
            if (act) {
                row.load(Qh + (size_t)idx * D);
                ni = nrm_all[(size_t)bh * Nv + idx];
            }
            if (c >= 2 && staged != bh) {
                staged = bh;
                // Sigma as pairs, four pairs per thread in flight at a time (once per head and
                // workgroup, so its registers matter more than its latency)
                constexpr int NP = D * D / 2 / NT, PF = 4;
#pragma unroll 1
                for (int h = 0; h < NP / PF; ++h) {
                    f64x2 v[PF];
                    const f64x2* s2 = reinterpret_cast<const f64x2*>(sigma) + rb_opaque_zero();
#pragma unroll
                    for (int k = 0; k < PF; ++k) v[k] = s2[t + (h * PF + k) * NT];
#pragma unroll
                    for (int k = 0; k < PF; ++k) {
                        const int e = 2 * (t + (h * PF + k) * NT), ra = e / D, cb = e % D;
                        if (cb >= ra) stri[rb_tri(ra, D) + cb - ra] = v[k][0];
                        if (cb + 1 >= ra) stri[rb_tri(ra, D) + cb + 1 - ra] = v[k][1];
                    }
                }
            }
            int sL0 = L0, sc = c, sid = 0;
            for (int k = 0; k < nsub; ++k) {
                const int ng = 1 << k;
                const bool split = act && sc >= 2;
                if (t < ng) sown[t] = INT_MAX;
                if (split) sany = 1;
                __syncthreads();
                // once every subgroup is a single leaf, no later sublevel splits either (subgroups only
                // shrink) and the leaves are final; the first sublevel splits when the group has two
                // leaves or more, and the flag is cleared at the end of each sublevel for the next
                if (k == 0 ? c < 2 : sany == 0) break;
                if (split) atomicMin(&sown[sid], t);
                __syncthreads();
                double cA = 0.0;
                uint64_t dk = 0;
                for (int step = 0; step < 3; ++step) {
                    // the pivot's thread publishes its row and norm; then g(P) of every splitting subgroup
                    if (split && sown[sid] == t) {
#pragma unroll
                        for (int q = 0; q < D / 8; ++q) {
                            float v[8];
                            row.p[q].widen(v);
                            *reinterpret_cast<f32x4*>(&qpv[sid][8 * q]) = f32x4{v[0], v[1], v[2], v[3]};
                            *reinterpret_cast<f32x4*>(&qpv[sid][8 * q + 4]) = f32x4{v[4], v[5], v[6], v[7]};
                        }
                        spn[sid] = ni;
                    }
                    __syncthreads();
                    for (int e = t; e < ng * D; e += NT) {
                        const int slot = e / D, a = e % D;
                        if (sown[slot] == INT_MAX) continue;
                        const double nP = spn[slot];
                        double gval = 0.0;
                        if (nP != 0.0) {
                            // Sigma_ab from the triangle: row min(a, b), column max(a, b).  Four values
                            // are read ahead of their four FMAs (same order), so the chain waits on one
                            // LDS round trip per four steps.
                            const int ta = rb_tri(a, D);
                            int tb = 0;
                            double acc = 0.0;
#pragma unroll 2
                            for (int b0 = 0; b0 < D; b0 += 4) {
                                double sv[4];
#pragma unroll
                                for (int j = 0; j < 4; ++j) {
                                    const int b = b0 + j;
                                    sv[j] = stri[b <= a ? tb + a - b : ta + b - a];
                                    tb += D - b;
                                }
#pragma unroll
                                for (int j = 0; j < 4; ++j) acc = fma(sv[j], (double)qpv[slot][b0 + j], acc);
                            }
                            gval = acc / nP;
                        }
                        gvs[slot][a] = gval;
                    }
                    if (t < ng) {
                        skey[t] = ~0ull;
                        sarg[t] = INT_MAX;
                    }
                    __syncthreads();
                    double cs = 0.0;
                    if (split) {
#pragma unroll
                        for (int q = 0; q < D / 8; ++q) rb_launder(row.p[q]);
                        const double acc = rb_dot<T, D>(row, &gvs[sid][0]);
                        cs = ni == 0.0 ? 0.0 : acc / ni;
                    }
                    if (step < 2) {
                        const uint64_t kk = asc_key(cs);
                        if (split) atomicMin(&skey[sid], (unsigned long long)kk);
                        __syncthreads();
                        if (split && kk == skey[sid]) atomicMin(&sarg[sid], t);
                        __syncthreads();
                        if (step == 1) cA = cs;
                        if (t < ng) sown[t] = sarg[t];
                        __syncthreads();
                    } else {
                        dk = ~asc_key(cA - cs);
                    }
                }
                {
                    uint64_t key = dk;
                    uint32_t val = ((split ? (uint32_t)sid : 0xffffu) << 16) | (uint32_t)t;
                    rb_bitonic_sort<NT>(key, val, tkey, tval);  // ascending (subgroup, dk, thread)
                    tval[t] = val;
                    __syncthreads();
                }
                {
                    const uint32_t v = tval[t], grp = v >> 16;
                    if (grp != 0xffffu && (t == 0 || (tval[t - 1] >> 16) != grp)) sstart[grp] = t;
                    __syncthreads();  // every sorted entry has been read: tval now takes the ranks
                    if (grp != 0xffffu) tval[v & 0xffffu] = (uint32_t)(t - sstart[grp]);
                    __syncthreads();
                }
                if (split) {
                    const int rank = (int)tval[t];
                    const int cl = (sc + 1) / 2;
                    if (rank < cl * BLK) {
                        sc = cl;
                        sid = 2 * sid;
                    } else {
                        sL0 += cl;
                        sc -= cl;
                        sid = 2 * sid + 1;
                    }
                } else {
                    sid = 2 * sid;
                }
                if (t == 0) sany = 0;  // every thread read it many barriers ago
                __syncthreads();
            }
            // position inside the leaf: members of the leaf in lower waves, then lower lanes of this wave
            const int lane = t & 63, w = t >> 6, lj = sL0 - L0;
            uint64_t mine = 0;
            for (int j = 0; j < c; ++j) {
                const uint64_t m = __ballot(act && lj == j);
                if (lane == 0) lcnt[j][w] = __popcll(m);
                if (lj == j) mine = m;
            }
            __syncthreads();
            if (act) {
                int r = __popcll(mine & (lane == 0 ? 0ull : (~0ull >> (64 - lane))));
                for (int v = 0; v < w; ++v) r += lcnt[lj][v];
                perm_all[(size_t)bh * Nv + (size_t)sL0 * BLK + r] = idx;
            }
            __syncthreads();  // this group's LDS is free for the next one
        }
    }
}

__global__ __launch_bounds__(256) void rb_iota_kernel(int32_t* __restrict__ ord, int Nv) {
    const int bh = blockIdx.y;
    for (int i = blockIdx.x * 256 + threadIdx.x; i < Nv; i += gridDim.x * 256) ord[(size_t)bh * Nv + i] = i;
}

template <typename T, int D>
static void launch_reblock_t(const LaunchCtx& L, const void* Q, const void* K, int32_t* perm, void* ws) {
    const RbLayout lay = rb_layout(L);
    char* w = (char*)ws;
    uint32_t* kmax = (uint32_t*)(w + lay.kmax);
    long long* sint = (long long*)(w + lay.sint);
    double* sigma = (double*)(w + lay.sigma);
    double* nrm = (double*)(w + lay.nrm);
    // zero max|k|, the integer sums and the group counters (one contiguous span at the start)
    const size_t zero_words = (lay.sigma - lay.kmax) / 8;
    hipLaunchKernelGGL(rb_zero_kernel, dim3(256), dim3(256), 0, L.stream, (uint64_t*)(w + lay.kmax), zero_words);
    hipLaunchKernelGGL((rb_kmax_kernel<T>), dim3(128, L.BH), dim3(256), 0, L.stream, (const T*)K, L.N, L.Nv, D, kmax);
    hipLaunchKernelGGL((rb_sigma_kernel<T, D>), dim3((L.Nv + kRbSigRows - 1) / kRbSigRows, L.BH),
                       dim3(RbSig<D>::NT), 0, L.stream, (const T*)K, L.N, L.Nv, kmax, sint);
    hipLaunchKernelGGL(rb_sigma_finalize_kernel, dim3((D * D + 255) / 256, L.BH), dim3(256), 0, L.stream, sint, kmax,
                       D, L.Nv, sigma);
    {
        // as many workgroups as stay resident at once (one per CU at d = 128: Sigma fills the LDS),
        // each an even share of the (head, 16-row block) items
        const auto kern = rb_norms_kernel<T, D>;
        const long long items = (long long)L.BH * ((L.Nv + 15) / 16);
        int dev = 0, ncu = 0, per_cu = 0;
        long long resident = 256;  // used only if the queries fail
        if (hipGetDevice(&dev) == hipSuccess &&
            hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess &&
            hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kern, 64 * kRbNrmWaves, 0) == hipSuccess &&
            ncu > 0 && per_cu > 0)
            resident = (long long)ncu * per_cu;
        const int grid = (int)std::min(items, resident);
        hipLaunchKernelGGL(kern, dim3(grid), dim3(64 * kRbNrmWaves), 0, L.stream, (const T*)Q, L.N, L.Nv, L.BH, sigma,
                           nrm);
    }
    int32_t* ord[2] = {(int32_t*)(w + lay.ord0), (int32_t*)(w + lay.ord1)};
    double* cbuf = (double*)(w + lay.cbuf);
    uint64_t* dk = (uint64_t*)(w + lay.dk);
    double* c0 = (double*)(w + lay.c0);
    double* gbuf = (double*)(w + lay.gbuf);
    uint64_t* pkey = (uint64_t*)(w + lay.pkey);
    int* pidx = (int*)(w + lay.pidx);
    const T* Qt = (const T*)Q;
    hipLaunchKernelGGL(rb_iota_kernel, dim3((L.Nv + 255) / 256, L.BH), dim3(256), 0, L.stream, L.M > 1 ? ord[0] : perm,
                       L.Nv);
    const int levels = rb_levels(L.M);
    // the first level whose groups fit the subtree kernel runs it to the end (the last level's
    // groups hold at most 2 leaves, so there always is one)
    int ls = levels;
    for (int lev = 0; lev < levels; ++lev)
        if ((((long long)L.M + (1ll << lev) - 1) >> lev) * L.block <= kRbSubThreads) {
            ls = lev;
            break;
        }
    for (int lev = 0; lev < ls; ++lev) {
        const int32_t* src = ord[lev & 1];
        int32_t* dst = ord[(lev + 1) & 1];
        const unsigned G = 1u << lev;
        const int nch = rb_chunks(L, lev);
        if (nch < 2) {
            hipLaunchKernelGGL((rb_level_kernel<T, D, 256>), dim3(G, L.BH), dim3(256), 0, L.stream, Qt, L.N, L.Nv,
                               L.block, L.M, lev, sigma, nrm, src, dst, cbuf, dk);
            continue;
        }
        const dim3 gp(G, L.BH), gc(G * nch, L.BH);
        hipLaunchKernelGGL((rb_chunk_pivot_kernel<T, D>), gp, dim3(D), 0, L.stream, Qt, L.N, L.Nv, L.block, L.M, lev,
                           nch, sigma, nrm, src, pkey, pidx, gbuf, 1);
        hipLaunchKernelGGL((rb_chunk_cos_kernel<T, D, 0>), gc, dim3(kRbChunkThreads), 0, L.stream, Qt, L.N, L.Nv,
                           L.block, L.M, lev, nch, nrm, src, gbuf, cbuf, dk, pkey, pidx, c0);
        hipLaunchKernelGGL((rb_chunk_pivot_kernel<T, D>), gp, dim3(D), 0, L.stream, Qt, L.N, L.Nv, L.block, L.M, lev,
                           nch, sigma, nrm, src, pkey, pidx, gbuf, 0);
        hipLaunchKernelGGL((rb_chunk_cos_kernel<T, D, 1>), gc, dim3(kRbChunkThreads), 0, L.stream, Qt, L.N, L.Nv,
                           L.block, L.M, lev, nch, nrm, src, gbuf, cbuf, dk, pkey, pidx, nullptr);
        hipLaunchKernelGGL((rb_chunk_pivot_kernel<T, D>), gp, dim3(D), 0, L.stream, Qt, L.N, L.Nv, L.block, L.M, lev,
                           nch, sigma, nrm, src, pkey, pidx, gbuf, 0);
        hipLaunchKernelGGL((rb_chunk_cos_kernel<T, D, 2>), gc, dim3(kRbChunkThreads), 0, L.stream, Qt, L.N, L.Nv,
                           L.block, L.M, lev, nch, nrm, src, gbuf, cbuf, dk, pkey, pidx, nullptr);
        hipLaunchKernelGGL((rb_chunk_split_kernel<1024>), gp, dim3(1024), 0, L.stream, L.Nv, L.block, L.M, lev, src,
                           dst, dk);
    }
    if (ls < levels) {
        // as many workgroups as stay resident at once; they claim the (head, group) items
        const auto kern = rb_subtree_kernel<T, D, kRbSubThreads>;
        const long long items = (1ll << ls) * L.BH;
        int dev = 0, ncu = 0, per_cu = 0;
        long long resident = 1024;  // used only if the queries fail
        if (hipGetDevice(&dev) == hipSuccess &&
            hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess &&
            hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kern, kRbSubThreads, 0) == hipSuccess &&
            ncu > 0 && per_cu > 0)
            resident = (long long)ncu * per_cu;
        const int grid = (int)std::min(items, resident);
        hipLaunchKernelGGL(kern, dim3(grid), dim3(kRbSubThreads), 0, L.stream, Qt, L.N, L.Nv, L.block, L.M, ls,
                           levels - ls, L.BH, sigma, nrm, ord[ls & 1], perm, (int32_t*)(w + lay.subq));
    }
}

void launch_reblock(const LaunchCtx& L, const void* Q, const void* K, int32_t* perm, void* ws) {
    if (L.dtype == SPARK_ATTN_BF16) {
        if (L.d == 64) launch_reblock_t<__bf16, 64>(L, Q, K, perm, ws);
        else launch_reblock_t<__bf16, 128>(L, Q, K, perm, ws);
    } else {
        if (L.d == 64) launch_reblock_t<float, 64>(L, Q, K, perm, ws);
        else launch_reblock_t<float, 128>(L, Q, K, perm, ws);
    }
}

}  // namespace spark
