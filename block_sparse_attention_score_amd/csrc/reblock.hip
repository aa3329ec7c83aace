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
//            sums of k^_a k^_b (binary64 partial sums over 2048 rows are exact), scaled back;
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

#include "kernels.hpp"

#pragma clang fp contract(off)

namespace spark {

typedef double f64x2 __attribute__((ext_vector_type(2)));
typedef uint64_t u64x2 __attribute__((ext_vector_type(2)));

constexpr int kRbSigmaRows = 2048;  // rows per exact binary64 partial sum (2^42 * 2^11 = 2^53)
constexpr int kRbMaxRows = 1 << 20; // int64 sums of <= 2^20 products of magnitude <= 2^42
constexpr int kRbChunk = 2048;      // order positions per workgroup of a chunked cos pass
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
    size_t kmax, sint, sigma, nrm, ord0, ord1, cbuf, dk, gbuf, pkey, pidx, total;
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
    r.sigma = take(BH * d * d * 8);
    r.nrm = take(BH * Nv * 8);
    r.ord0 = take(BH * Nv * 4);
    r.ord1 = take(BH * Nv * 4);
    r.cbuf = take(BH * Nv * 8);
    r.dk = take(BH * Nv * 8);
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
    for (size_t e = (size_t)blockIdx.x * 256 + threadIdx.x; e < n8; e += (size_t)gridDim.x * 256) {
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

// Tiles of Sigma on or above the diagonal: TB*(TB+1)/2 of 4x4, one per thread.
template <int D>
struct RbSigmaTiles {
    static constexpr int TB = D / 4;
    static constexpr int NTILE = TB * (TB + 1) / 2;
    static constexpr int NTH = (NTILE + 63) / 64 * 64;
};

// Exact fixed-point K^T K: workgroup (bh, row chunk of 2048 rows), one thread per 4x4 tile of
// Sigma on or above the diagonal.  Rows are staged 64 at a time as k^ = rint(k 2^s) (exact in
// fp32, |k^| <= 2^21); products and the chunk's partial sums are exact in binary64.
template <typename T, int D>
__global__ __launch_bounds__(RbSigmaTiles<D>::NTH) void rb_sigma_kernel(const T* __restrict__ K, int N, int Nv,
                                                                       const uint32_t* __restrict__ kmax,
                                                                       long long* __restrict__ sint) {
    constexpr int TB = RbSigmaTiles<D>::TB, NTILE = RbSigmaTiles<D>::NTILE, NTH = RbSigmaTiles<D>::NTH;
    __shared__ __attribute__((aligned(16))) float ks[64][D];
    const int bh = blockIdx.y;
    const int r0 = blockIdx.x * kRbSigmaRows, r1 = min(Nv, r0 + kRbSigmaRows);
    const int sh = fixed_point_shift(kmax[bh]);
    // tile p -> (ta, tc), ta <= tc, rows of the upper triangle one after another
    const int p = threadIdx.x;
    const bool live = p < NTILE;
    int ta = 0, tc = 0;
    {
        int rest = live ? p : 0;
        while (rest >= TB - ta) {
            rest -= TB - ta;
            ++ta;
        }
        tc = ta + rest;
    }
    double acc[4][4] = {};
    const T* kh = K + (size_t)bh * N * D;
    // the next 64 rows are in flight in registers while the current 64 are multiplied
    constexpr int NC = (64 * D / 8 + NTH - 1) / NTH;  // eight-element chunks per thread and batch
    Raw8<T> nxt[NC];
    auto fetch = [&](int rs) __attribute__((always_inline)) {
#pragma unroll
        for (int u = 0; u < NC; ++u) {
            const int e = threadIdx.x + u * NTH, r = rs + e / (D / 8);
            if (e < 64 * D / 8 && r < r1) nxt[u].load(kh + (size_t)r * D + (e % (D / 8)) * 8);
        }
    };
    fetch(r0);
    for (int rs = r0; rs < r1; rs += 64) {
        __syncthreads();
#pragma unroll
        for (int u = 0; u < NC; ++u) {
            const int e = threadIdx.x + u * NTH;
            if (e >= 64 * D / 8) continue;
            const int r = rs + e / (D / 8), c8 = (e % (D / 8)) * 8;
            float v[8] = {};
            if (r < r1) nxt[u].widen(v);
#pragma unroll
            for (int j = 0; j < 8; ++j) v[j] = (float)rint(ldexp((double)v[j], sh));
            *reinterpret_cast<f32x4*>(&ks[e / (D / 8)][c8]) = f32x4{v[0], v[1], v[2], v[3]};
            *reinterpret_cast<f32x4*>(&ks[e / (D / 8)][c8 + 4]) = f32x4{v[4], v[5], v[6], v[7]};
        }
        __syncthreads();
        if (rs + 64 < r1) fetch(rs + 64);
        if (live) {
            for (int r = 0; r < 64; ++r) {
                const f32x4 a = *reinterpret_cast<const f32x4*>(&ks[r][ta * 4]);
                const f32x4 c = *reinterpret_cast<const f32x4*>(&ks[r][tc * 4]);
#pragma unroll
                for (int i = 0; i < 4; ++i)
#pragma unroll
                    for (int j = 0; j < 4; ++j) acc[i][j] = fma((double)a[i], (double)c[j], acc[i][j]);
            }
        }
    }
    if (live) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j)
                atomicAdd((unsigned long long*)&sint[((size_t)bh * D + ta * 4 + i) * D + tc * 4 + j],
                          (unsigned long long)(long long)acc[i][j]);
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

// n_i for every video query: TPL tokens per thread; t in chunks of QC accumulators, each t_a
// still one chain over b = 0..D-1.  The workgroup stages the chunk's columns of Sigma in LDS
// (Sigma_ab read as Sigma[b][a]); every value read there feeds the TPL tokens of a thread, and
// each token's next row elements are in flight while the current eight b steps run.  Then r over
// a in ascending order across the chunks.
constexpr int kRbNormQC = 32;
constexpr int kRbNormTPL = 2;
constexpr int kRbNormAhead = 3;  // row chunks of eight elements in flight per token

template <typename T, int D>
__global__ __launch_bounds__(256) void rb_norms_kernel(const T* __restrict__ Q, int N, int Nv,
                                                       const double* __restrict__ sigma, double* __restrict__ nrm) {
    constexpr int QC = kRbNormQC, TPL = kRbNormTPL, PD = kRbNormAhead, NK = D / 8;
    __shared__ __attribute__((aligned(16))) double sl[D * QC];
    const int bh = blockIdx.y, i0 = blockIdx.x * 256 * TPL + threadIdx.x;
    const T* q[TPL];
#pragma unroll
    for (int u = 0; u < TPL; ++u) q[u] = Q + ((size_t)bh * N + min(i0 + 256 * u, Nv - 1)) * D;
    const double* S = sigma + (size_t)bh * D * D;
    double r[TPL];
#pragma unroll
    for (int u = 0; u < TPL; ++u) r[u] = 0.0;
#pragma unroll 1
    for (int h0 = 0; h0 < D; h0 += QC) {
        __syncthreads();
        for (int e2 = threadIdx.x; e2 < D * QC / 2; e2 += 256) {
            const int b = e2 / (QC / 2), a2 = e2 % (QC / 2);
            *reinterpret_cast<f64x2*>(&sl[b * QC + 2 * a2]) =
                *reinterpret_cast<const f64x2*>(&S[(size_t)b * D + h0 + 2 * a2]);
        }
        __syncthreads();
        double t[TPL][QC];
#pragma unroll
        for (int u = 0; u < TPL; ++u)
#pragma unroll
            for (int a = 0; a < QC; ++a) t[u][a] = 0.0;
        Raw8<T> ring[TPL][PD];
#pragma unroll
        for (int u = 0; u < TPL; ++u)
#pragma unroll
            for (int j = 0; j < PD; ++j) ring[u][j].load(q[u] + 8 * j);
#pragma unroll 1
        for (int k = 0; k < NK; ++k) {
            float v[TPL][8];
#pragma unroll
            for (int u = 0; u < TPL; ++u) {
                ring[u][0].widen(v[u]);
#pragma unroll
                for (int j = 0; j + 1 < PD; ++j) ring[u][j] = ring[u][j + 1];
                if (k + PD < NK) ring[u][PD - 1].load(q[u] + 8 * (k + PD));
            }
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const double* Sb = sl + (8 * k + e) * QC;
#pragma unroll
                for (int a = 0; a < QC; ++a) {
                    const double sab = Sb[a];
#pragma unroll
                    for (int u = 0; u < TPL; ++u) t[u][a] = fma(sab, (double)v[u][e], t[u][a]);
                }
            }
        }
#pragma unroll
        for (int u = 0; u < TPL; ++u) {
            Raw8<T> qa[QC / 8];
#pragma unroll
            for (int k = 0; k < QC / 8; ++k) qa[k].load(q[u] + h0 + 8 * k);
#pragma unroll
            for (int k = 0; k < QC / 8; ++k) {
                float v[8];
                qa[k].widen(v);
#pragma unroll
                for (int e = 0; e < 8; ++e) r[u] = fma((double)v[e], t[u][8 * k + e], r[u]);
            }
        }
    }
#pragma unroll
    for (int u = 0; u < TPL; ++u) {
        const int i = i0 + 256 * u;
        if (i < Nv) nrm[(size_t)bh * Nv + i] = r[u] > 0.0 ? sqrt(r[u]) : 0.0;
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
// jb + tid, jb + tid + NT, ... below je of an order segment; f(j, i, cos) sees each one.  The next
// position's row and norm are in flight while the current dot product runs, and the order entry
// after that one is loaded a step earlier still.
template <typename T, int D, int NT, typename F>
__device__ __forceinline__ void rb_cos_range(const T* __restrict__ Qh, const double* __restrict__ nrm,
                                             const int32_t* __restrict__ seg, int jb, int je, const double* gv,
                                             F&& f) {
    int j = jb + (int)threadIdx.x;
    if (j >= je) return;
    int i = seg[j];
    int i1 = j + NT < je ? seg[j + NT] : 0;
    RbRow<T, D> r;
    r.load(Qh + (size_t)i * D);
    double ni = nrm[i];
    for (;;) {
        const int jn = j + NT;
        const bool more = jn < je;
        RbRow<T, D> rn;
        double nn = 0.0;
        if (more) {
            rn.load(Qh + (size_t)i1 * D);
            nn = nrm[i1];
        }
        const int i2 = jn + NT < je ? seg[jn + NT] : 0;
        const double acc = rb_dot<T, D>(r, gv + rb_opaque_zero());
        f(j, i, ni == 0.0 ? 0.0 : acc / ni);
        if (!more) break;
        j = jn;
        i = i1;
        i1 = i2;
        r = rn;
        ni = nn;
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
    int sel_digit, sel_rem;
};

// Split a group of n order entries with keys dk (order (dk, index) ascending = (cos(., A) -
// cos(., B)) descending, index ascending): a radix select finds the nl-th smallest (dk, index)
// (8 digits of dk, then 3 of the index, which is below 2^24); a stable partition writes the nl
// smallest, in their current order, to out[0 .. nl) and the rest to out[nl .. n).
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
                unsigned cum = before;
                int dsel = 4 * lane + 3;
                for (int q = 0; q < 4; ++q) {
                    if ((int)(cum + cnt[q]) >= rem) {
                        dsel = 4 * lane + q;
                        break;
                    }
                    cum += cnt[q];
                }
                sh.sel_digit = dsel;
                sh.sel_rem = rem - (int)cum;
            }
        }
        __syncthreads();
        const unsigned dsel = (unsigned)sh.sel_digit;
        rem = sh.sel_rem;
        if (pass < 8) pre_hi = (pre_hi << 8) | dsel;
        else pre_lo = (pre_lo << 8) | dsel;
        __syncthreads();
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

    rb_pivot<T, D, NT>(sigma, nrm, Qh, seg[0], gv);
    __syncthreads();
    // A = argmin cos(., P0), ties to the lower index
    uint64_t kmin = ~0ull;
    int A = INT_MAX;
    rb_cos_range<T, D, NT>(Qh, nrm, seg, 0, n, gv, [&](int, int i, double cs) {
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
    rb_cos_range<T, D, NT>(Qh, nrm, seg, 0, n, gv, [&](int j, int i, double cs) {
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
    rb_cos_range<T, D, NT>(Qh, nrm, seg, 0, n, gv,
                           [&](int j, int, double cs) { dk[j] = ~asc_key(cb[j] - cs); });
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
    const int s0 = L0 * BLK, n = min(s0 + c * BLK, Nv) - s0;
    int P;
    if (first) {
        P = ord_in_all[(size_t)bh * Nv + s0];
    } else {
        const size_t base = ((size_t)bh * G + g) * nch;
        const int nc = (n + kRbChunk - 1) / kRbChunk;
        uint64_t k = ~0ull;
        P = INT_MAX;
        for (int ch = threadIdx.x; ch < nc; ch += D) {
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
template <typename T, int D, int MODE>
__global__ __launch_bounds__(kRbChunkThreads) void rb_chunk_cos_kernel(
    const T* __restrict__ Q, int N, int Nv, int BLK, int M, int lev, int nch, const double* __restrict__ nrm_all,
    const int32_t* __restrict__ ord_in_all, const double* __restrict__ gbuf, double* __restrict__ cbuf_all,
    uint64_t* __restrict__ dk_all, uint64_t* __restrict__ pkey, int* __restrict__ pidx) {
    constexpr int NT = kRbChunkThreads;
    __shared__ double gv[D];
    __shared__ uint64_t skey[NT / 64];
    __shared__ int sidx[NT / 64];
    const int bh = blockIdx.y, g = blockIdx.x / nch, ch = blockIdx.x % nch, G = gridDim.x / nch;
    int L0, c;
    rb_group(g, lev, M, L0, c);
    if (c <= 1) return;
    const int s0 = L0 * BLK, n = min(s0 + c * BLK, Nv) - s0;
    const int jb = ch * kRbChunk;
    if (jb >= n) return;
    const int je = min(n, jb + kRbChunk);
    const double* gsrc = gbuf + ((size_t)bh * G + g) * D;
    for (int a = threadIdx.x; a < D; a += NT) gv[a] = gsrc[a];
    __syncthreads();
    const T* Qh = Q + (size_t)bh * N * D;
    const double* nrm = nrm_all + (size_t)bh * Nv;
    const int32_t* seg = ord_in_all + (size_t)bh * Nv + s0;
    double* cb = cbuf_all + (size_t)bh * Nv + s0;
    uint64_t* dk = dk_all + (size_t)bh * Nv + s0;
    if (MODE == 2) {
        rb_cos_range<T, D, NT>(Qh, nrm, seg, jb, je, gv,
                               [&](int j, int, double cs) { dk[j] = ~asc_key(cb[j] - cs); });
        return;
    }
    uint64_t kmin = ~0ull;
    int P = INT_MAX;
    rb_cos_range<T, D, NT>(Qh, nrm, seg, jb, je, gv, [&](int j, int i, double cs) {
        if (MODE == 1) cb[j] = cs;
        const uint64_t k = asc_key(cs);
        if (rb_before(k, i, kmin, P)) {
            kmin = k;
            P = i;
        }
    });
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
// exactly the membership the radix select and stable partition give.  At the end a token's
// position is its leaf's start plus the number of members of the same leaf with a lower index.
// Members are in ascending index with the thread number, so thread numbers stand in for indexes
// in every tie-break.  Workgroups are laid out so that each XCD (every eighth workgroup id) takes
// a contiguous range of (head, group) and so reads only a few heads' data.
constexpr int kRbSubThreads = 512;  // largest subtree: threads = tokens

__host__ __device__ constexpr int rb_tri(int a, int D) { return a * (2 * D - a + 1) / 2; }

template <typename T, int D, int NT>
__global__ __launch_bounds__(NT) void rb_subtree_kernel(const T* __restrict__ Q, int N, int Nv, int BLK,
                                                                   int M, int lev0, int nsub, int BH,
                                                                   const double* __restrict__ sigma_all,
                                                                   const double* __restrict__ nrm_all,
                                                                   const int32_t* __restrict__ ord_in_all,
                                                                   int32_t* __restrict__ perm_all) {
    // a subtree holds at most NT/64 leaves (block >= 64), so at most NT/128 subgroups split at
    // one sub-level
    constexpr int SG = NT / 128;
    __shared__ double stri[D * (D + 1) / 2];
    __shared__ double gvs[SG][D];
    __shared__ __attribute__((aligned(16))) float qpv[SG][D];
    __shared__ double spn[SG];
    __shared__ unsigned long long skey[SG];
    __shared__ int sown[SG], sarg[SG];
    __shared__ __attribute__((aligned(16))) uint64_t tkey[NT];
    __shared__ __attribute__((aligned(8))) signed char tgrp[NT];
    __shared__ int lcnt[NT / 64][NT / 64];

    const int G = 1 << lev0, total = G * BH, per = (total + 7) / 8;
    const int wi = (int)(blockIdx.x % 8) * per + (int)(blockIdx.x / 8);
    if (wi >= total) return;
    const int bh = wi / G, g = wi % G, t = threadIdx.x;
    int L0, c;
    rb_group(g, lev0, M, L0, c);
    if (c <= 0) return;
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
    if (c >= 2) {
        // Sigma as pairs, eight pairs per thread in flight at a time
        constexpr int NP = D * D / 2 / NT, HALF = NP / 2;
        const f64x2* s2 = reinterpret_cast<const f64x2*>(sigma);
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            f64x2 v[HALF];
#pragma unroll
            for (int k = 0; k < HALF; ++k) v[k] = s2[t + (h * HALF + k) * NT];
#pragma unroll
            for (int k = 0; k < HALF; ++k) {
                const int e = 2 * (t + (h * HALF + k) * NT), ra = e / D, cb = e % D;
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
        __syncthreads();
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
                    // Sigma_ab from the triangle: row min(a, b), column max(a, b)
                    const int ta = rb_tri(a, D);
                    int tb = 0;
                    double acc = 0.0;
#pragma unroll 8
                    for (int b = 0; b < D; ++b) {
                        const int off = b <= a ? tb + a - b : ta + b - a;
                        acc = fma(stri[off], (double)qpv[slot][b], acc);
                        tb += D - b;
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
        tkey[t] = dk;
        tgrp[t] = split ? (signed char)sid : (signed char)-1;
        __syncthreads();
        if (split) {
            // entries past n carry subgroup -1; eight entries per step
            int rank = 0;
            for (int u0 = 0; u0 < n; u0 += 8) {
                const uint64_t gg = *reinterpret_cast<const uint64_t*>(&tgrp[u0]);
                u64x2 kk[4];
#pragma unroll
                for (int q = 0; q < 4; ++q) kk[q] = *reinterpret_cast<const u64x2*>(&tkey[u0 + 2 * q]);
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const uint64_t k2 = kk[j / 2][j % 2];
                    const int gj = (int)(signed char)(gg >> (8 * j));
                    rank += gj == sid && (k2 < dk || (k2 == dk && u0 + j < t));
                }
            }
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
    // zero max|k| and the integer sums (one contiguous span at the start of the layout)
    const size_t zero_words = (lay.sigma - lay.kmax) / 8;
    hipLaunchKernelGGL(rb_zero_kernel, dim3(256), dim3(256), 0, L.stream, (uint64_t*)(w + lay.kmax), zero_words);
    hipLaunchKernelGGL((rb_kmax_kernel<T>), dim3(128, L.BH), dim3(256), 0, L.stream, (const T*)K, L.N, L.Nv, D, kmax);
    hipLaunchKernelGGL((rb_sigma_kernel<T, D>), dim3((L.Nv + kRbSigmaRows - 1) / kRbSigmaRows, L.BH),
                       dim3(RbSigmaTiles<D>::NTH), 0, L.stream, (const T*)K, L.N, L.Nv, kmax, sint);
    hipLaunchKernelGGL(rb_sigma_finalize_kernel, dim3((D * D + 255) / 256, L.BH), dim3(256), 0, L.stream, sint, kmax,
                       D, L.Nv, sigma);
    hipLaunchKernelGGL((rb_norms_kernel<T, D>), dim3((L.Nv + 256 * kRbNormTPL - 1) / (256 * kRbNormTPL), L.BH),
                       dim3(256), 0, L.stream, (const T*)Q,
                       L.N, L.Nv, sigma, nrm);
    int32_t* ord[2] = {(int32_t*)(w + lay.ord0), (int32_t*)(w + lay.ord1)};
    double* cbuf = (double*)(w + lay.cbuf);
    uint64_t* dk = (uint64_t*)(w + lay.dk);
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
                           L.block, L.M, lev, nch, nrm, src, gbuf, cbuf, dk, pkey, pidx);
        hipLaunchKernelGGL((rb_chunk_pivot_kernel<T, D>), gp, dim3(D), 0, L.stream, Qt, L.N, L.Nv, L.block, L.M, lev,
                           nch, sigma, nrm, src, pkey, pidx, gbuf, 0);
        hipLaunchKernelGGL((rb_chunk_cos_kernel<T, D, 1>), gc, dim3(kRbChunkThreads), 0, L.stream, Qt, L.N, L.Nv,
                           L.block, L.M, lev, nch, nrm, src, gbuf, cbuf, dk, pkey, pidx);
        hipLaunchKernelGGL((rb_chunk_pivot_kernel<T, D>), gp, dim3(D), 0, L.stream, Qt, L.N, L.Nv, L.block, L.M, lev,
                           nch, sigma, nrm, src, pkey, pidx, gbuf, 0);
        hipLaunchKernelGGL((rb_chunk_cos_kernel<T, D, 2>), gc, dim3(kRbChunkThreads), 0, L.stream, Qt, L.N, L.Nv,
                           L.block, L.M, lev, nch, nrm, src, gbuf, cbuf, dk, pkey, pidx);
        hipLaunchKernelGGL((rb_chunk_split_kernel<1024>), gp, dim3(1024), 0, L.stream, L.Nv, L.block, L.M, lev, src,
                           dst, dk);
    }
    if (ls < levels) {
        const int total = (1 << ls) * L.BH;
        hipLaunchKernelGGL((rb_subtree_kernel<T, D, kRbSubThreads>), dim3(8 * ((total + 7) / 8)), dim3(kRbSubThreads), 0,
                           L.stream, Qt, L.N, L.Nv, L.block, L.M, ls, levels - ls, L.BH, sigma, nrm, ord[ls & 1], perm);
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
