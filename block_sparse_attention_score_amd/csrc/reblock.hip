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
// Argmins use integer atomicMin on order-preserving keys and the balanced split is a radix select
// on (key, index), so nothing depends on thread timing.
//
// Kernels: max|k| and the fixed-point Sigma and the norms are wide (all CUs); the level loop runs
// in one persistent 1024-thread workgroup per (batch, head), with barriers between phases.
#include <limits.h>

#include "kernels.hpp"

#pragma clang fp contract(off)

namespace spark {

constexpr int kRbThreads = 1024;
constexpr int kRbSigmaRows = 2048;  // rows per exact binary64 partial sum (2^42 * 2^11 = 2^53)
constexpr int kRbMaxRows = 1 << 20; // int64 sums of <= 2^20 products of magnitude <= 2^42

struct RbLayout {
    size_t kmax, sint, sigma, nrm, grp, cbuf, dk, gstart, gc, gcnt, gp0, ga, gb, grem, gmin, gpre_hi, gpre_lo,
        gvec, hist, total;
};

static RbLayout rb_layout(const LaunchCtx& L) {
    RbLayout r;
    const size_t BH = L.BH, Nv = L.Nv, M = L.M, d = L.d;
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
    r.grp = take(BH * Nv * 4);
    r.cbuf = take(BH * Nv * 8);
    r.dk = take(BH * Nv * 8);
    r.gstart = take(BH * M * 4);
    r.gc = take(BH * M * 4);
    r.gcnt = take(BH * M * 4);
    r.gp0 = take(BH * M * 4);
    r.ga = take(BH * M * 4);
    r.gb = take(BH * M * 4);
    r.grem = take(BH * M * 4);
    r.gmin = take(BH * M * 8);
    r.gpre_hi = take(BH * M * 8);
    r.gpre_lo = take(BH * M * 8);
    r.gvec = take(BH * M * d * 8);
    r.hist = take(BH * M * 256 * 4);
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

template <typename U> __device__ __forceinline__ U aload(const U* p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__global__ __launch_bounds__(256) void rb_zero_kernel(uint64_t* __restrict__ p, size_t n) {
    for (size_t e = (size_t)blockIdx.x * 256 + threadIdx.x; e < n; e += (size_t)gridDim.x * 256) p[e] = 0;
}

// max |k| over the video keys of each (batch, head), as float bits (non-negative floats order as
// unsigned integers).
template <typename T>
__global__ __launch_bounds__(256) void rb_kmax_kernel(const T* __restrict__ K, int N, int Nv, int d,
                                                      uint32_t* __restrict__ kmax) {
    const int bh = blockIdx.y;
    const T* kh = K + (size_t)bh * N * d;
    const size_t n = (size_t)Nv * d;
    float m = 0.f;
    for (size_t e = (size_t)blockIdx.x * 256 + threadIdx.x; e < n; e += (size_t)gridDim.x * 256)
        m = fmaxf(m, fabsf(elem_f<T>(kh + e)));
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
    if ((threadIdx.x & 63) == 0) atomicMax(&kmax[bh], __float_as_uint(m));
}

__device__ __forceinline__ int fixed_point_shift(uint32_t kmax_bits) {
    int E = 0;
    (void)frexp((double)__uint_as_float(kmax_bits), &E);
    return 21 - E;
}

// Exact fixed-point K^T K: workgroup (bh, row chunk of 2048 rows), one thread per 4x4 tile of
// Sigma on or above the diagonal.  Rows are staged 64 at a time as k^ = rint(k 2^s) (exact in
// fp32, |k^| <= 2^21); products and the chunk's partial sums are exact in binary64.
template <typename T, int D>
__global__ __launch_bounds__(D * D / 16) void rb_sigma_kernel(const T* __restrict__ K, int N, int Nv,
                                                              const uint32_t* __restrict__ kmax,
                                                              long long* __restrict__ sint) {
    constexpr int NTH = D * D / 16, TB = D / 4;  // threads, 4x4 tiles per side
    __shared__ __attribute__((aligned(16))) float ks[64][D];
    const int bh = blockIdx.y;
    const int r0 = blockIdx.x * kRbSigmaRows, r1 = min(Nv, r0 + kRbSigmaRows);
    const int sh = fixed_point_shift(kmax[bh]);
    const int ta = threadIdx.x / TB, tc = threadIdx.x % TB;
    const bool live = ta <= tc;
    double acc[4][4] = {};
    const T* kh = K + (size_t)bh * N * D;
    for (int rs = r0; rs < r1; rs += 64) {
        __syncthreads();
        for (int e = threadIdx.x; e < 64 * D; e += NTH) {
            const int r = rs + e / D;
            float v = 0.f;
            if (r < r1) v = (float)rint(ldexp((double)elem_f<T>(kh + (size_t)r * D + e % D), sh));
            ks[e / D][e % D] = v;
        }
        __syncthreads();
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

// n_i for every video query: one thread per token, t in two halves of D/2 accumulators (each
// t_a is still one chain over b = 0..D-1), then r over a in ascending order.
template <typename T, int D>
__global__ __launch_bounds__(256) void rb_norms_kernel(const T* __restrict__ Q, int N, int Nv,
                                                       const double* __restrict__ sigma, double* __restrict__ nrm) {
    const int bh = blockIdx.y, i = blockIdx.x * 256 + threadIdx.x;
    if (i >= Nv) return;
    const T* q = Q + ((size_t)bh * N + i) * D;
    const double* S = sigma + (size_t)bh * D * D;
    constexpr int HALF = D / 2;
    double r = 0.0;
    for (int h0 = 0; h0 < D; h0 += HALF) {
        double t[HALF];
#pragma unroll
        for (int a = 0; a < HALF; ++a) t[a] = 0.0;
        for (int b = 0; b < D; ++b) {
            const double qb = (double)elem_f<T>(q + b);
            const double* Sb = S + (size_t)b * D + h0;  // Sigma[b][a] == Sigma[a][b]
#pragma unroll
            for (int a = 0; a < HALF; ++a) t[a] = fma(Sb[a], qb, t[a]);
        }
#pragma unroll
        for (int a = 0; a < HALF; ++a) r = fma((double)elem_f<T>(q + h0 + a), t[a], r);
    }
    nrm[(size_t)bh * Nv + i] = r > 0.0 ? sqrt(r) : 0.0;
}

struct RbHead {
    const double* sigma;
    const double* nrm;
    int* grp;
    double* cbuf;
    uint64_t* dk;
    int *gstart, *gc, *gcnt, *gp0, *ga, *gb, *grem;
    uint64_t *gmin, *gpre_hi, *gpre_lo;
    double* gvec;
    unsigned* hist;
};

// g(P) = t(P) / n_P for the group starting at leaf G, computed by one wave (lane a-owners).
template <typename T, int D>
__device__ __forceinline__ void pivot_vec(const RbHead& s, const T* Qh, int P, int G) {
    const int lane = threadIdx.x & 63;
    const double nP = s.nrm[P];
    const T* qp = Qh + (size_t)P * D;
#pragma unroll
    for (int k = 0; k < D / 64; ++k) {
        const int a = lane + 64 * k;
        double g = 0.0;
        if (nP != 0.0) {
            const double* Sa = s.sigma + (size_t)a * D;
            double t = 0.0;
            for (int b = 0; b < D; ++b) t = fma(Sa[b], (double)elem_f<T>(qp + b), t);
            g = t / nP;
        }
        s.gvec[(size_t)G * D + a] = g;
    }
}

template <typename T, int D>
__device__ __forceinline__ double cos_to(const RbHead& s, const T* Qh, int i, int G) {
    const double ni = s.nrm[i];
    if (ni == 0.0) return 0.0;
    const T* q = Qh + (size_t)i * D;
    const double* g = s.gvec + (size_t)G * D;
    double acc = 0.0;
    for (int a = 0; a < D; ++a) acc = fma((double)elem_f<T>(q + a), g[a], acc);
    return acc / ni;
}

template <typename T, int D>
__global__ __launch_bounds__(kRbThreads) void rb_levels_kernel(const T* __restrict__ Q, int N, int Nv, int BLK,
                                                               int M, RbLayout lay, char* ws, int32_t* __restrict__ perm) {
    const int bh = blockIdx.x, tid = threadIdx.x, w = tid >> 6;
    constexpr int NW = kRbThreads / 64;
    const T* Qh = Q + (size_t)bh * N * D;
    RbHead s;
    s.sigma = (const double*)(ws + lay.sigma) + (size_t)bh * D * D;
    s.nrm = (const double*)(ws + lay.nrm) + (size_t)bh * Nv;
    s.grp = (int*)(ws + lay.grp) + (size_t)bh * Nv;
    s.cbuf = (double*)(ws + lay.cbuf) + (size_t)bh * Nv;
    s.dk = (uint64_t*)(ws + lay.dk) + (size_t)bh * Nv;
    s.gstart = (int*)(ws + lay.gstart) + (size_t)bh * M;
    s.gc = (int*)(ws + lay.gc) + (size_t)bh * M;
    s.gcnt = (int*)(ws + lay.gcnt) + (size_t)bh * M;
    s.gp0 = (int*)(ws + lay.gp0) + (size_t)bh * M;
    s.ga = (int*)(ws + lay.ga) + (size_t)bh * M;
    s.gb = (int*)(ws + lay.gb) + (size_t)bh * M;
    s.grem = (int*)(ws + lay.grem) + (size_t)bh * M;
    s.gmin = (uint64_t*)(ws + lay.gmin) + (size_t)bh * M;
    s.gpre_hi = (uint64_t*)(ws + lay.gpre_hi) + (size_t)bh * M;
    s.gpre_lo = (uint64_t*)(ws + lay.gpre_lo) + (size_t)bh * M;
    s.gvec = (double*)(ws + lay.gvec) + (size_t)bh * M * D;
    s.hist = (unsigned*)(ws + lay.hist) + (size_t)bh * M * 256;

    // one group of all N_v tokens holding M leaves
    for (int i = tid; i < Nv; i += kRbThreads) s.grp[i] = 0;
    for (int G = tid; G < M; G += kRbThreads) {
        s.gstart[G] = G == 0;
        s.gc[G] = G == 0 ? M : 0;
        s.gcnt[G] = G == 0 ? Nv : 0;
    }
    __syncthreads();
    int levels = 0;
    while ((1 << levels) < M) ++levels;

    auto splitting = [&](int G) { return s.gstart[G] && s.gc[G] > 1; };

    for (int lev = 0; lev < levels; ++lev) {
        // ---- group state for this level
        for (int G = tid; G < M; G += kRbThreads)
            if (splitting(G)) {
                s.gp0[G] = INT_MAX;
                s.ga[G] = INT_MAX;
                s.gb[G] = INT_MAX;
                s.gmin[G] = ~0ull;
            }
        __syncthreads();
        // ---- P0: lowest token index of the group
        for (int i = tid; i < Nv; i += kRbThreads) {
            const int G = s.grp[i];
            if (s.gc[G] > 1) atomicMin(&s.gp0[G], i);
        }
        __syncthreads();
        for (int G = w; G < M; G += NW)
            if (splitting(G)) pivot_vec<T, D>(s, Qh, aload(&s.gp0[G]), G);
        __syncthreads();
        // ---- A = argmin cos(., P0), ties to the lower index
        for (int i = tid; i < Nv; i += kRbThreads) {
            const int G = s.grp[i];
            if (s.gc[G] > 1) {
                const double c = cos_to<T, D>(s, Qh, i, G);
                s.cbuf[i] = c;
                atomicMin((unsigned long long*)&s.gmin[G], (unsigned long long)asc_key(c));
            }
        }
        __syncthreads();
        for (int i = tid; i < Nv; i += kRbThreads) {
            const int G = s.grp[i];
            if (s.gc[G] > 1 && asc_key(s.cbuf[i]) == aload(&s.gmin[G])) atomicMin(&s.ga[G], i);
        }
        __syncthreads();
        for (int G = w; G < M; G += NW)
            if (splitting(G)) pivot_vec<T, D>(s, Qh, aload(&s.ga[G]), G);
        for (int G = tid; G < M; G += kRbThreads)
            if (splitting(G)) s.gmin[G] = ~0ull;
        __syncthreads();
        // ---- B = argmin cos(., A); cos(., A) is kept for the key
        for (int i = tid; i < Nv; i += kRbThreads) {
            const int G = s.grp[i];
            if (s.gc[G] > 1) {
                const double c = cos_to<T, D>(s, Qh, i, G);
                s.cbuf[i] = c;
                atomicMin((unsigned long long*)&s.gmin[G], (unsigned long long)asc_key(c));
            }
        }
        __syncthreads();
        for (int i = tid; i < Nv; i += kRbThreads) {
            const int G = s.grp[i];
            if (s.gc[G] > 1 && asc_key(s.cbuf[i]) == aload(&s.gmin[G])) atomicMin(&s.gb[G], i);
        }
        __syncthreads();
        for (int G = w; G < M; G += NW)
            if (splitting(G)) pivot_vec<T, D>(s, Qh, aload(&s.gb[G]), G);
        __syncthreads();
        // ---- key = cos(., A) - cos(., B); order (key desc, index asc) = (~asc_key(key), index) asc
        for (int i = tid; i < Nv; i += kRbThreads) {
            const int G = s.grp[i];
            if (s.gc[G] > 1) {
                const double key = s.cbuf[i] - cos_to<T, D>(s, Qh, i, G);
                s.dk[i] = ~asc_key(key);
            }
        }
        for (int G = tid; G < M; G += kRbThreads)
            if (splitting(G)) {
                s.grem[G] = ((s.gc[G] + 1) / 2) * BLK;  // rank of the last left token (1-based)
                s.gpre_hi[G] = 0;
                s.gpre_lo[G] = 0;
            }
        __syncthreads();
        // ---- radix select of the grem-th smallest (dk, index): 8 digits of dk, then 4 of index
        for (int pass = 0; pass < 12; ++pass) {
            for (int G = w; G < M; G += NW)
                if (splitting(G))
                    for (int b = tid & 63; b < 256; b += 64) s.hist[(size_t)G * 256 + b] = 0u;
            __syncthreads();
            for (int i = tid; i < Nv; i += kRbThreads) {
                const int G = s.grp[i];
                if (s.gc[G] <= 1) continue;
                const uint64_t k = s.dk[i];
                bool match;
                unsigned digit;
                if (pass < 8) {
                    match = pass == 0 || (k >> (64 - 8 * pass)) == s.gpre_hi[G];
                    digit = (unsigned)(k >> (56 - 8 * pass)) & 255u;
                } else {
                    const int p = pass - 8;
                    match = k == s.gpre_hi[G] && (p == 0 || ((uint64_t)i >> (32 - 8 * p)) == s.gpre_lo[G]);
                    digit = ((unsigned)i >> (24 - 8 * p)) & 255u;
                }
                if (match) atomicAdd(&s.hist[(size_t)G * 256 + digit], 1u);
            }
            __syncthreads();
            for (int G = tid; G < M; G += kRbThreads)
                if (splitting(G)) {
                    int rem = s.grem[G], cum = 0, dsel = 255;
                    for (int b = 0; b < 256; ++b) {
                        const int hcount = (int)aload(&s.hist[(size_t)G * 256 + b]);
                        if (cum + hcount >= rem) {
                            dsel = b;
                            break;
                        }
                        cum += hcount;
                    }
                    s.grem[G] = rem - cum;
                    if (pass < 8) s.gpre_hi[G] = (s.gpre_hi[G] << 8) | (uint64_t)dsel;
                    else s.gpre_lo[G] = (s.gpre_lo[G] << 8) | (uint64_t)dsel;
                }
            __syncthreads();
        }
        // ---- children: left = keys <= the selected one (ceil(c/2) leaves), right starts after
        for (int i = tid; i < Nv; i += kRbThreads) {
            const int G = s.grp[i];
            const int c = s.gc[G];
            if (c <= 1) continue;
            const uint64_t k = s.dk[i], th = s.gpre_hi[G];
            const bool left = k < th || (k == th && (uint64_t)i <= s.gpre_lo[G]);
            if (!left) s.grp[i] = G + (c + 1) / 2;
        }
        __syncthreads();
        for (int G = tid; G < M; G += kRbThreads)
            if (splitting(G)) {
                const int c = s.gc[G], cl = (c + 1) / 2, nl = cl * BLK;
                s.gc[G + cl] = c - cl;
                s.gcnt[G + cl] = s.gcnt[G] - nl;
                s.gstart[G + cl] = 1;
                s.gc[G] = cl;
                s.gcnt[G] = nl;
            }
        __syncthreads();
    }

    // ---- perm: leaf L holds positions L*BLK .., tokens in ascending index (stable, chunked)
    __shared__ int cnt[kMaxBlocks];
    __shared__ int sleaf[kRbThreads];
    for (int L = tid; L < M; L += kRbThreads) cnt[L] = 0;
    __syncthreads();
    int32_t* pr = perm + (size_t)bh * Nv;
    for (int base = 0; base < Nv; base += kRbThreads) {
        const int i = base + tid;
        const int leaf = i < Nv ? s.grp[i] : -1;
        sleaf[tid] = leaf;
        __syncthreads();
        if (i < Nv) {
            int rank = 0;
            for (int j = 0; j < tid; ++j) rank += sleaf[j] == leaf;
            pr[(size_t)leaf * BLK + cnt[leaf] + rank] = i;
        }
        __syncthreads();
        if (i < Nv) atomicAdd(&cnt[leaf], 1);
        __syncthreads();
    }
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
    hipLaunchKernelGGL((rb_kmax_kernel<T>), dim3(64, L.BH), dim3(256), 0, L.stream, (const T*)K, L.N, L.Nv, D, kmax);
    hipLaunchKernelGGL((rb_sigma_kernel<T, D>), dim3((L.Nv + kRbSigmaRows - 1) / kRbSigmaRows, L.BH),
                       dim3(D * D / 16), 0, L.stream, (const T*)K, L.N, L.Nv, kmax, sint);
    hipLaunchKernelGGL(rb_sigma_finalize_kernel, dim3((D * D + 255) / 256, L.BH), dim3(256), 0, L.stream, sint, kmax,
                       D, L.Nv, sigma);
    hipLaunchKernelGGL((rb_norms_kernel<T, D>), dim3((L.Nv + 255) / 256, L.BH), dim3(256), 0, L.stream, (const T*)Q,
                       L.N, L.Nv, sigma, nrm);
    hipLaunchKernelGGL((rb_levels_kernel<T, D>), dim3(L.BH), dim3(kRbThreads), 0, L.stream, (const T*)Q, L.N, L.Nv,
                       L.block, L.M, lay, w, perm);
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
