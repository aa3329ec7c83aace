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
// occupy in the permutation (leaves L0 .. L0+c-1 of a group own positions L0*block ..).  Each level
// is one launch with one workgroup per group; a stable partition writes the next level's order,
// so inside every leaf the tokens stay in ascending index and the last level writes the
// permutation itself.
#include <limits.h>

#include "kernels.hpp"

#pragma clang fp contract(off)

namespace spark {

constexpr int kRbThreads = 1024;
constexpr int kRbSigmaRows = 2048;  // rows per exact binary64 partial sum (2^42 * 2^11 = 2^53)
constexpr int kRbMaxRows = 1 << 20; // int64 sums of <= 2^20 products of magnitude <= 2^42

struct RbLayout {
    size_t kmax, sint, sigma, nrm, ord0, ord1, cbuf, dk, total;
};

static RbLayout rb_layout(const LaunchCtx& L) {
    RbLayout r;
    const size_t BH = L.BH, Nv = L.Nv, d = L.d;
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

// cos(i, P) = (fma chain over a of q_ia g_a(P)) / n_i, 0 when n_i = 0.
template <typename T, int D>
__device__ __forceinline__ double rb_cos(const T* __restrict__ Qh, const double* __restrict__ nrm, int i,
                                         const double* gv) {
    const double ni = nrm[i];
    if (ni == 0.0) return 0.0;
    const T* q = Qh + (size_t)i * D;
    double acc = 0.0;
#pragma unroll 8
    for (int a = 0; a < D; ++a) acc = fma((double)elem_f<T>(q + a), gv[a], acc);
    return acc / ni;
}

// Lexicographic minimum of (key, idx) over the workgroup (result in every thread).
template <int NT>
__device__ __forceinline__ void rb_argmin(uint64_t& key, int& idx, uint64_t* skey, int* sidx) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
        const uint64_t k2 = __shfl_xor(key, o);
        const int i2 = __shfl_xor(idx, o);
        if (k2 < key || (k2 == key && i2 < idx)) {
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
        if (k2 < key || (k2 == key && i2 < idx)) {
            key = k2;
            idx = i2;
        }
    }
    __syncthreads();
}

// One level of the partition: workgroup (group g of this level, (batch, head)).  The group's
// leaves [L0, L0 + c) follow from g's bits (most significant first: 0 = left child, which takes
// ceil(c/2) leaves).  A group of one leaf is copied; a group of more leaves is split.
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
    __shared__ unsigned hist[NW][256];
    __shared__ int sel_digit, sel_rem, wcount[2][NW];

    const int bh = blockIdx.y, g = blockIdx.x, tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    int L0 = 0, c = M;
    for (int b = lev - 1; b >= 0; --b) {
        const int cl = (c + 1) / 2;
        if ((g >> b) & 1) {
            L0 += cl;
            c -= cl;
        } else {
            c = cl;
        }
    }
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

    // P0: lowest token index of the group
    int P0 = INT_MAX;
    for (int j = tid; j < n; j += NT) P0 = min(P0, (int)seg[j]);
    {
        uint64_t k0 = 0;
        rb_argmin<NT>(k0, P0, skey, sidx);
    }
    rb_pivot<T, D, NT>(sigma, nrm, Qh, P0, gv);
    __syncthreads();
    // A = argmin cos(., P0), ties to the lower index
    uint64_t kmin = ~0ull;
    int A = INT_MAX;
    for (int j = tid; j < n; j += NT) {
        const int i = seg[j];
        const uint64_t k = asc_key(rb_cos<T, D>(Qh, nrm, i, gv));
        if (k < kmin || (k == kmin && i < A)) {
            kmin = k;
            A = i;
        }
    }
    rb_argmin<NT>(kmin, A, skey, sidx);
    rb_pivot<T, D, NT>(sigma, nrm, Qh, A, gv);
    __syncthreads();
    // B = argmin cos(., A); cos(., A) is kept for the key
    kmin = ~0ull;
    int B = INT_MAX;
    for (int j = tid; j < n; j += NT) {
        const int i = seg[j];
        const double cA = rb_cos<T, D>(Qh, nrm, i, gv);
        cb[j] = cA;
        const uint64_t k = asc_key(cA);
        if (k < kmin || (k == kmin && i < B)) {
            kmin = k;
            B = i;
        }
    }
    rb_argmin<NT>(kmin, B, skey, sidx);
    rb_pivot<T, D, NT>(sigma, nrm, Qh, B, gv);
    __syncthreads();
    // key = cos(., A) - cos(., B); order (key desc, index asc) = (~asc_key(key), index) asc
    for (int j = tid; j < n; j += NT) {
        const int i = seg[j];
        dk[j] = ~asc_key(cb[j] - rb_cos<T, D>(Qh, nrm, i, gv));
    }
    __syncthreads();
    // radix select of the nl-th smallest (dk, index): 8 digits of dk, then 3 of the index (< 2^24)
    const int nl = ((c + 1) / 2) * BLK;
    uint64_t pre_hi = 0;
    uint32_t pre_lo = 0;
    int rem = nl;
    for (int pass = 0; pass < 11; ++pass) {
        for (int b = lane; b < 256; b += 64) hist[w][b] = 0u;
        __syncthreads();
        for (int j = tid; j < n; j += NT) {
            const uint64_t k = dk[j];
            const uint32_t i = (uint32_t)seg[j];
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
            if (match) atomicAdd(&hist[w][digit], 1u);
        }
        __syncthreads();
        if (w == 0) {
            // lane l owns bins 4l .. 4l+3
            unsigned cnt[4], tot = 0;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                unsigned v = 0;
                for (int u = 0; u < NW; ++u) v += hist[u][4 * lane + q];
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
                sel_digit = dsel;
                sel_rem = rem - (int)cum;
            }
        }
        __syncthreads();
        const unsigned dsel = (unsigned)sel_digit;
        rem = sel_rem;
        if (pass < 8) pre_hi = (pre_hi << 8) | dsel;
        else pre_lo = (pre_lo << 8) | dsel;
        __syncthreads();
    }
    // stable partition: the nl smallest (dk, index) first, in their current order, then the rest
    int lbase = 0, rbase = 0;
    for (int j0 = 0; j0 < n; j0 += NT) {
        const int j = j0 + tid;
        bool left = false;
        int i = 0;
        if (j < n) {
            const uint64_t k = dk[j];
            i = seg[j];
            left = k < pre_hi || (k == pre_hi && (uint32_t)i <= pre_lo);
        }
        const uint64_t bl = __ballot(left && j < n), br = __ballot(!left && j < n);
        const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
        if (lane == 0) {
            wcount[0][w] = __popcll(bl);
            wcount[1][w] = __popcll(br);
        }
        __syncthreads();
        int lw = 0, rw = 0, lt = 0, rt = 0;
        for (int v = 0; v < NW; ++v) {
            if (v < w) {
                lw += wcount[0][v];
                rw += wcount[1][v];
            }
            lt += wcount[0][v];
            rt += wcount[1][v];
        }
        if (j < n) {
            if (left) out[lbase + lw + __popcll(bl & below)] = i;
            else out[nl + rbase + rw + __popcll(br & below)] = i;
        }
        lbase += lt;
        rbase += rt;
        __syncthreads();
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
    hipLaunchKernelGGL((rb_kmax_kernel<T>), dim3(64, L.BH), dim3(256), 0, L.stream, (const T*)K, L.N, L.Nv, D, kmax);
    hipLaunchKernelGGL((rb_sigma_kernel<T, D>), dim3((L.Nv + kRbSigmaRows - 1) / kRbSigmaRows, L.BH),
                       dim3(D * D / 16), 0, L.stream, (const T*)K, L.N, L.Nv, kmax, sint);
    hipLaunchKernelGGL(rb_sigma_finalize_kernel, dim3((D * D + 255) / 256, L.BH), dim3(256), 0, L.stream, sint, kmax,
                       D, L.Nv, sigma);
    hipLaunchKernelGGL((rb_norms_kernel<T, D>), dim3((L.Nv + 255) / 256, L.BH), dim3(256), 0, L.stream, (const T*)Q,
                       L.N, L.Nv, sigma, nrm);
    int32_t* ord[2] = {(int32_t*)(w + lay.ord0), (int32_t*)(w + lay.ord1)};
    double* cbuf = (double*)(w + lay.cbuf);
    uint64_t* dk = (uint64_t*)(w + lay.dk);
    hipLaunchKernelGGL(rb_iota_kernel, dim3((L.Nv + 255) / 256, L.BH), dim3(256), 0, L.stream, L.M > 1 ? ord[0] : perm,
                       L.Nv);
    int levels = 0;
    while ((1 << levels) < L.M) ++levels;
    for (int lev = 0; lev < levels; ++lev) {
        int32_t* dst = lev + 1 == levels ? perm : ord[(lev + 1) & 1];
        const dim3 grid(1u << lev, L.BH);
        // wide workgroups while the groups are few and large, narrow ones once they are many
        if ((1 << lev) <= 32)
            hipLaunchKernelGGL((rb_level_kernel<T, D, 1024>), grid, dim3(1024), 0, L.stream, (const T*)Q, L.N, L.Nv,
                               L.block, L.M, lev, sigma, nrm, ord[lev & 1], dst, cbuf, dk);
        else
            hipLaunchKernelGGL((rb_level_kernel<T, D, 256>), grid, dim3(256), 0, L.stream, (const T*)Q, L.N, L.Nv,
                               L.block, L.M, lev, sigma, nrm, ord[lev & 1], dst, cbuf, dk);
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
