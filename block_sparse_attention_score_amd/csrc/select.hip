// Top-K key-block selection per query block (core sparse-attention node page, section
// "ブロックスパースアテンション": each query block is routed to a subset of key blocks; the top-k
// mode keeps a fixed fraction of them; Spark-H3 page, "ワークフロー": topk_mode=topk_ratio).
//
// Two kernels:
//  1. block_scores: S_IJ = s * q_mean_I . k_mean_J for every (batch, head), a batched GEMM on the
//     bf16 matrix cores (v_mfma_f32_32x32x16_bf16; 128 x 128 output tile per workgroup, 64 x 64 per
//     wave).  Scores must be fp32-accurate: a near-tie between the K-th and (K+1)-th block is decided
//     by them, so one bf16 rounding of the means is not allowed.  Each fp32 mean is written exactly
//     as the sum of three bf16 parts (x = h + m + l, |m| <= 2^-8 |x|, |l| <= 2^-16 |x|), and the
//     six part products of weight at least 2^-16 are accumulated (small ones first).  The dropped
//     ones (m.l, l.m, l.l) stay below 2^-23 of sum |q||k|, under the worst-case fp32 rounding of
//     a d-term sum (about d * 2^-24).
//  2. topk_rows: one wave per score row.  The row's scores live in registers as order-preserving
//     integer keys (KPL per lane); the K-th largest key is found by counting keys >= a candidate
//     with wave ballots and popcounts: first at candidates guessed from the row's mean and spread
//     (they bracket the threshold and usually hit a candidate with exactly K keys above it, which
//     ends the search), then bit by bit inside the bracket; ties at the threshold go to the lower
//     block index; the chosen blocks are written in ascending order by a ballot/popcount
//     compaction.  Deterministic, no atomics.
#include <cmath>

#include "kernels.hpp"

namespace spark {

constexpr int kST = 128;      // score tile (rows and columns) of a workgroup
constexpr int kSD = 32;       // d per LDS stage
constexpr int kSP = kSD;      // LDS row of a bf16 part plane (elements, 64 bytes, four 16-byte chunks)

// LDS element offset of element c of row r in a part plane: the 16-byte chunk index is XORed with
// bits 1..2 of the row, so the 16-byte operand reads of 8 consecutive rows at one chunk touch 8
// different 16-byte bank groups (two rows per 128 bytes, four chunk positions each)
__device__ __forceinline__ int plane_at(int r, int c) { return r * kSP + ((((c >> 3) ^ (r >> 1)) & 3) << 3) + (c & 7); }

// x = h + m + l exactly, each part bf16 (round to nearest even at every step).  h is x rounded to 8
// significant bits, so x - h is exact (Sterbenz) and holds at most 16 significant bits; m rounds that
// to 8, and the remainder holds at most 8, so l is exact: the three parts carry every bit of x.
// (Parts that fall below the smallest normal number may be flushed; that moves x by < 2^-126.)
__device__ __forceinline__ void split3(float x, __bf16& h, __bf16& m, __bf16& l) {
    h = (__bf16)x;
    const float r1 = x - (float)h;
    m = (__bf16)r1;
    l = (__bf16)(r1 - (float)m);
}

// S [BH][Mq][Mk]: query-block means (A, rows) against key-block means (B, columns).  The workgroup
// stages 128 rows of each operand, 32 d at a time: the fp32 values are read with coalesced 16-byte
// loads, split into their three bf16 parts once, and stored as three planes.  Wave w computes rows
// 64 (w / 2) and columns 64 (w % 2) of the tile as 2 x 2 MFMA tiles of 32 x 32.  For each 16-d step,
// lane (i, g) feeds the 8 d values 8g .. 8g+7 of row i of A and of B (the same d for both operands,
// as the MFMA pairs them); the part products go into one accumulator in the order l.h, m.m, h.l,
// m.h, h.m, h.h (the dropped m.l, l.m and l.l are below 2^-23 of h.h).  Accumulator register r of
// lane (i, g) is row 8 (r / 4) + 4 g + r % 4, column i of its 32 x 32 tile.
__global__ __launch_bounds__(256, 3) void block_scores_kernel(const float* __restrict__ q_mean,
                                                              const float* __restrict__ k_mean, int Mq, int M,
                                                              int D, float scale, float* __restrict__ S) {
    __shared__ __attribute__((aligned(16))) __bf16 As[3][kST * kSP];
    __shared__ __attribute__((aligned(16))) __bf16 Bs[3][kST * kSP];
    // Workgroup w runs on XCD w % 8.  Tiles are numbered row band by row band (column tile fastest)
    // and each XCD takes one contiguous run of them, so the column tiles of a band run side by side
    // on one XCD: the cache lines that straddle two column tiles (rows are not line-aligned) are
    // completed in that XCD's L2 and written back once, and a head's operands stay in one L2.
    const int n = gridDim.x, q8 = n >> 3, r8 = n & 7, xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
    const int tile = xcd < r8 ? xcd * (q8 + 1) + slot : r8 * (q8 + 1) + (xcd - r8) * q8 + slot;
    const int gx = (M + kST - 1) / kST, gy = (Mq + kST - 1) / kST;
    const int bh = tile / (gx * gy), I0 = (tile / gx % gy) * kST, J0 = (tile % gx) * kST;
    const int t = threadIdx.x, w = t >> 6, lane = t & 63, i = lane & 31, g = lane >> 5;
    const float* qb = q_mean + (size_t)bh * Mq * D;
    const float* kb = k_mean + (size_t)bh * M * D;
    const int r0 = 64 * (w >> 1), c0 = 64 * (w & 1);
    f32x16 acc[2][2];
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[a][b][r] = 0.f;
    // 128 rows x 32 d = 1024 float4 per operand, four per thread; the next stage's values are
    // loaded before the current stage's products are issued, so the loads run under them
    f32x4 qv[4], kv[4];
    auto load_stage = [&](int d0) __attribute__((always_inline)) {
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int e = t + 256 * k, r = e >> 3, c = (e & 7) * 4;
            qv[k] = f32x4{0.f, 0.f, 0.f, 0.f};
            kv[k] = f32x4{0.f, 0.f, 0.f, 0.f};
            if (I0 + r < Mq) qv[k] = *reinterpret_cast<const f32x4*>(qb + (size_t)(I0 + r) * D + d0 + c);
            if (J0 + r < M) kv[k] = *reinterpret_cast<const f32x4*>(kb + (size_t)(J0 + r) * D + d0 + c);
        }
    };
    load_stage(0);
    for (int d0 = 0; d0 < D; d0 += kSD) {
        __syncthreads();  // every wave is done with the previous stage's planes
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int e = t + 256 * k, r = e >> 3, c = (e & 7) * 4;
            bf16x4 qh, qm, ql, kh, km, kl;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                __bf16 x0, x1, x2;
                split3(qv[k][j], x0, x1, x2);
                qh[j] = x0, qm[j] = x1, ql[j] = x2;
                split3(kv[k][j], x0, x1, x2);
                kh[j] = x0, km[j] = x1, kl[j] = x2;
            }
            const int o = plane_at(r, c);
            *reinterpret_cast<bf16x4*>(&As[0][o]) = qh;
            *reinterpret_cast<bf16x4*>(&As[1][o]) = qm;
            *reinterpret_cast<bf16x4*>(&As[2][o]) = ql;
            *reinterpret_cast<bf16x4*>(&Bs[0][o]) = kh;
            *reinterpret_cast<bf16x4*>(&Bs[1][o]) = km;
            *reinterpret_cast<bf16x4*>(&Bs[2][o]) = kl;
        }
        __syncthreads();
        if (d0 + kSD < D) load_stage(d0 + kSD);
#pragma unroll
        for (int ks = 0; ks < kSD / 16; ++ks) {
            bf16x8 a[2][3], b[2][3];
#pragma unroll
            for (int x = 0; x < 2; ++x)
#pragma unroll
                for (int p = 0; p < 3; ++p) {
                    a[x][p] = *reinterpret_cast<const bf16x8*>(&As[p][plane_at(r0 + 32 * x + i, 16 * ks + 8 * g)]);
                    b[x][p] = *reinterpret_cast<const bf16x8*>(&Bs[p][plane_at(c0 + 32 * x + i, 16 * ks + 8 * g)]);
                }
#pragma unroll
            for (int x = 0; x < 2; ++x)
#pragma unroll
                for (int y = 0; y < 2; ++y) {
                    f32x16 c = acc[x][y];
                    c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[x][2], b[y][0], c, 0, 0, 0);
                    c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[x][1], b[y][1], c, 0, 0, 0);
                    c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[x][0], b[y][2], c, 0, 0, 0);
                    c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[x][1], b[y][0], c, 0, 0, 0);
                    c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[x][0], b[y][1], c, 0, 0, 0);
                    acc[x][y] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[x][0], b[y][0], c, 0, 0, 0);
                }
        }
    }
#pragma unroll
    for (int y = 0; y < 2; ++y) {
        const int J = J0 + c0 + 32 * y + i;
        if (J >= M) continue;
#pragma unroll
        for (int x = 0; x < 2; ++x)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int I = I0 + r0 + 32 * x + 8 * (r >> 2) + 4 * g + (r & 3);
                if (I < Mq) S[((size_t)bh * Mq + I) * M + J] = scale * acc[x][y][r];
            }
    }
}

// Order-preserving map float -> uint32 (larger float, larger key); -0 is folded onto +0.  Every
// finite score maps to a key >= 1, so 0 can pad a row.
__device__ __forceinline__ uint32_t score_key(float f) {
    f = f + 0.0f;
    const uint32_t u = __float_as_uint(f);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Number of keys >= c in the row (c wave-uniform and >= 1, so the padding key 0 never counts).
// number of set bits of a wave mask m in the lanes below this one (two mbcnt instructions)
__device__ __forceinline__ int rank_below(uint64_t m) {
    return (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

template <int KPL>
__device__ __forceinline__ int count_ge(const uint32_t (&key)[KPL], uint32_t c) {
    int n = 0;
#pragma unroll
    for (int j = 0; j < KPL; ++j) n += __popcll(__ballot(key[j] >= c));
    return n;
}

__device__ __forceinline__ float uniform_f32(float v) {
    return __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(v)));
}

// The K largest of a row of M scores held in registers (lane l: block l + 64 j; f the scores, key
// their order-preserving keys; past the row end f holds 0 and key the padding key 0), written to out[0 .. K) in ascending
// block order.  T, the K-th largest key, is max{t : #{keys >= t} >= K}.  The search keeps a bracket
// lo < hi of counted candidates, #{>= lo} >= K > #{>= hi}, and stops as soon as a candidate has
// exactly K keys at or above it: those are the K largest, written out as they are (no key outside
// them equals one inside, so no tie is left to break).
//  1. Guesses.  The row's mean mu and standard deviation sd (fp32) place the first candidate at
//     mu + zk * sd, zk the standard normal quantile of 1 - K / M; then Newton steps with the normal
//     density at zk (dens_c = 1 / (M * phi(zk))) until the bracket closes on both sides, then secant
//     steps between its ends.  On block scores, whose upper tail is close to normal, this lands on
//     an exact count after about four counts.  The guesses only choose which candidates get counted:
//     any row distribution (ties, constant rows, NaN statistics) still ends in the exact T.
//  2. Bit-serial completion (when no guess hit an exact count): T takes each bit from the top when at
//     least K keys are >= T with it; candidates at or below lo take the bit and candidates at or
//     above hi do not, without a count; the exact-count stop applies here too.
// Otherwise T is exact and ties at T go to the lower block index.
template <int KPL>
__device__ __forceinline__ void topk_of_row(const uint32_t (&key)[KPL], const float (&f)[KPL], int M, int K,
                                            float zk, float dens_c, int32_t* out) {
    const int lane = threadIdx.x & 63;
    float s = 0.f, s2 = 0.f;  // columns past the row end hold 0 in f and add nothing
#pragma unroll
    for (int j = 0; j < KPL; ++j) {
        s += f[j];
        s2 = fmaf(f[j], f[j], s2);
    }
    const float mu = uniform_f32(wave_sum(s) / (float)M);
    const float sd = uniform_f32(sqrtf(fmaxf(wave_sum(s2) / (float)M - mu * mu, 0.f)));
    uint32_t lo = 0;                 // #{>= 0} = M >= K
    uint64_t hi = 1ull << 32;        // #{>= 2^32} = 0 < K
    int c_lo = M, c_hi = 0;
    float x_lo = 0.f, x_hi = 0.f;
    bool has_xlo = false, has_xhi = false, exact = false;
    float x = fmaf(zk, sd, mu);
    for (int it = 0; it < 8; ++it) {
        const uint32_t cand = max(score_key(x), 1u);
        if (!(cand > lo && (uint64_t)cand < hi)) break;  // also a NaN guess
        const int c = count_ge(key, cand);
        if (c >= K) {
            lo = cand, c_lo = c, x_lo = x, has_xlo = true;
            if (c == K) {
                exact = true;
                break;
            }
        } else {
            hi = cand, c_hi = c, x_hi = x, has_xhi = true;
        }
        if (has_xlo && has_xhi)
            x = fmaf((float)(c_lo - K) / (float)(c_lo - c_hi), x_hi - x_lo, x_lo);
        else
            x = fmaf((float)(c - K) * dens_c, sd, x);
        x = uniform_f32(x);
    }
    uint32_t T = 0;
    if (!exact) {
        for (int bit = 31; bit >= 0; --bit) {
            const uint32_t cand = T | (1u << bit);
            if (cand <= lo) {
                T = cand;
                continue;
            }
            if ((uint64_t)cand >= hi) continue;
            const int c = count_ge(key, cand);
            if (c >= K) {
                T = lo = cand;
                if (c == K) {
                    exact = true;
                    break;
                }
            } else {
                hi = cand;
            }
        }
    }
    if (exact) {  // exactly the K largest are >= lo: they are the output, with no tie to break
        int pos = 0;
#pragma unroll
        for (int j = 0; j < KPL; ++j) {
            const bool sel = key[j] >= lo;
            const uint64_t sb = __ballot(sel);
            if (sel) out[pos + rank_below(sb)] = lane + 64 * j;
            pos += __popcll(sb);
        }
        return;
    }
    int gt = 0;
#pragma unroll
    for (int j = 0; j < KPL; ++j) gt += __popcll(__ballot(key[j] > T));
    const int need = K - gt;  // keys equal to T still to take, lowest block index first
    int pos = 0, eq_seen = 0;
#pragma unroll
    for (int j = 0; j < KPL; ++j) {
        const uint32_t kk = key[j];
        const uint64_t eqb = __ballot(kk == T);
        const int eq_rank = eq_seen + rank_below(eqb);
        const bool sel = kk > T || (kk == T && eq_rank < need);
        const uint64_t sb = __ballot(sel);
        if (sel) out[pos + rank_below(sb)] = lane + 64 * j;
        pos += __popcll(sb);
        eq_seen += __popcll(eqb);
    }
}

// KPL > 0: the row is held in KPL registers per lane (M <= 64 * KPL).  KPL == 0: the row is
// re-read from memory on every pass (any M).
template <int KPL>
__global__ __launch_bounds__(256) void topk_rows_kernel(const float* __restrict__ S, int rows, int M, int K,
                                                        float zk, float dens_c, int32_t* __restrict__ idx) {
    const int lane = threadIdx.x & 63;
    const int row = __builtin_amdgcn_readfirstlane(blockIdx.x * 4 + (threadIdx.x >> 6));  // one row per wave
    if (row >= rows) return;
    const float* Sr = S + (size_t)row * M;
    int32_t* const out = idx + (size_t)row * K;
    if constexpr (KPL > 0) {
        // every load is unconditional so that all of them are in flight together: buffer loads with
        // the row as the buffer's extent (a column past the row end reads 0), one offset register
        // and the column step in the instruction; those columns then take the padding key
        const __amdgpu_buffer_rsrc_t rs =
            __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(Sr), (short)0, M * 4, 0x00020000);
        float f[KPL];
#pragma unroll
        for (int j = 0; j < KPL; ++j)
            f[j] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rs, lane * 4 + 256 * j, 0, 0));
        uint32_t key[KPL];
#pragma unroll
        for (int j = 0; j < KPL; ++j) key[j] = lane + 64 * j < M ? score_key(f[j]) : 0u;
        topk_of_row<KPL>(key, f, M, K, zk, dens_c, out);
        return;
    } else {
        // the row is re-read from memory on every pass (any M)
        auto key_at = [&](int j) -> uint32_t {  // key of block lane + 64 j
            const int J = lane + 64 * j;
            return J < M ? score_key(Sr[J]) : 0u;
        };
        const int chunks = (M + 63) / 64;
        // largest T with #{J : key_J >= T} >= K, i.e. the K-th largest key
        uint32_t T = 0;
        for (int bit = 31; bit >= 0; --bit) {
            const uint32_t cand = T | (1u << bit);
            int cnt = 0;
            for (int j = 0; j < chunks; ++j) cnt += __popcll(__ballot(key_at(j) >= cand));
            if (cnt >= K) T = cand;
        }
        int gt = 0;
        for (int j = 0; j < chunks; ++j) gt += __popcll(__ballot(key_at(j) > T));
        const int need = K - gt;  // keys equal to T still to take, lowest block index first
        const uint64_t below = lanemask_lt();
        int pos = 0, eq_seen = 0;
        for (int j = 0; j < chunks; ++j) {
            const uint32_t kk = key_at(j);
            const uint64_t eqb = __ballot(kk == T);
            const int eq_rank = eq_seen + __popcll(eqb & below);
            const bool sel = kk > T || (kk == T && eq_rank < need);
            const uint64_t sb = __ballot(sel);
            if (sel) out[pos + __popcll(sb & below)] = lane + 64 * j;
            pos += __popcll(sb);
            eq_seen += __popcll(eqb);
        }
    }
}

// ---- adaptive-tau selection (core node page, "ブロックスパースアテンション", Sol-Attn bullet: a
// per-head threshold in sigma units of the score distribution).  Over the M x M scores of a
// (batch, head): mu = mean, sigma = population standard deviation, both in binary64 from sums of
// S and S^2 (per-workgroup partial sums in a fixed order, then the partials in a fixed order, so
// the result does not depend on timing); row I keeps every J with S_IJ > mu + tau * sigma.
constexpr int kTauParts = 64;

size_t tau_partials_bytes(const LaunchCtx& L) { return (size_t)L.BH * kTauParts * 2 * sizeof(double); }

__device__ __forceinline__ double wave_sum_f64(double v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
    return v;
}

// grid (kTauParts, BH): partial sums of S and S^2 over one contiguous part of a head's scores
__global__ __launch_bounds__(256) void tau_partial_kernel(const float* __restrict__ S, int M,
                                                          double* __restrict__ partial) {
    __shared__ double red[2][4];
    const int bh = blockIdx.y, part = blockIdx.x, t = threadIdx.x;
    const size_t MM = (size_t)M * M, chunk = (MM + kTauParts - 1) / kTauParts;
    const size_t lo = (size_t)part * chunk, hi = min(MM, lo + chunk);
    const float* Sh = S + (size_t)bh * MM;
    double s = 0.0, q = 0.0;
    for (size_t e = lo + t; e < hi; e += 256) {
        const double x = (double)Sh[e];
        s += x;
        q += x * x;
    }
    s = wave_sum_f64(s);
    q = wave_sum_f64(q);
    if ((t & 63) == 0) {
        red[0][t >> 6] = s;
        red[1][t >> 6] = q;
    }
    __syncthreads();
    if (t == 0) {
        double ts = 0.0, tq = 0.0;
        for (int w = 0; w < 4; ++w) {
            ts += red[0][w];
            tq += red[1][w];
        }
        partial[((size_t)bh * kTauParts + part) * 2] = ts;
        partial[((size_t)bh * kTauParts + part) * 2 + 1] = tq;
    }
}

// one wave per score row: the head's threshold from the partials, then the kept blocks of the row
// in ascending order (ballot compaction) and their count
__global__ __launch_bounds__(256) void tau_rows_kernel(const float* __restrict__ S, int rows, int M, float tau,
                                                       const double* __restrict__ partial,
                                                       int32_t* __restrict__ idx, int32_t* __restrict__ counts,
                                                       float* __restrict__ stats) {
    const int lane = threadIdx.x & 63;
    const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (row >= rows) return;
    const int bh = row / M;
    const double* pp = partial + (size_t)bh * kTauParts * 2;
    const double MM = (double)M * (double)M;
    const double sum = wave_sum_f64(lane < kTauParts ? pp[2 * lane] : 0.0);
    const double sumsq = wave_sum_f64(lane < kTauParts ? pp[2 * lane + 1] : 0.0);
    const double mu = sum / MM;
    const double sigma = sqrt(fmax(sumsq / MM - mu * mu, 0.0));
    const double thr = mu + (double)tau * sigma;
    const float* Sr = S + (size_t)row * M;
    int32_t* out = idx + (size_t)row * M;
    const uint64_t below = lanemask_lt();
    int pos = 0;
    // eight column chunks at a time, loaded unconditionally (clamped column) so that the loads of a
    // batch are in flight together
    for (int J0 = 0; J0 < M; J0 += 64 * 8) {
        float f[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) f[u] = Sr[min(J0 + 64 * u + lane, M - 1)];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int J = J0 + 64 * u + lane;
            const bool keep = J < M && (double)f[u] > thr;
            const uint64_t kb = __ballot(keep);
            if (keep) out[pos + __popcll(kb & below)] = J;
            pos += __popcll(kb);
        }
    }
    if (lane == 0) {
        counts[row] = pos;
        if (stats && row % M == 0) {
            stats[2 * bh] = (float)mu;
            stats[2 * bh + 1] = (float)sigma;
        }
    }
}

void launch_select_tau(const LaunchCtx& L, float tau, const float* q_mean, const float* k_mean, int32_t* idx,
                       int32_t* counts, float* stats, float* scores, double* partials) {
    const dim3 sgrid(((L.M + kST - 1) / kST) * ((L.M + kST - 1) / kST) * L.BH);
    hipLaunchKernelGGL(block_scores_kernel, sgrid, dim3(256), 0, L.stream, q_mean, k_mean, L.M, L.M, L.d, L.scale,
                       scores);
    hipLaunchKernelGGL(tau_partial_kernel, dim3(kTauParts, L.BH), dim3(256), 0, L.stream, scores, L.M, partials);
    const int rows = L.BH * L.M;
    hipLaunchKernelGGL(tau_rows_kernel, dim3((rows + 3) / 4), dim3(256), 0, L.stream, scores, rows, L.M, tau,
                       partials, idx, counts, stats);
}

size_t select_workspace_bytes(const LaunchCtx& L) { return (size_t)L.BH * L.M * L.Mk * 4; }

void launch_select(const LaunchCtx& L, const float* q_mean, const float* k_mean, int32_t* idx, float* scores) {
    const dim3 sgrid(((L.Mk + kST - 1) / kST) * ((L.M + kST - 1) / kST) * L.BH);
    hipLaunchKernelGGL(block_scores_kernel, sgrid, dim3(256), 0, L.stream, q_mean, k_mean, L.M, L.Mk, L.d,
                       L.scale, scores);
    const int rows = L.BH * L.M;
    const dim3 tgrid((rows + 3) / 4);
    const int need = (L.Mk + 63) / 64;
    // search hints for the register-resident top-K: the standard normal quantile zk of 1 - K / Mk and
    // 1 / (Mk * phi(zk)), phi the standard normal density (they steer the search, not its result)
    const double p = 1.0 - (double)L.K / (double)L.Mk;
    double zlo = -8.0, zhi = 8.0;  // Phi(z) = p by bisection on Phi(z) = erfc(-z / sqrt 2) / 2
    for (int it = 0; it < 60; ++it) {
        const double zm = 0.5 * (zlo + zhi);
        (0.5 * std::erfc(-zm / std::sqrt(2.0)) < p ? zlo : zhi) = zm;
    }
    const double zk = 0.5 * (zlo + zhi);
    const double dens_c = 1.0 / ((double)L.Mk * std::exp(-0.5 * zk * zk) / std::sqrt(2.0 * M_PI));
#define SPARK_TOPK(KPL)                                                                                      \
    hipLaunchKernelGGL((topk_rows_kernel<KPL>), tgrid, dim3(256), 0, L.stream, scores, rows, L.Mk, L.K, (float)zk, \
                       (float)dens_c, idx)
    if (need <= 1) SPARK_TOPK(1);
    else if (need <= 2) SPARK_TOPK(2);
    else if (need <= 4) SPARK_TOPK(4);
    else if (need <= 8) SPARK_TOPK(8);
    else if (need <= 16) SPARK_TOPK(16);
    else if (need <= 32) SPARK_TOPK(32);
    else if (need <= 64) SPARK_TOPK(64);
    else SPARK_TOPK(0);
#undef SPARK_TOPK
}

}  // namespace spark
