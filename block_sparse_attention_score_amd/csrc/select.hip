// Top-K key-block selection per query block (core sparse-attention node page, section
// "ブロックスパースアテンション": each query block is routed to a subset of key blocks; the top-k
// mode keeps a fixed fraction of them; Spark-H3 page, "ワークフロー": topk_mode=topk_ratio).
//
// Two kernels:
//  1. block_scores: S_IJ = s * q_mean_I . k_mean_J for every (batch, head), a batched fp32 GEMM on
//     the fp32 matrix cores (v_mfma_f32_32x32x2_f32; 64 x 64 output tile per workgroup, 32 x 32
//     per wave, d staged through LDS 32 at a time).  Scores must be fp32-accurate: a near-tie between the K-th and (K+1)-th block is
//     decided by them, so no bf16 rounding is allowed here.
//  2. topk_rows: one wave per score row.  The row's scores live in registers as order-preserving
//     integer keys (KPL per lane); the K-th largest key is found bit by bit from the top, counting
//     keys >= candidate with wave ballots and popcounts, and stops early once exactly K keys lie
//     above the candidate; ties at the threshold go to the lower block index; the chosen blocks
//     are written in ascending order by a ballot/popcount compaction.  Deterministic, no atomics.
#include "kernels.hpp"

namespace spark {

constexpr int kGT = 64;   // score tile (rows and columns) of a workgroup
constexpr int kGD = 32;   // d per LDS stage

// S [BH][Mq][Mk]: query-block means against key-block means.  The workgroup stages 64 rows of
// each operand, 32 d at a time, in LDS (coalesced row reads); wave w computes the 32 x 32 tile
// (rows 32 (w / 2), columns 32 (w % 2) of the workgroup's).  Lane (i, h) feeds row i of both
// operands (A: a query-block mean, B: a key-block mean) with the four d values 8t + 4h .. +3 of
// step t from one 16-byte LDS read each; MFMA j of the step takes element j, so its two k slots
// hold d = 8t + j and 8t + 4 + j for both operands alike, and over a step every d of the eight
// comes once.  Accumulator register r of lane (i, h) is row 8 (r / 4) + 4 h + r % 4, column i.
__global__ __launch_bounds__(256) void block_scores_kernel(const float* __restrict__ q_mean,
                                                           const float* __restrict__ k_mean, int Mq, int M,
                                                           int D, float scale, float* __restrict__ S) {
    constexpr int LD = kGD + 4;  // padded LDS row (floats)
    __shared__ __attribute__((aligned(16))) float Qs[kGT * LD];
    __shared__ __attribute__((aligned(16))) float Ks[kGT * LD];
    const int bh = blockIdx.z, I0 = blockIdx.y * kGT, J0 = blockIdx.x * kGT;
    const int t = threadIdx.x, w = t >> 6, lane = t & 63, i = lane & 31, h = lane >> 5;
    const float* qb = q_mean + (size_t)bh * Mq * D;
    const float* kb = k_mean + (size_t)bh * M * D;
    const int qrow = 32 * (w >> 1) + i, krow = 32 * (w & 1) + i;
    f32x16 acc;
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[r] = 0.f;
    for (int d0 = 0; d0 < D; d0 += kGD) {
        __syncthreads();
#pragma unroll
        for (int k = 0; k < 2; ++k) {  // 64 rows x 32 d = 512 float4 per operand
            const int e = t + 256 * k, r = e / 8, c = (e % 8) * 4;
            f32x4 qv = {0.f, 0.f, 0.f, 0.f}, kv = {0.f, 0.f, 0.f, 0.f};
            if (I0 + r < Mq) qv = *reinterpret_cast<const f32x4*>(qb + (size_t)(I0 + r) * D + d0 + c);
            if (J0 + r < M) kv = *reinterpret_cast<const f32x4*>(kb + (size_t)(J0 + r) * D + d0 + c);
            *reinterpret_cast<f32x4*>(&Qs[r * LD + c]) = qv;
            *reinterpret_cast<f32x4*>(&Ks[r * LD + c]) = kv;
        }
        __syncthreads();
#pragma unroll
        for (int s8 = 0; s8 < kGD / 8; ++s8) {
            const f32x4 a = *reinterpret_cast<const f32x4*>(&Qs[qrow * LD + 8 * s8 + 4 * h]);
            const f32x4 b = *reinterpret_cast<const f32x4*>(&Ks[krow * LD + 8 * s8 + 4 * h]);
#pragma unroll
            for (int j = 0; j < 4; ++j) acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a[j], b[j], acc, 0, 0, 0);
        }
    }
    const int J = J0 + krow;
    if (J >= M) return;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        const int I = I0 + 32 * (w >> 1) + 8 * (r >> 2) + 4 * h + (r & 3);
        if (I < Mq) S[((size_t)bh * Mq + I) * M + J] = scale * acc[r];
    }
}

// Order-preserving map float -> uint32 (larger float, larger key); -0 is folded onto +0.  Every
// finite score maps to a key >= 1, so 0 can pad a row.
__device__ __forceinline__ uint32_t score_key(float f) {
    f = f + 0.0f;
    const uint32_t u = __float_as_uint(f);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// The K largest of each of R rows held as keys in registers (lane l: block l + 64 j for j < chunks,
// padding key 0), written to out[q][0 .. K) in ascending block order (rows with a null out are
// skipped).  The K-th largest key T of a row is found bit by bit from the top: T takes the bit when
// at least K keys are >= T with it (counted with wave ballots and popcounts).  When exactly K keys
// are >= that candidate, they are the K largest, so T is their minimum and the search stops there
// (about half the passes on continuous scores).  Ties at T go to the lower block index.  The R
// rows' searches run interleaved (independent chains).
template <int KPL, int R>
__device__ __forceinline__ void topk_of_rows(const uint32_t (&key)[R][KPL], int chunks, int K,
                                             int32_t* const (&out)[R]) {
    const int lane = threadIdx.x & 63;
    uint32_t T[R];
    bool done[R];
#pragma unroll
    for (int q = 0; q < R; ++q) {
        T[q] = 0;
        done[q] = out[q] == nullptr;
    }
    for (int bit = 31; bit >= 0; --bit) {
        bool all = true;
#pragma unroll
        for (int q = 0; q < R; ++q) all = all && done[q];
        if (all) break;
        int cnt[R];
#pragma unroll
        for (int q = 0; q < R; ++q) cnt[q] = 0;
#pragma unroll
        for (int j = 0; j < KPL; ++j)
            if (j < chunks)
#pragma unroll
                for (int q = 0; q < R; ++q)
                    if (!done[q]) cnt[q] += __popcll(__ballot(key[q][j] >= (T[q] | (1u << bit))));
#pragma unroll
        for (int q = 0; q < R; ++q) {
            if (done[q] || cnt[q] < K) continue;
            T[q] |= 1u << bit;
            if (cnt[q] == K) {  // exactly the K largest are >= T: the K-th largest is their minimum
                uint32_t m = 0xffffffffu;
#pragma unroll
                for (int j = 0; j < KPL; ++j)
                    if (j < chunks && key[q][j] >= T[q]) m = min(m, key[q][j]);
#pragma unroll
                for (int o = 32; o >= 1; o >>= 1) m = min(m, (uint32_t)__shfl_xor((int)m, o));
                T[q] = m;
                done[q] = true;
            }
        }
    }
    const uint64_t below = lanemask_lt();
#pragma unroll
    for (int q = 0; q < R; ++q) {
        if (!out[q]) continue;
        int gt = 0;
#pragma unroll
        for (int j = 0; j < KPL; ++j)
            if (j < chunks) gt += __popcll(__ballot(key[q][j] > T[q]));
        const int need = K - gt;  // keys equal to T still to take, lowest block index first
        int pos = 0, eq_seen = 0;
#pragma unroll
        for (int j = 0; j < KPL; ++j) {
            if (j < chunks) {
                const uint32_t kk = key[q][j];
                const uint64_t eqb = __ballot(kk == T[q]);
                const int eq_rank = eq_seen + __popcll(eqb & below);
                const bool sel = kk > T[q] || (kk == T[q] && eq_rank < need);
                const uint64_t sb = __ballot(sel);
                if (sel) out[q][pos + __popcll(sb & below)] = lane + 64 * j;
                pos += __popcll(sb);
                eq_seen += __popcll(eqb);
            }
        }
    }
}

// KPL > 0: the row is held in KPL registers per lane (M <= 64 * KPL).  KPL == 0: the row is
// re-read from memory on every pass (any M).
template <int KPL>
__global__ __launch_bounds__(256) void topk_rows_kernel(const float* __restrict__ S, int rows, int M, int K,
                                                        int32_t* __restrict__ idx) {
    const int lane = threadIdx.x & 63;
    const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (row >= rows) return;
    const float* Sr = S + (size_t)row * M;
    int32_t* const out[1] = {idx + (size_t)row * K};
    if constexpr (KPL > 0) {
        // every load is unconditional (from a clamped column) so that all of them are in flight
        // together; columns past the row end are then replaced by the padding key
        float f[KPL];
#pragma unroll
        for (int j = 0; j < KPL; ++j) f[j] = Sr[min(lane + 64 * j, M - 1)];
        uint32_t key[1][KPL];
#pragma unroll
        for (int j = 0; j < KPL; ++j) key[0][j] = lane + 64 * j < M ? score_key(f[j]) : 0u;
        topk_of_rows<KPL, 1>(key, KPL, K, out);
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
            if (sel) out[0][pos + __popcll(sb & below)] = lane + 64 * j;
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
    const dim3 sgrid((L.M + kGT - 1) / kGT, (L.M + kGT - 1) / kGT, L.BH);
    hipLaunchKernelGGL(block_scores_kernel, sgrid, dim3(256), 0, L.stream, q_mean, k_mean, L.M, L.M, L.d, L.scale,
                       scores);
    hipLaunchKernelGGL(tau_partial_kernel, dim3(kTauParts, L.BH), dim3(256), 0, L.stream, scores, L.M, partials);
    const int rows = L.BH * L.M;
    hipLaunchKernelGGL(tau_rows_kernel, dim3((rows + 3) / 4), dim3(256), 0, L.stream, scores, rows, L.M, tau,
                       partials, idx, counts, stats);
}

size_t select_workspace_bytes(const LaunchCtx& L) { return (size_t)L.BH * L.M * L.Mk * 4; }

void launch_select(const LaunchCtx& L, const float* q_mean, const float* k_mean, int32_t* idx, float* scores) {
    const dim3 sgrid((L.Mk + kGT - 1) / kGT, (L.M + kGT - 1) / kGT, L.BH);
    hipLaunchKernelGGL(block_scores_kernel, sgrid, dim3(256), 0, L.stream, q_mean, k_mean, L.M, L.Mk, L.d,
                       L.scale, scores);
    const int rows = L.BH * L.M;
    const dim3 tgrid((rows + 3) / 4);
    const int need = (L.Mk + 63) / 64;
#define SPARK_TOPK(KPL) \
    hipLaunchKernelGGL((topk_rows_kernel<KPL>), tgrid, dim3(256), 0, L.stream, scores, rows, L.Mk, L.K, idx)
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
