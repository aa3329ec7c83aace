/*
 * Oracle for two-branch block-sparse attention (Spark-Attn style) and for the Spark-Reblock
 * partition.  TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the benchmark's CPU
 * baseline load it; the library under test never does.  It shares no code with the HIP path.
 *
 * Plain and slow on purpose: every quantity is computed in binary64 straight from its
 * definition, one (batch, head, block) at a time, with no tiling, fusion or reordering.
 * OpenMP only distributes independent (batch, head, block) units over host cores.
 *
 * Sources (the pages):
 *  [SH3]  "Spark-H3: ブロックスパースアテンションでComfyUIのMiniMax-H3を高速化" (comfyui-wiki news,
 *         2026-10-11), section "Spark-Attnが変えるもの" (what Spark-Attn changes): the exact
 *         branch / compressed branch split, the Spark-Reblock bullet and the Spark-Reweight
 *         bullet; section "ワークフロー" (workflows): topk_mode=topk_ratio, reblock_layout=q_reuse_k.
 *  [CORE] "ComfyUI にコアのスパースアテンションノードと Comfy Compiler が追加されました" (comfyui-wiki
 *         news, 2026-09-08), section "ブロックスパースアテンション：1 つのノード、3 つのバックエンド":
 *         per-query-block routing, the top-k (SLA) fixed keep fraction, sink_conditioning.
 *  [H3O]  "H3 Optimizations" README, section "Nodes": non-video queries kept dense; section
 *         "Manual Sparse Sage recovery": the FP8 carrier of the FlexAttention fallback.
 *
 * Where the pages leave a step open, the reading taken is stated at the function.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

typedef struct {
    int B, H, N, d, n_sink, block;
    float topk_ratio;  /* fraction of key blocks kept per query block (a binary32 value) */
    int pool_mode;     /* 0: plain mean pool, 1: anchor-weighted summary + log-mass bias */
    double scale;      /* softmax scale; 0 means 1/sqrt(d) */
    int block_k;       /* key block size; 0 means the query block size `block` */
} orc_params;

static double scale_of(const orc_params *p) { return p->scale != 0.0 ? p->scale : 1.0 / sqrt((double)p->d); }
static int n_video(const orc_params *p) { return p->N - p->n_sink; }

int orc_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Threads used by later calls (for timing a single-core sample); no effect on any result. */
void orc_set_num_threads(int n)
{
#ifdef _OPENMP
    if (n > 0) omp_set_num_threads(n);
#else
    (void)n;
#endif
}

/* Query blocks M = ceil(N_v / block) and key blocks M_k = ceil(N_v / block_k); a last block may be
 * partial.  Reading of the asymmetric route [H3O, "Manual Sparse Sage recovery": the sparse
 * backends consume a 128Q x 64KV route]: query blocks of `block` rows are routed to key blocks
 * of `block_k` keys; pooling, scores, the budget and the compressed branch are per key block. */
static int key_block(const orc_params *p) { return p->block_k > 0 ? p->block_k : p->block; }
int orc_num_blocks(const orc_params *p) { return (n_video(p) + p->block - 1) / p->block; }
int orc_num_key_blocks(const orc_params *p) { return (n_video(p) + key_block(p) - 1) / key_block(p); }

/* Top-K budget from topk_mode=topk_ratio [SH3 "ワークフロー"], the fixed keep fraction of the
 * top-k mode [CORE]: K = floor(r*M + 1/2) in binary64, clamped to [1, M]. */
int orc_topk_count(int M, float ratio)
{
    double k = floor((double)ratio * (double)M + 0.5);
    if (k < 1.0) k = 1.0;
    if (k > (double)M) k = (double)M;
    return (int)k;
}

static int block_len(int Nv, int b, int J)
{
    int lo = J * b, hi = lo + b;
    if (hi > Nv) hi = Nv;
    return hi - lo;
}

static double dot_fd(const float *x, const double *y, int d)
{
    double s = 0.0;
    for (int c = 0; c < d; ++c) s += (double)x[c] * y[c];
    return s;
}

static double dot_ff(const float *x, const float *y, int d)
{
    double s = 0.0;
    for (int c = 0; c < d; ++c) s += (double)x[c] * (double)y[c];
    return s;
}

/*
 * Block pooling for one (batch, head).  X points at the N x d rows of that head, video rows
 * first.  Outputs (binary64):
 *   q_mean[M][d], k_mean[M][d]  per-block means of the video queries / keys;
 *   anchor[d]                    the mean of all video queries of the head [SH3, Reweight bullet:
 *                                one anchor per head, the video-query mean];
 *   k_sum[M][d], v_sum[M][d], bias[M]   the compressed summary of each key block.
 * Reweight reading [SH3, Reweight bullet]: with x_i = s * a.k_i over the block's keys, the
 * weights are the anchor's softmax inside the block, w_i = exp(x_i - m)/Z (m = max x, Z = sum
 * exp(x_i - m)); the summary is k~ = sum w_i k_i, v~ = sum w_i v_i, and the log-mass bias is
 * beta = m + ln Z - s * a.k~, so that exp(s*a.k~ + beta) is the block's exact mass at q = a.
 * Mean-pool reading: k~ = mean k, v~ = mean v, beta = ln n_J (the block stands for n_J tokens).
 */
static void pool_head(const orc_params *p, const float *Qh, const float *Kh, const float *Vh,
                      double *q_mean, double *k_mean, double *k_sum, double *v_sum,
                      double *bias, double *anchor)
{
    const int d = p->d, bq = p->block, b = key_block(p), Nv = n_video(p), Mq = orc_num_blocks(p);
    const int M = orc_num_key_blocks(p);
    const double s = scale_of(p);

    for (int c = 0; c < d; ++c) anchor[c] = 0.0;
    for (int i = 0; i < Nv; ++i)
        for (int c = 0; c < d; ++c) anchor[c] += (double)Qh[(size_t)i * d + c];
    for (int c = 0; c < d; ++c) anchor[c] /= (double)Nv;

    for (int I = 0; I < Mq; ++I) {
        const int lo = I * bq, n = block_len(Nv, bq, I);
        double *qm = q_mean + (size_t)I * d;
        for (int c = 0; c < d; ++c) {
            double sq = 0.0;
            for (int i = lo; i < lo + n; ++i) sq += (double)Qh[(size_t)i * d + c];
            qm[c] = sq / n;
        }
    }
    double *x = (double *)malloc(sizeof(double) * (size_t)b);
    for (int J = 0; J < M; ++J) {
        const int lo = J * b, n = block_len(Nv, b, J);
        double *km = k_mean + (size_t)J * d;
        double *ks = k_sum + (size_t)J * d, *vs = v_sum + (size_t)J * d;
        for (int c = 0; c < d; ++c) {
            double sk = 0.0;
            for (int i = lo; i < lo + n; ++i) sk += (double)Kh[(size_t)i * d + c];
            km[c] = sk / n;
        }
        if (p->pool_mode == 0) {
            for (int c = 0; c < d; ++c) {
                double sv = 0.0;
                for (int i = lo; i < lo + n; ++i) sv += (double)Vh[(size_t)i * d + c];
                ks[c] = km[c];
                vs[c] = sv / n;
            }
            bias[J] = log((double)n);
        } else {
            double m = -INFINITY;
            for (int t = 0; t < n; ++t) {
                x[t] = s * dot_fd(Kh + (size_t)(lo + t) * d, anchor, d);
                if (x[t] > m) m = x[t];
            }
            double Z = 0.0;
            for (int t = 0; t < n; ++t) Z += exp(x[t] - m);
            for (int c = 0; c < d; ++c) { ks[c] = 0.0; vs[c] = 0.0; }
            for (int t = 0; t < n; ++t) {
                const double w = exp(x[t] - m) / Z;
                for (int c = 0; c < d; ++c) {
                    ks[c] += w * (double)Kh[(size_t)(lo + t) * d + c];
                    vs[c] += w * (double)Vh[(size_t)(lo + t) * d + c];
                }
            }
            double ak = 0.0;
            for (int c = 0; c < d; ++c) ak += anchor[c] * ks[c];
            bias[J] = m + log(Z) - s * ak;
        }
    }
    free(x);
}

void orc_pool(const orc_params *p, const float *Q, const float *K, const float *V,
              double *q_mean, double *k_mean, double *k_sum, double *v_sum, double *bias,
              double *anchor)
{
    const int Mq = orc_num_blocks(p), M = orc_num_key_blocks(p), d = p->d;
    const size_t row = (size_t)p->N * d;
#pragma omp parallel for schedule(dynamic, 1)
    for (int bh = 0; bh < p->B * p->H; ++bh) {
        const size_t o = (size_t)bh * M * d;
        pool_head(p, Q + bh * row, K + bh * row, V + bh * row, q_mean + (size_t)bh * Mq * d, k_mean + o,
                  k_sum + o, v_sum + o, bias + (size_t)bh * M, anchor + (size_t)bh * d);
    }
}

/* Block scores S[I][J] = s * mean(q in I) . mean(k in J) for every (batch, head).  Reading: the
 * pages do not say how blocks are ranked; plain mean-pooled block scores are used, and the
 * ranking is shared by all queries of a block [CORE: each query block is routed to a subset of
 * key blocks]. */
void orc_scores(const orc_params *p, const double *q_mean, const double *k_mean, double *S)
{
    const int Mq = orc_num_blocks(p), M = orc_num_key_blocks(p), d = p->d;
    const double s = scale_of(p);
#pragma omp parallel for collapse(2) schedule(static)
    for (int bh = 0; bh < p->B * p->H; ++bh)
        for (int I = 0; I < Mq; ++I) {
            const double *qi = q_mean + ((size_t)bh * Mq + I) * d;
            for (int J = 0; J < M; ++J) {
                const double *kj = k_mean + ((size_t)bh * M + J) * d;
                double acc = 0.0;
                for (int c = 0; c < d; ++c) acc += qi[c] * kj[c];
                S[((size_t)bh * Mq + I) * M + J] = s * acc;
            }
        }
}

typedef struct { double key; int idx; } keyed;

/* descending score, then ascending block index */
static int cmp_score_desc(const void *a, const void *b)
{
    const keyed *x = (const keyed *)a, *y = (const keyed *)b;
    if (x->key > y->key) return -1;
    if (x->key < y->key) return 1;
    return (x->idx > y->idx) - (x->idx < y->idx);
}

static int cmp_int(const void *a, const void *b)
{
    const int x = *(const int *)a, y = *(const int *)b;
    return (x > y) - (x < y);
}

/* Top-K of one score row: order blocks by (score descending, index ascending), keep the first
 * K, return them in ascending index order. */
static void topk_row(const double *row, int M, int K, int32_t *out, keyed *tmp)
{
    for (int J = 0; J < M; ++J) { tmp[J].key = row[J]; tmp[J].idx = J; }
    qsort(tmp, (size_t)M, sizeof(keyed), cmp_score_desc);
    for (int k = 0; k < K; ++k) out[k] = tmp[k].idx;
    qsort(out, (size_t)K, sizeof(int32_t), cmp_int);
}

void orc_select(const orc_params *p, const double *S, int32_t *idx)
{
    const int Mq = orc_num_blocks(p), M = orc_num_key_blocks(p), K = orc_topk_count(M, p->topk_ratio);
#pragma omp parallel
    {
        keyed *tmp = (keyed *)malloc(sizeof(keyed) * (size_t)M);
#pragma omp for collapse(2) schedule(static)
        for (int bh = 0; bh < p->B * p->H; ++bh)
            for (int I = 0; I < Mq; ++I)
                topk_row(S + ((size_t)bh * Mq + I) * M, M, K, idx + ((size_t)bh * Mq + I) * K, tmp);
        free(tmp);
    }
}

/* softmax-weighted average of the given logits / value rows; writes out[d] and returns LSE */
typedef struct {
    int n;              /* logits collected */
    double *logit;      /* [cap] */
    const float **vf;   /* value row (float input) or NULL */
    const double **vd;  /* value row (binary64 summary) or NULL */
} logit_set;

static double finish_softmax(const logit_set *L, int d, double *out)
{
    double m = -INFINITY;
    for (int t = 0; t < L->n; ++t) if (L->logit[t] > m) m = L->logit[t];
    double Z = 0.0;
    for (int c = 0; c < d; ++c) out[c] = 0.0;
    for (int t = 0; t < L->n; ++t) {
        const double e = exp(L->logit[t] - m);
        Z += e;
        if (L->vf[t]) for (int c = 0; c < d; ++c) out[c] += e * (double)L->vf[t][c];
        else          for (int c = 0; c < d; ++c) out[c] += e * L->vd[t][c];
    }
    for (int c = 0; c < d; ++c) out[c] /= Z;
    return m + log(Z);
}

/*
 * Attention of the video queries of block I of one (batch, head).  Every query of the block
 * attends, in one softmax:
 *   - exactly to every key of its K selected blocks (the exact branch [SH3]);
 *   - exactly to every sink row [CORE: sink_conditioning attends packed conditioning rows
 *     exactly];
 *   - to one pseudo-key per unselected block J, logit s*q.k~_J + beta_J, value v~_J (the
 *     compressed branch [SH3]).
 * Reading: the compressed branch enters the same softmax as the exact branch, per query
 * token, so the two branches are merged by their log-sum-exp.
 */
static void attend_video_block(const orc_params *p, const float *Qh, const float *Kh,
                               const float *Vh, const double *k_sum, const double *v_sum,
                               const double *bias, const int32_t *sel, int K, int I,
                               double *Oh, double *lseh)
{
    const int d = p->d, bq = p->block, b = key_block(p), Nv = n_video(p), M = orc_num_key_blocks(p);
    const int N = p->N;
    const double s = scale_of(p);
    const int cap = K * b + p->n_sink + M;
    logit_set L;
    L.logit = (double *)malloc(sizeof(double) * (size_t)cap);
    L.vf = (const float **)malloc(sizeof(float *) * (size_t)cap);
    L.vd = (const double **)malloc(sizeof(double *) * (size_t)cap);
    char *chosen = (char *)calloc((size_t)M, 1);
    for (int k = 0; k < K; ++k) chosen[sel[k]] = 1;

    const int lo = I * bq, n = block_len(Nv, bq, I);
    for (int i = lo; i < lo + n; ++i) {
        const float *q = Qh + (size_t)i * d;
        L.n = 0;
        for (int k = 0; k < K; ++k) {
            const int J = sel[k], jlo = J * b, jn = block_len(Nv, b, J);
            for (int t = jlo; t < jlo + jn; ++t) {
                L.logit[L.n] = s * dot_ff(q, Kh + (size_t)t * d, d);
                L.vf[L.n] = Vh + (size_t)t * d; L.vd[L.n] = NULL; ++L.n;
            }
        }
        for (int t = Nv; t < N; ++t) {
            L.logit[L.n] = s * dot_ff(q, Kh + (size_t)t * d, d);
            L.vf[L.n] = Vh + (size_t)t * d; L.vd[L.n] = NULL; ++L.n;
        }
        for (int J = 0; J < M; ++J) {
            if (chosen[J]) continue;
            L.logit[L.n] = s * dot_fd(q, k_sum + (size_t)J * d, d) + bias[J];
            L.vf[L.n] = NULL; L.vd[L.n] = v_sum + (size_t)J * d; ++L.n;
        }
        lseh[i] = finish_softmax(&L, d, Oh + (size_t)i * d);
    }
    free(chosen); free(L.logit); free(L.vf); free(L.vd);
}

/* Non-video (sink) query rows attend densely to all N keys [H3O "Nodes": non-video queries
 * stay dense]. */
static void attend_dense_row(const orc_params *p, const float *Qh, const float *Kh,
                             const float *Vh, int i, double *Oh, double *lseh)
{
    const int d = p->d, N = p->N;
    const double s = scale_of(p);
    logit_set L;
    L.logit = (double *)malloc(sizeof(double) * (size_t)N);
    L.vf = (const float **)malloc(sizeof(float *) * (size_t)N);
    L.vd = (const double **)malloc(sizeof(double *) * (size_t)N);
    L.n = 0;
    for (int t = 0; t < N; ++t) {
        L.logit[L.n] = s * dot_ff(Qh + (size_t)i * d, Kh + (size_t)t * d, d);
        L.vf[L.n] = Vh + (size_t)t * d; L.vd[L.n] = NULL; ++L.n;
    }
    lseh[i] = finish_softmax(&L, d, Oh + (size_t)i * d);
    free(L.logit); free(L.vf); free(L.vd);
}

/* Dense softmax attention over all N keys, every row: the textbook operation the method reduces
 * to at full density or with one-token blocks. */
void orc_dense(const orc_params *p, const float *Q, const float *K, const float *V, double *O,
               double *lse)
{
    const size_t row = (size_t)p->N * p->d;
#pragma omp parallel for collapse(2) schedule(dynamic, 16)
    for (int bh = 0; bh < p->B * p->H; ++bh)
        for (int i = 0; i < p->N; ++i)
            attend_dense_row(p, Q + bh * row, K + bh * row, V + bh * row, i, O + bh * row,
                             lse + (size_t)bh * p->N);
}

/*
 * Attention for selected query blocks only (sampled parity at full size, and the CPU baseline).
 * Inputs are already in the block layout the route refers to (permuted when a partition is
 * used).  qb[n] = (bh, I) pairs: I < M is a video query block, I >= M is sink row N_v + (I - M).
 * Pooled key summaries (k_sum, v_sum, bias; M_k key blocks) and the route idx [B*H][M][K] are
 * full arrays.
 * O_out[n][rows][d] / lse_out[n][rows] receive the block's rows (rows = block, or 1 for a sink
 * row); rows past a partial block are left untouched.
 */
void orc_attend_blocks(const orc_params *p, const float *Q, const float *K, const float *V,
                       const double *k_sum, const double *v_sum, const double *bias,
                       const int32_t *idx, int Ksel, const int32_t *qb, int nqb, double *O_out,
                       double *lse_out)
{
    const int d = p->d, b = p->block, M = orc_num_blocks(p), Mk = orc_num_key_blocks(p), N = p->N;
    const size_t row = (size_t)N * d;
#pragma omp parallel
    {
        double *Oh = (double *)malloc(sizeof(double) * row);
        double *lh = (double *)malloc(sizeof(double) * (size_t)N);
#pragma omp for schedule(dynamic, 1)
        for (int n = 0; n < nqb; ++n) {
            const int bh = qb[2 * n], I = qb[2 * n + 1];
            const float *Qh = Q + bh * row, *Kh = K + bh * row, *Vh = V + bh * row;
            if (I < M) {
                attend_video_block(p, Qh, Kh, Vh, k_sum + (size_t)bh * Mk * d,
                                   v_sum + (size_t)bh * Mk * d, bias + (size_t)bh * Mk,
                                   idx + ((size_t)bh * M + I) * Ksel, Ksel, I, Oh, lh);
                const int lo = I * b, rows = block_len(n_video(p), b, I);
                memcpy(O_out + (size_t)n * b * d, Oh + (size_t)lo * d, sizeof(double) * (size_t)rows * d);
                memcpy(lse_out + (size_t)n * b, lh + lo, sizeof(double) * (size_t)rows);
            } else {
                const int i = n_video(p) + (I - M);
                attend_dense_row(p, Qh, Kh, Vh, i, Oh, lh);
                memcpy(O_out + (size_t)n * b * d, Oh + (size_t)i * d, sizeof(double) * d);
                lse_out[(size_t)n * b] = lh[i];
            }
        }
        free(Oh); free(lh);
    }
}

/* Gather the video rows of every (batch, head) by perm: new row p holds old row perm[p]; the
 * sink rows stay in place (reblock_layout=q_reuse_k [SH3 "ワークフロー"]: keys and values reuse
 * the query partition). */
static float *permute_rows(const orc_params *p, const float *X, const int32_t *perm)
{
    const int d = p->d, N = p->N, Nv = n_video(p);
    const size_t row = (size_t)N * d;
    float *Y = (float *)malloc(sizeof(float) * row * p->B * p->H);
    for (int bh = 0; bh < p->B * p->H; ++bh) {
        const float *x = X + bh * row;
        float *y = Y + bh * row;
        for (int q = 0; q < Nv; ++q)
            memcpy(y + (size_t)q * d, x + (size_t)perm[(size_t)bh * Nv + q] * d, sizeof(float) * d);
        memcpy(y + (size_t)Nv * d, x + (size_t)Nv * d, sizeof(float) * (size_t)(N - Nv) * d);
    }
    return Y;
}

/*
 * The whole forward: [gather by the partitions] -> pool -> scores -> top-K -> attention ->
 * [un-permute].
 *   perm     [B*H][N_v] or NULL: the query partition (query blocks, and the output rows);
 *   perm_k   [B*H][N_v] or NULL: a separate key partition for keys and values (key blocks and
 *            their summaries are then taken over the key leaves); NULL means keys and values reuse
 *            perm (reblock_layout=q_reuse_k [SH3 "ワークフロー"]);
 *   idx_in   [B*H][M][K] route to use instead of the oracle's own selection, or NULL;
 *   O [B,H,N,d], lse [B,H,N] binary64 outputs; idx_out [B*H][M][K] (may be NULL).
 */
void orc_forward(const orc_params *p, const float *Q, const float *K, const float *V,
                 const int32_t *perm, const int32_t *perm_k, const int32_t *idx_in, double *O,
                 double *lse, int32_t *idx_out)
{
    const int d = p->d, N = p->N, Nv = n_video(p), M = orc_num_blocks(p), Mk = orc_num_key_blocks(p);
    const int Ksel = orc_topk_count(Mk, p->topk_ratio);
    const size_t BH = (size_t)p->B * p->H, row = (size_t)N * d;
    const float *Qp = Q, *Kp = K, *Vp = V;
    float *tq = NULL, *tk = NULL, *tv = NULL;
    const int32_t *pk = perm_k ? perm_k : perm;
    if (perm) {
        tq = permute_rows(p, Q, perm);
        Qp = tq;
    }
    if (pk) {
        tk = permute_rows(p, K, pk); tv = permute_rows(p, V, pk);
        Kp = tk; Vp = tv;
    }
    double *qm = (double *)malloc(sizeof(double) * BH * M * d);
    double *km = (double *)malloc(sizeof(double) * BH * Mk * d);
    double *ks = (double *)malloc(sizeof(double) * BH * Mk * d);
    double *vs = (double *)malloc(sizeof(double) * BH * Mk * d);
    double *bias = (double *)malloc(sizeof(double) * BH * Mk);
    double *anc = (double *)malloc(sizeof(double) * BH * d);
    orc_pool(p, Qp, Kp, Vp, qm, km, ks, vs, bias, anc);
    int32_t *idx = (int32_t *)malloc(sizeof(int32_t) * BH * M * Ksel);
    if (idx_in) {
        memcpy(idx, idx_in, sizeof(int32_t) * BH * M * Ksel);
    } else {
        double *S = (double *)malloc(sizeof(double) * BH * M * Mk);
        orc_scores(p, qm, km, S);
        orc_select(p, S, idx);
        free(S);
    }
    if (idx_out) memcpy(idx_out, idx, sizeof(int32_t) * BH * M * Ksel);

    double *Op = (double *)malloc(sizeof(double) * BH * row);
    double *lp = (double *)malloc(sizeof(double) * BH * N);
#pragma omp parallel for collapse(2) schedule(dynamic, 1)
    for (int bh = 0; bh < (int)BH; ++bh)
        for (int I = 0; I < M + p->n_sink; ++I) {
            const float *Qh = Qp + bh * row, *Kh = Kp + bh * row, *Vh = Vp + bh * row;
            if (I < M)
                attend_video_block(p, Qh, Kh, Vh, ks + (size_t)bh * Mk * d, vs + (size_t)bh * Mk * d,
                                   bias + (size_t)bh * Mk, idx + ((size_t)bh * M + I) * Ksel, Ksel,
                                   I, Op + bh * row, lp + (size_t)bh * N);
            else
                attend_dense_row(p, Qh, Kh, Vh, Nv + (I - M), Op + bh * row, lp + (size_t)bh * N);
        }

    /* un-permute the video rows: O[perm[q]] = O'[q] */
    for (size_t bh = 0; bh < BH; ++bh) {
        for (int q = 0; q < Nv; ++q) {
            const int src = perm ? perm[bh * Nv + q] : q;
            memcpy(O + bh * row + (size_t)src * d, Op + bh * row + (size_t)q * d, sizeof(double) * d);
            lse[bh * N + src] = lp[bh * N + q];
        }
        memcpy(O + bh * row + (size_t)Nv * d, Op + bh * row + (size_t)Nv * d,
               sizeof(double) * (size_t)(N - Nv) * d);
        memcpy(lse + bh * N + Nv, lp + bh * N + Nv, sizeof(double) * (size_t)(N - Nv));
    }
    free(Op); free(lp); free(idx); free(qm); free(km); free(ks); free(vs); free(bias); free(anc);
    free(tq); free(tk); free(tv);
}

/* ------------------------------------------------------------------------------------------
 * Adaptive-tau selection [core node page, "ブロックスパースアテンション", Sol-Attn bullet]: a per-head
 * threshold placed in units of the spread of the head's score distribution, with no trained
 * weights.  Reading: over all M x M block scores S_IJ of a (batch, head), mu = their mean and
 * sigma = their population standard deviation (two passes); query block I keeps every key block J
 * with S_IJ > mu + tau * sigma (strictly), so a row may keep any number of blocks, none included
 * (its queries then see the compressed branch and the sinks only).  For Gaussian scores the kept
 * fraction is the normal tail: tau 1.0 / 1.5 / 2.0 keep about 15.9% / 6.7% / 2.3% of the blocks.
 *   S        [B*H][M][M] block scores (orc_scores);
 *   idx      [B*H][M][M]: row I lists its kept blocks ascending in its first counts[I] entries;
 *   counts   [B*H][M];  stats [B*H][2] = (mu, sigma), may be NULL.
 */
void orc_select_tau(const orc_params *p, double tau, const double *S, int32_t *idx, int32_t *counts,
                    double *stats)
{
    const int M = orc_num_blocks(p);
    const size_t MM = (size_t)M * M;
#pragma omp parallel for schedule(static)
    for (int bh = 0; bh < p->B * p->H; ++bh) {
        const double *Sh = S + (size_t)bh * MM;
        double sum = 0.0;
        for (size_t e = 0; e < MM; ++e) sum += Sh[e];
        const double mu = sum / (double)MM;
        double sq = 0.0;
        for (size_t e = 0; e < MM; ++e) sq += (Sh[e] - mu) * (Sh[e] - mu);
        const double sigma = sqrt(sq / (double)MM);
        const double thr = mu + tau * sigma;
        if (stats) { stats[2 * bh] = mu; stats[2 * bh + 1] = sigma; }
        for (int I = 0; I < M; ++I) {
            int32_t *row = idx + ((size_t)bh * M + I) * M;
            int c = 0;
            for (int J = 0; J < M; ++J)
                if (Sh[(size_t)I * M + J] > thr) row[c++] = J;
            counts[(size_t)bh * M + I] = c;
        }
    }
}

/*
 * The forward with adaptive-tau routes: pool -> scores -> tau selection -> attention.  Each video
 * query block attends exactly to its counts[I] kept blocks, to every sink, and to one pseudo-key
 * per other block, in one softmax; sink queries are dense.
 *   idx_in / counts_in: a route to use instead of the oracle's own selection, or NULL;
 *   idx_out [B*H][M][M], counts_out [B*H][M] (may be NULL).
 */
void orc_forward_tau(const orc_params *p, double tau, const float *Q, const float *K, const float *V,
                     const int32_t *idx_in, const int32_t *counts_in, double *O, double *lse,
                     int32_t *idx_out, int32_t *counts_out)
{
    const int d = p->d, N = p->N, Nv = n_video(p), M = orc_num_blocks(p);
    const size_t BH = (size_t)p->B * p->H, row = (size_t)N * d;
    double *qm = (double *)malloc(sizeof(double) * BH * M * d);
    double *km = (double *)malloc(sizeof(double) * BH * M * d);
    double *ks = (double *)malloc(sizeof(double) * BH * M * d);
    double *vs = (double *)malloc(sizeof(double) * BH * M * d);
    double *bias = (double *)malloc(sizeof(double) * BH * M);
    double *anc = (double *)malloc(sizeof(double) * BH * d);
    orc_pool(p, Q, K, V, qm, km, ks, vs, bias, anc);
    int32_t *idx = (int32_t *)malloc(sizeof(int32_t) * BH * M * M);
    int32_t *cnt = (int32_t *)malloc(sizeof(int32_t) * BH * M);
    if (idx_in && counts_in) {
        memcpy(idx, idx_in, sizeof(int32_t) * BH * M * M);
        memcpy(cnt, counts_in, sizeof(int32_t) * BH * M);
    } else {
        double *S = (double *)malloc(sizeof(double) * BH * M * M);
        orc_scores(p, qm, km, S);
        orc_select_tau(p, tau, S, idx, cnt, NULL);
        free(S);
    }
    if (idx_out) memcpy(idx_out, idx, sizeof(int32_t) * BH * M * M);
    if (counts_out) memcpy(counts_out, cnt, sizeof(int32_t) * BH * M);
#pragma omp parallel for collapse(2) schedule(dynamic, 1)
    for (int bh = 0; bh < (int)BH; ++bh)
        for (int I = 0; I < M + p->n_sink; ++I) {
            const float *Qh = Q + bh * row, *Kh = K + bh * row, *Vh = V + bh * row;
            if (I < M)
                attend_video_block(p, Qh, Kh, Vh, ks + (size_t)bh * M * d, vs + (size_t)bh * M * d,
                                   bias + (size_t)bh * M, idx + ((size_t)bh * M + I) * M,
                                   cnt[(size_t)bh * M + I], I, O + bh * row, lse + (size_t)bh * N);
            else
                attend_dense_row(p, Qh, Kh, Vh, Nv + (I - M), O + bh * row, lse + (size_t)bh * N);
        }
    free(idx); free(cnt); free(qm); free(km); free(ks); free(vs); free(bias); free(anc);
}

/* ------------------------------------------------------------------------------------------
 * FP8 exact branch [H3O, section "Manual Sparse Sage recovery", the FP8 FlexAttention fallback]:
 * Q, K and V are carried as E4M3 with one scale per head, the Q/K scale is restored before the
 * softmax, the output returns in the original floating type, and the route is the same.
 * Readings:
 *  - E4M3 is the OCP 8-bit float with 4 exponent bits (bias 7) and 3 mantissa bits: normal
 *    values 2^(e-7) (1 + m/8), subnormal spacing 2^-9, largest finite value 448.  A value goes to
 *    the nearest representable one, ties to an even mantissa.
 *  - Per (batch, head) and per tensor, amax = max |x| over all N rows (video and sinks); in
 *    binary32, r = 448 / amax and s = amax / 448 (both 1 when amax = 0).  The carrier of x is
 *    e4m3(x * r), the product rounded to binary32 first.
 *  - The compressed pseudo-keys (k~, v~) travel with the keys' and values' scales: a convex
 *    combination of a block's rows stays inside their range.  Their binary64 summaries are
 *    rounded to binary32 before the scaling.  The bias beta and the route come from the
 *    unquantized inputs, exactly as in the plain forward.
 *  - Every logit is s_att * s_Q * s_K * (q8 . k8), plus beta for a pseudo-key; every value is
 *    s_V * v8.  The softmax itself is exact (binary64).
 */

/* E4M3 rounding of x (the value, as binary32).  Magnitudes that round above 448 are outside the
 * format: NaN. */
float orc_e4m3(float x)
{
    if (x == 0.0f || isnan(x)) return x;
    const double a = fabs((double)x);
    int e;
    (void)frexp(a, &e);       /* a = f 2^e with f in [1/2, 1): the leading bit is 2^(e-1) */
    int lead = e - 1;
    if (lead < -6) lead = -6; /* below the smallest normal binade the spacing stays 2^-9 */
    const double q = ldexp(1.0, lead - 3);
    const double y = rint(a / q) * q; /* a / q is exact; rint rounds ties to even */
    if (y > 448.0) return NAN;
    return (float)(x < 0.0f ? -y : y);
}

void orc_e4m3_array(const float *x, float *y, size_t n)
{
    for (size_t i = 0; i < n; ++i) y[i] = orc_e4m3(x[i]);
}

/* Per (batch, head): scales[6] = r_Q, s_Q, r_K, s_K, r_V, s_V (binary32). */
void orc_fp8_scales(const orc_params *p, const float *Q, const float *K, const float *V, float *scales)
{
    const size_t row = (size_t)p->N * p->d;
    for (int bh = 0; bh < p->B * p->H; ++bh) {
        const float *X[3] = {Q + bh * row, K + bh * row, V + bh * row};
        for (int t = 0; t < 3; ++t) {
            float amax = 0.0f;
            for (size_t e = 0; e < row; ++e) amax = fmaxf(amax, fabsf(X[t][e]));
            float r = 1.0f, sc = 1.0f;
            if (amax > 0.0f) {
                r = 448.0f / amax;
                sc = amax / 448.0f;
            }
            scales[(size_t)bh * 6 + 2 * t] = r;
            scales[(size_t)bh * 6 + 2 * t + 1] = sc;
        }
    }
}

/* The forward of orc_forward (reblock_layout=q_reuse_k when perm is given) with the exact branch,
 * the sinks and the pseudo-keys on E4M3 carriers.  scales_out [B*H][6] may be NULL. */
void orc_forward_fp8(const orc_params *p, const float *Q, const float *K, const float *V,
                     const int32_t *perm, const int32_t *idx_in, double *O, double *lse,
                     int32_t *idx_out, float *scales_out)
{
    const int d = p->d, N = p->N, Nv = n_video(p), M = orc_num_blocks(p), Mk = orc_num_key_blocks(p);
    const int Ksel = orc_topk_count(Mk, p->topk_ratio);
    const size_t BH = (size_t)p->B * p->H, row = (size_t)N * d;
    const float *Qp = Q, *Kp = K, *Vp = V;
    float *tq = NULL, *tk = NULL, *tv = NULL;
    if (perm) {
        tq = permute_rows(p, Q, perm); tk = permute_rows(p, K, perm); tv = permute_rows(p, V, perm);
        Qp = tq; Kp = tk; Vp = tv;
    }
    double *qm = (double *)malloc(sizeof(double) * BH * M * d);
    double *km = (double *)malloc(sizeof(double) * BH * Mk * d);
    double *ks = (double *)malloc(sizeof(double) * BH * Mk * d);
    double *vs = (double *)malloc(sizeof(double) * BH * Mk * d);
    double *bias = (double *)malloc(sizeof(double) * BH * Mk);
    double *anc = (double *)malloc(sizeof(double) * BH * d);
    orc_pool(p, Qp, Kp, Vp, qm, km, ks, vs, bias, anc);
    int32_t *idx = (int32_t *)malloc(sizeof(int32_t) * BH * M * Ksel);
    if (idx_in) {
        memcpy(idx, idx_in, sizeof(int32_t) * BH * M * Ksel);
    } else {
        double *S = (double *)malloc(sizeof(double) * BH * M * Mk);
        orc_scores(p, qm, km, S);
        orc_select(p, S, idx);
        free(S);
    }
    if (idx_out) memcpy(idx_out, idx, sizeof(int32_t) * BH * M * Ksel);

    /* carriers, held as their (exact) binary32 / binary64 values */
    float *sc = (float *)malloc(sizeof(float) * BH * 6);
    orc_fp8_scales(p, Qp, Kp, Vp, sc);
    if (scales_out) memcpy(scales_out, sc, sizeof(float) * BH * 6);
    float *q8 = (float *)malloc(sizeof(float) * BH * row);
    float *k8 = (float *)malloc(sizeof(float) * BH * row);
    float *v8 = (float *)malloc(sizeof(float) * BH * row);
    double *ks8 = (double *)malloc(sizeof(double) * BH * Mk * d);
    double *vs8 = (double *)malloc(sizeof(double) * BH * Mk * d);
    for (size_t bh = 0; bh < BH; ++bh) {
        const float *s6 = sc + bh * 6;
        for (size_t e = 0; e < row; ++e) {
            q8[bh * row + e] = orc_e4m3(Qp[bh * row + e] * s6[0]);
            k8[bh * row + e] = orc_e4m3(Kp[bh * row + e] * s6[2]);
            v8[bh * row + e] = orc_e4m3(Vp[bh * row + e] * s6[4]);
        }
        for (size_t e = 0; e < (size_t)Mk * d; ++e) {
            ks8[bh * Mk * d + e] = (double)orc_e4m3((float)ks[bh * Mk * d + e] * s6[2]);
            vs8[bh * Mk * d + e] = (double)orc_e4m3((float)vs[bh * Mk * d + e] * s6[4]);
        }
    }

    double *Op = (double *)malloc(sizeof(double) * BH * row);
    double *lp = (double *)malloc(sizeof(double) * BH * N);
#pragma omp parallel for collapse(2) schedule(dynamic, 1)
    for (int bh = 0; bh < (int)BH; ++bh)
        for (int I = 0; I < M + p->n_sink; ++I) {
            orc_params ph = *p;
            ph.scale = scale_of(p) * (double)sc[(size_t)bh * 6 + 1] * (double)sc[(size_t)bh * 6 + 3];
            const float *Qh = q8 + bh * row, *Kh = k8 + bh * row, *Vh = v8 + bh * row;
            if (I < M)
                attend_video_block(&ph, Qh, Kh, Vh, ks8 + (size_t)bh * Mk * d, vs8 + (size_t)bh * Mk * d,
                                   bias + (size_t)bh * Mk, idx + ((size_t)bh * M + I) * Ksel, Ksel,
                                   I, Op + bh * row, lp + (size_t)bh * N);
            else
                attend_dense_row(&ph, Qh, Kh, Vh, Nv + (I - M), Op + bh * row, lp + (size_t)bh * N);
        }

    /* values restored by s_V; video rows un-permuted: O[perm[q]] = O'[q] */
    for (size_t bh = 0; bh < BH; ++bh) {
        const double sV = (double)sc[bh * 6 + 5];
        for (size_t e = 0; e < row; ++e) Op[bh * row + e] *= sV;
        for (int q = 0; q < Nv; ++q) {
            const int src = perm ? perm[bh * Nv + q] : q;
            memcpy(O + bh * row + (size_t)src * d, Op + bh * row + (size_t)q * d, sizeof(double) * d);
            lse[bh * N + src] = lp[bh * N + q];
        }
        memcpy(O + bh * row + (size_t)Nv * d, Op + bh * row + (size_t)Nv * d,
               sizeof(double) * (size_t)(N - Nv) * d);
        memcpy(lse + bh * N + Nv, lp + bh * N + Nv, sizeof(double) * (size_t)(N - Nv));
    }
    free(Op); free(lp); free(idx); free(qm); free(km); free(ks); free(vs); free(bias); free(anc);
    free(sc); free(q8); free(k8); free(v8); free(ks8); free(vs8);
    free(tq); free(tk); free(tv);
}

/* ------------------------------------------------------------------------------------------
 * Spark-Reblock [SH3, Reblock bullet]: two queries are alike when their score patterns against
 * the keys are alike, measured by the cosine under the metric of the keys' second moment; a
 * hierarchical partitioner keeps splitting groups until every leaf holds the block size, in
 * O(N log N).  Readings (the pages give no formulas):
 *   R1  Sigma = K^T K / N_v over the video keys of the head (uncentred second moment), summed
 *       exactly in fixed point: with max|k| < 2^E (E from frexp) and s = 21 - E, every key entry
 *       becomes the integer k^ = rint(k * 2^s) (ties to even; |k^| <= 2^21, and k^ = k * 2^s exactly
 *       for entries within 13 binades of the maximum when the keys are bf16), the products
 *       k^_ia * k^_ib are added in int64 (no overflow for N_v <= 2^20), and
 *       Sigma_ab = ((double)sum * 2^(-2s)) / N_v.
 *   R2  t(i) = Sigma q_i with t_a = fma(Sigma_ab, q_ib, t_a) for b = 0..d-1 from 0;
 *       r_i = fma(q_ia, t_a(i), r_i) for a = 0..d-1 from 0; n_i = sqrt(r_i) if r_i > 0 else 0.
 *   R3  Groups carry a leaf count c: one group of all N_v video tokens with c = M to start.
 *   R4  A group with c > 1 splits.  P0 = its lowest token index; g(P) = t(P) / n_P (0 if
 *       n_P = 0); cos(i, P) = (fma chain over a of q_ia * g_a(P)) / n_i (0 if n_i = 0).
 *       A = argmin_i cos(i, P0), B = argmin_i cos(i, A) (ties: lower index);
 *       key_i = cos(i, A) - cos(i, B).  Ordered by (key descending, index ascending), the
 *       first ceil(c/2)*block tokens form the left child (ceil(c/2) leaves), the rest the right
 *       child (floor(c/2) leaves; it keeps the partial remainder).
 *   R5  Children split in turn until c = 1.
 *   R6  perm lists the leaves left to right; inside a leaf, ascending token index.
 * All binary64 arithmetic above is single IEEE operations in a fixed order (this file is built
 * with -ffp-contract=off), so the result is fixed bit for bit.
 * ---------------------------------------------------------------------------------------- */

/* R1 for one head; Kh points at its video rows. */
static void reblock_sigma(const float *Kh, int Nv, int d, double *Sigma)
{
    double mx = 0.0;
    for (size_t i = 0; i < (size_t)Nv * d; ++i) {
        const double a = fabs((double)Kh[i]);
        if (a > mx) mx = a;
    }
    if (mx == 0.0) { memset(Sigma, 0, sizeof(double) * (size_t)d * d); return; }
    int E;
    frexp(mx, &E); /* mx = f * 2^E with f in [0.5, 1), so mx < 2^E */
    const int sh = 21 - E;
    for (int a = 0; a < d; ++a)
        for (int c = 0; c < d; ++c) {
            int64_t acc = 0;
            for (int i = 0; i < Nv; ++i) {
                const int64_t ka = (int64_t)rint(ldexp((double)Kh[(size_t)i * d + a], sh));
                const int64_t kc = (int64_t)rint(ldexp((double)Kh[(size_t)i * d + c], sh));
                acc += ka * kc;
            }
            Sigma[(size_t)a * d + c] = ldexp((double)acc, -2 * sh) / (double)Nv;
        }
}

/* t = Sigma q (R2's fma chain) */
static void sigma_times(const double *Sigma, const float *q, int d, double *t)
{
    for (int a = 0; a < d; ++a) {
        double acc = 0.0;
        for (int c = 0; c < d; ++c) acc = fma(Sigma[(size_t)a * d + c], (double)q[c], acc);
        t[a] = acc;
    }
}

typedef struct {
    const float *Qh;
    const double *Sigma;
    const double *nrm;
    int d, block;
    double *g, *cosA, *cosB;  /* scratch: g[d], cos values [N_v] */
    keyed *tmp;               /* [N_v] */
    int *leaf;                /* leaf id per token */
} rb_ctx;

static double cos_to(const rb_ctx *x, int i, const double *g)
{
    if (x->nrm[i] == 0.0) return 0.0;
    const float *q = x->Qh + (size_t)i * x->d;
    double acc = 0.0;
    for (int a = 0; a < x->d; ++a) acc = fma((double)q[a], g[a], acc);
    return acc / x->nrm[i];
}

static void pivot_dir(const rb_ctx *x, int P, double *g)
{
    if (x->nrm[P] == 0.0) { for (int a = 0; a < x->d; ++a) g[a] = 0.0; return; }
    sigma_times(x->Sigma, x->Qh + (size_t)P * x->d, x->d, g);
    for (int a = 0; a < x->d; ++a) g[a] = g[a] / x->nrm[P];
}

/* argmin over the group's tokens of cos(i, g); ties to the lower index; cos values into out */
static int argmin_cos(const rb_ctx *x, const int *tok, int n, const double *g, double *out)
{
    int best = -1;
    double bv = 0.0;
    for (int k = 0; k < n; ++k) {
        const int i = tok[k];
        const double c = cos_to(x, i, g);
        out[i] = c;
        if (best < 0 || c < bv || (c == bv && i < best)) { best = i; bv = c; }
    }
    return best;
}

static void reblock_split(rb_ctx *x, int *tok, int n, int c, int leaf0)
{
    if (c == 1) {
        for (int k = 0; k < n; ++k) x->leaf[tok[k]] = leaf0;
        return;
    }
    int P0 = tok[0];
    for (int k = 1; k < n; ++k) if (tok[k] < P0) P0 = tok[k];
    pivot_dir(x, P0, x->g);
    const int A = argmin_cos(x, tok, n, x->g, x->cosB);
    pivot_dir(x, A, x->g);
    const int Bp = argmin_cos(x, tok, n, x->g, x->cosA);
    pivot_dir(x, Bp, x->g);
    for (int k = 0; k < n; ++k) x->cosB[tok[k]] = cos_to(x, tok[k], x->g);
    for (int k = 0; k < n; ++k) {
        const int i = tok[k];
        x->tmp[k].key = x->cosA[i] - x->cosB[i];
        x->tmp[k].idx = i;
    }
    qsort(x->tmp, (size_t)n, sizeof(keyed), cmp_score_desc);
    for (int k = 0; k < n; ++k) tok[k] = x->tmp[k].idx;
    const int cl = (c + 1) / 2, nl = cl * x->block;
    reblock_split(x, tok, nl, cl, leaf0);
    reblock_split(x, tok + nl, n - nl, c - cl, leaf0 + cl);
}

/* R2 for every video query of one head, from that head's Sigma. */
static void reblock_norms(const float *Qh, int Nv, int d, const double *Sg, double *nrm)
{
    double *t = (double *)malloc(sizeof(double) * d);
    for (int i = 0; i < Nv; ++i) {
        const float *q = Qh + (size_t)i * d;
        sigma_times(Sg, q, d, t);
        double r = 0.0;
        for (int a = 0; a < d; ++a) r = fma((double)q[a], t[a], r);
        nrm[i] = r > 0.0 ? sqrt(r) : 0.0;
    }
    free(t);
}

/* Exposed for tests: Sigma [B*H][d][d] and norms [B*H][N_v]. */
void orc_reblock_metric(const orc_params *p, const float *Q, const float *K, double *Sigma,
                        double *nrm)
{
    const int d = p->d, Nv = n_video(p);
    const size_t row = (size_t)p->N * d;
#pragma omp parallel for schedule(dynamic, 1)
    for (int bh = 0; bh < p->B * p->H; ++bh) {
        double *Sg = Sigma + (size_t)bh * d * d;
        reblock_sigma(K + bh * row, Nv, d, Sg);
        reblock_norms(Q + bh * row, Nv, d, Sg, nrm + (size_t)bh * Nv);
    }
}

/* R2..R6 for every (batch, head) from the given Sigma [B*H][d][d]. */
static void reblock_from_sigma(const orc_params *p, const float *Q, const double *Sigma, int32_t *perm)
{
    const int d = p->d, Nv = n_video(p), M = orc_num_blocks(p), b = p->block;
    const size_t row = (size_t)p->N * d, BH = (size_t)p->B * p->H;
    double *nrm = (double *)malloc(sizeof(double) * BH * Nv);
#pragma omp parallel for schedule(dynamic, 1)
    for (int bh = 0; bh < (int)BH; ++bh)
        reblock_norms(Q + bh * row, Nv, d, Sigma + (size_t)bh * d * d, nrm + (size_t)bh * Nv);
#pragma omp parallel for schedule(dynamic, 1)
    for (int bh = 0; bh < (int)BH; ++bh) {
        rb_ctx x;
        x.Qh = Q + bh * row; x.Sigma = Sigma + (size_t)bh * d * d; x.nrm = nrm + (size_t)bh * Nv;
        x.d = d; x.block = b;
        x.g = (double *)malloc(sizeof(double) * d);
        x.cosA = (double *)malloc(sizeof(double) * Nv);
        x.cosB = (double *)malloc(sizeof(double) * Nv);
        x.tmp = (keyed *)malloc(sizeof(keyed) * Nv);
        x.leaf = (int *)malloc(sizeof(int) * Nv);
        int *tok = (int *)malloc(sizeof(int) * Nv);
        for (int i = 0; i < Nv; ++i) tok[i] = i;
        reblock_split(&x, tok, Nv, M, 0);
        /* R6: leaves in order, ascending token index inside each leaf */
        int *fill = (int *)calloc((size_t)M, sizeof(int));
        int32_t *pr = perm + (size_t)bh * Nv;
        for (int i = 0; i < Nv; ++i) {
            const int L = x.leaf[i];
            pr[(size_t)L * b + fill[L]++] = i;
        }
        free(fill); free(tok); free(x.g); free(x.cosA); free(x.cosB); free(x.tmp); free(x.leaf);
    }
    free(nrm);
}

/* perm [B*H][N_v]: position q of the reblocked layout holds token perm[q]. */
void orc_reblock(const orc_params *p, const float *Q, const float *K, int32_t *perm)
{
    const int d = p->d, Nv = n_video(p);
    const size_t row = (size_t)p->N * d, BH = (size_t)p->B * p->H;
    double *Sigma = (double *)malloc(sizeof(double) * BH * d * d);
#pragma omp parallel for schedule(dynamic, 1)
    for (int bh = 0; bh < (int)BH; ++bh) reblock_sigma(K + bh * row, Nv, d, Sigma + (size_t)bh * d * d);
    reblock_from_sigma(p, Q, Sigma, perm);
    free(Sigma);
}

/* Exposed for tests: R2..R6 from a caller's Sigma [B*H][d][d] in place of R1's (to measure how the
 * partition depends on the reading of Sigma). */
void orc_reblock_given_sigma(const orc_params *p, const float *Q, const double *Sigma, int32_t *perm)
{
    reblock_from_sigma(p, Q, Sigma, perm);
}
