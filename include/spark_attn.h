/*
 * spark_attn.h — C ABI of a gfx950 (MI355X) library for two-branch block-sparse video attention
 * in the Spark-Attn style, forward only.
 *
 * The method (from the pages it is built from):
 *  - Spark-H3 news page ("Spark-H3: ブロックスパースアテンションでComfyUIのMiniMax-H3を高速化",
 *    comfyui-wiki, 2026-10-11), section "Spark-Attnが変えるもの" (what Spark-Attn changes):
 *    attention over video tokens is split into an exact branch over the top-ranked key/value
 *    blocks and a compressed branch covering the remaining blocks; the Spark-Reweight bullet
 *    replaces the compressed branch's mean-pooled key/value with a summary weighted at one
 *    anchor per head (the mean video query) plus a log-mass bias; the Spark-Reblock bullet
 *    replaces fixed raster tiles by a hierarchical partition under a cosine measured in the
 *    metric of the other side's second moment.  Section "ワークフロー" (workflows): the budget
 *    is topk_mode=topk_ratio and keys reuse the query partition (reblock_layout=q_reuse_k).
 *  - Core sparse-attention node page ("ComfyUI にコアのスパースアテンションノードと Comfy Compiler
 *    が追加されました", comfyui-wiki, 2026-09-08), section "ブロックスパースアテンション：1 つの
 *    ノード、3 つのバックエンド": every query block is routed to a subset of key blocks (top-k
 *    keeps a fixed fraction of key blocks); sink_conditioning attends packed conditioning rows
 *    exactly.
 *  - "H3 Optimizations" README, section "Nodes": non-video queries stay dense; an explicitly
 *    requested sparse backend that cannot run is an error, never a silent fallback.
 *
 * Conventions shared by every call
 *  - Tensors are contiguous [B, H, N, d] (row = one token of one (batch, head)).  Rows
 *    [0, N_v) are video tokens, rows [N_v, N) with N_v = N - n_sink are sink (conditioning)
 *    rows.  Video rows are cut into M = ceil(N_v / block) blocks of `block` consecutive rows;
 *    the last block may be shorter.  Blocks never include sink rows.
 *  - Every pointer is a DEVICE pointer owned by the caller, 16-byte aligned.  The library
 *    never allocates, frees or synchronises; all work is enqueued on `stream` (a hipStream_t
 *    passed as void*, NULL = the null stream).  It keeps no state between calls.
 *  - Return value: SPARK_ATTN_OK or a negative status.  Arguments are validated before any
 *    work is enqueued, so an error return means nothing was launched (except
 *    SPARK_ATTN_HIP_ERROR, which reports a failed launch).  Faults inside kernels surface at
 *    the caller's next synchronisation.
 *  - There is no fallback: an unsupported shape or dtype returns SPARK_ATTN_UNSUPPORTED.
 *  - Supported: d in {64, 128}; block in {64, 128}; dtype bf16 or fp32 (fp32 inputs are
 *    pooled and ranked in fp32 and rounded to bf16 for the matrix-core stages); M <= 16384;
 *    B*H*N*d < 2^31.
 */
#ifndef SPARK_ATTN_H
#define SPARK_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum spark_attn_status {
    SPARK_ATTN_OK = 0,
    SPARK_ATTN_INVALID_ARGUMENT = -1,   /* null required pointer, bad size, ratio outside (0,1] */
    SPARK_ATTN_UNSUPPORTED = -2,        /* d, block, dtype or size outside the supported set */
    SPARK_ATTN_WORKSPACE_TOO_SMALL = -3,
    SPARK_ATTN_HIP_ERROR = -4,          /* a kernel launch failed */
    SPARK_ATTN_MISALIGNED = -5,         /* a pointer is not 16-byte aligned */
    SPARK_ATTN_SCRATCH_TOO_SMALL = -6   /* the problem exceeds the library's static scratch */
};

enum spark_attn_dtype { SPARK_ATTN_BF16 = 0, SPARK_ATTN_FP32 = 1 };
enum spark_attn_pool_mode { SPARK_ATTN_POOL_MEAN = 0, SPARK_ATTN_POOL_REWEIGHT = 1 };

typedef struct {
    int B, H;          /* batch, heads */
    int N;             /* rows per (batch, head): video rows followed by n_sink sink rows */
    int d;             /* head dimension */
    int n_sink;        /* sink rows at the tail of every (batch, head), 0 <= n_sink < N */
    int block;         /* query block size (and key block size when block_k is 0) */
    float topk_ratio;  /* kept fraction of key blocks, in (0, 1]; K = clamp(floor(r*M_k + 1/2), 1,
                          M_k) evaluated in binary64 from this binary32 value */
    int pool_mode;     /* spark_attn_pool_mode */
    int dtype;         /* spark_attn_dtype of Q, K, V and O */
    float scale;       /* softmax scale s; 0 means 1/sqrt(d) */
    int block_k;       /* key block size; 0 means `block`.  The asymmetric route (H3 Optimizations
                          README, "Manual Sparse Sage recovery": the sparse backends consume a
                          128Q x 64KV route): query blocks of `block` rows are routed to key blocks
                          of `block_k` keys; key summaries, scores' columns, the budget and the
                          compressed branch are per key block.  Adaptive tau needs block_k =
                          block; reblock leaves are query blocks. */
} spark_attn_params;

/* ---- host-only helpers (no GPU needed) ---------------------------------------------------- */

/* M = ceil(N_v / block) query blocks, or a negative status for invalid params. */
int spark_attn_num_blocks(const spark_attn_params *p);
/* M_k = ceil(N_v / block_k) key blocks (M when block_k is 0 or block), or a negative status. */
int spark_attn_num_key_blocks(const spark_attn_params *p);

/* Top-K budget of topk_mode=topk_ratio: clamp(floor(ratio*M + 0.5), 1, M) in binary64.
 * Returns a negative status if M < 1 or ratio is outside (0, 1]. */
int spark_attn_topk_count(int M, float ratio);

/* Bytes of device workspace a call needs, or 0 for invalid params:
 *   what = 0: spark_attn_forward without perm;  what = 2: spark_attn_forward with perm (or
 *             spark_attn_forward_kv with either partition);
 *   what = 1: spark_attn_reblock;               what = 3: spark_attn_select without `scores`;
 *   what = 4: the packed key/value tiles of spark_attn_pack / spark_attn_attend;
 *   what = 5: spark_attn_select_tau;            what = 6: spark_attn_forward_tau;
 *   what = 7: spark_attn_forward_fp8 without perm; what = 8: spark_attn_forward_fp8 with perm;
 *   what = 9: the packed E4M3 tiles of spark_attn_pack_fp8 / spark_attn_attend_fp8. */
size_t spark_attn_workspace_size(const spark_attn_params *p, int what);

/* Static description of a status code. */
const char *spark_attn_status_str(int status);

/* ---- device calls --------------------------------------------------------------------------- */

/*
 * Block pooling (Spark-H3 page, "Spark-Attnが変えるもの", Spark-Reweight bullet).
 * In:  Q, K, V [B,H,N,d] in p->dtype.
 * Out (fp32, caller-allocated):
 *   q_mean, k_mean [B,H,M,d]  per-block means of video queries / keys (used for ranking);
 *   anchor [B,H,d]            mean of all video queries of the (batch, head);
 *   k_sum, v_sum [B,H,M,d]    compressed summary of each key block;
 *   bias [B,H,M]              its log-mass bias.
 * pool_mode REWEIGHT: with x_i = s*anchor.k_i over the block's keys, w = softmax(x) inside the
 *   block, k_sum = sum w_i k_i, v_sum = sum w_i v_i, bias = logsumexp(x) - s*anchor.k_sum, so that
 *   exp(s*anchor.k_sum + bias) equals the block's exact attention mass at the anchor.
 * pool_mode MEAN: k_sum = mean k, v_sum = mean v, bias = ln(block length).
 */
int spark_attn_pool(const spark_attn_params *p, const void *Q, const void *K, const void *V,
                    float *q_mean, float *k_mean, float *k_sum, float *v_sum, float *bias,
                    float *anchor, void *stream);

/*
 * Top-K key-block selection per query block (core node page, "ブロックスパースアテンション":
 * route each query block to a subset of key blocks; top-k keeps a fixed fraction).
 * In:  q_mean, k_mean [B,H,M,d] fp32 (from spark_attn_pool).
 * Out: idx [B,H,M,K] int32: for query block I, the K key blocks J with the largest block scores
 *      S_IJ = s * q_mean_I . k_mean_J (fp32), ties to the lower J, listed in ascending J.
 *      scores [B,H,M,M] fp32, optional: receives S.  When NULL, S is kept in `workspace`, which
 *      must then hold spark_attn_workspace_size(p, 3) bytes (ignored otherwise).
 */
int spark_attn_select(const spark_attn_params *p, const float *q_mean, const float *k_mean,
                      int32_t *idx, float *scores, void *workspace, size_t ws_bytes, void *stream);

/*
 * spark_attn_select without a workspace, for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid allocation).  The same
 * kernels and the same route as spark_attn_select with scores = NULL; the score matrix lives in
 * a static scratch array the library holds on each device until the process ends
 * (SPARK_ATTN_NOALLOC_SCRATCH_BYTES, 64 MiB: up to 16,777,216 scores, B*H*M*M_k; the 720p
 * workload, 24 x 591 x 591, takes 33.5 MB).  The scratch of a device is looked up once, on the
 * first call made with that device current; pass a stream of the current device.
 * In:  q_mean, k_mean as for spark_attn_select.  Out: idx [B,H,M,K] as for spark_attn_select.
 * Errors: as spark_attn_select; SPARK_ATTN_SCRATCH_TOO_SMALL (nothing launched) when
 * B*H*M*M_k*4 exceeds the scratch; SPARK_ATTN_HIP_ERROR when the scratch cannot be located.
 * Calls that overlap on one device (different streams, or threads) share the scratch and race;
 * calls on one stream are ordered and safe.  The entry point allocates and frees nothing.
 */
#define SPARK_ATTN_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
int spark_attn_select_noalloc(const spark_attn_params *p, const float *q_mean, const float *k_mean,
                              int32_t *idx, void *stream);

/*
 * Packing of the keys and values the attention stage reads.  `packed` (device memory of at least
 * spark_attn_workspace_size(p, 4) bytes, caller-owned) receives, per (batch, head), 64-key tiles of
 * bf16 K rows and transposed V for the video keys, the sink keys and the compressed pseudo-keys
 * (k_sum / v_sum rows), plus one fp32 additive logit row per tile (log2 units: 0 for real keys,
 * log2(e) * bias for pseudo-keys, -inf for padding).  The layout is private to the library: fill it
 * with this call, read it with spark_attn_attend.
 * In:  K, V [B,H,N,d] in p->dtype; k_sum, v_sum [B,H,M,d], bias [B,H,M] fp32 (spark_attn_pool).
 */
int spark_attn_pack(const spark_attn_params *p, const void *K, const void *V, const float *k_sum,
                    const float *v_sum, const float *bias, void *packed, size_t packed_bytes,
                    void *stream);

/*
 * spark_attn_pool followed by spark_attn_pack, with K and V read from memory once: the kernel
 * that pools a key block also writes its packed tiles (same outputs, same layout, same values).
 * Arguments as in those two calls; every pointer is required.  Error behaviour as theirs:
 * SPARK_ATTN_INVALID_ARGUMENT for a NULL pointer, SPARK_ATTN_MISALIGNED, and
 * SPARK_ATTN_WORKSPACE_TOO_SMALL when packed_bytes < spark_attn_workspace_size(p, 4).
 */
int spark_attn_pool_pack(const spark_attn_params *p, const void *Q, const void *K, const void *V,
                         float *q_mean, float *k_mean, float *k_sum, float *v_sum, float *bias,
                         float *anchor, void *packed, size_t packed_bytes, void *stream);

/*
 * The attention stage (exact branch + sinks + compressed branch, one softmax).
 * In:  Q [B,H,N,d] (in the block layout idx refers to); packed (spark_attn_pack of the matching
 *      K, V and summaries); idx [B,H,M,K] int32, distinct entries in [0, M) per row.
 *      perm [B,H,N_v] int32 or NULL: when given, output row q of the video part is written to
 *      row perm[q] of O and lse (undoing a partition).
 * Out: O [B,H,N,d] in p->dtype; lse [B,H,N] fp32 (natural log), optional.
 * Video query i of block I attends in one softmax to every key of its K selected blocks, to
 * every sink row, and to one pseudo-key per unselected block J (logit s*q.k_sum_J + bias_J,
 * value v_sum_J).  Sink query rows attend densely to all N keys.
 * The call also writes a small region at the end of `packed` that the library keeps for itself
 * (a flag per query tile and eight tile counters): calls that share one packed buffer must not
 * overlap in time; the tiles themselves are only read.
 */
int spark_attn_attend(const spark_attn_params *p, const void *Q, const void *packed,
                      size_t packed_bytes, const int32_t *idx, const int32_t *perm, void *O,
                      float *lse, void *stream);

/*
 * Adaptive-tau selection (core node page, "ブロックスパースアテンション", Sol-Attn bullet: a
 * per-head threshold placed in sigma units of the score distribution, no trained weights).
 * Over the M x M block scores S_IJ = s * q_mean_I . k_mean_J (fp32) of each (batch, head):
 * mu = their mean and sigma = their population standard deviation (binary64, fixed summation
 * order); query block I keeps every key block J with S_IJ > mu + tau * sigma, so the number of
 * kept blocks varies per query block (none is allowed).
 * In:  tau (finite); q_mean, k_mean [B,H,M,d] fp32 (from spark_attn_pool).
 * Out: idx [B,H,M,M] int32: row I lists its kept blocks in ascending order in its first counts[I]
 *      entries (the rest are left as they were); counts [B,H,M] int32; stats [B,H,2] fp32 =
 *      (mu, sigma) per (batch, head), or NULL.
 * workspace: at least spark_attn_workspace_size(p, 5) bytes.
 */
int spark_attn_select_tau(const spark_attn_params *p, float tau, const float *q_mean,
                          const float *k_mean, int32_t *idx, int32_t *counts, float *stats,
                          void *workspace, size_t ws_bytes, void *stream);

/*
 * The attention stage with a variable route (as spark_attn_attend otherwise): query block I
 * attends exactly to the counts[I] blocks listed in row I of idx [B,H,M,M], to every sink, and
 * to one pseudo-key per other block.  counts [B,H,M] int32 in [0, M]; perm as in
 * spark_attn_attend or NULL.
 */
int spark_attn_attend_var(const spark_attn_params *p, const void *Q, const void *packed,
                          size_t packed_bytes, const int32_t *idx, const int32_t *counts,
                          const int32_t *perm, void *O, float *lse, void *stream);

/*
 * The forward with adaptive-tau routes: pool -> spark_attn_select_tau -> pack -> attend, in
 * token order.  Out: O, lse (or NULL) as spark_attn_forward; idx_out [B,H,M,M] and counts_out
 * [B,H,M] (each may be NULL): the route used.  workspace: spark_attn_workspace_size(p, 6) bytes.
 */
int spark_attn_forward_tau(const spark_attn_params *p, float tau, const void *Q, const void *K,
                           const void *V, void *O, float *lse, int32_t *idx_out,
                           int32_t *counts_out, void *workspace, size_t ws_bytes, void *stream);

/*
 * The whole forward: [gather rows by perm] -> pool -> select -> pack -> attend (-> un-permute).
 * In:  Q, K, V [B,H,N,d] in p->dtype; perm [B,H,N_v] int32 or NULL (a permutation of [0,N_v)
 *      per (batch, head), e.g. from spark_attn_reblock: block layout row q holds token perm[q];
 *      keys and values reuse it).
 * Out: O [B,H,N,d] in p->dtype (original token order); lse [B,H,N] fp32 or NULL;
 *      idx_out [B,H,M,K] int32 or NULL: the route used (in the permuted block layout).
 * workspace: device memory of at least spark_attn_workspace_size(p, perm ? 2 : 0) bytes.
 */
int spark_attn_forward(const spark_attn_params *p, const void *Q, const void *K, const void *V,
                       const int32_t *perm, void *O, float *lse, int32_t *idx_out,
                       void *workspace, size_t ws_bytes, void *stream);

/*
 * The forward with a separate key partition (Spark-H3 page, Spark-Reblock bullet: each side is
 * partitioned in the metric of the opposite side's second moment; "ワークフロー":
 * reblock_layout=q_reuse_k is the layout where keys reuse the query partition, this call is the
 * other one).  Query blocks and the output rows follow perm_q; key blocks, their compressed
 * summaries and the values follow perm_k.  A key partition is spark_attn_reblock called with
 * the roles exchanged: (p, K, Q, perm_k, ...), keys bisected under Sigma_Q = Q^T Q / N_v.
 * In:  Q, K, V [B,H,N,d] in p->dtype; perm_q, perm_k [B,H,N_v] int32, each NULL or a permutation
 *      of [0,N_v) per (batch, head) (row q of the block layout holds token perm[q]).
 * Out: as spark_attn_forward (O and lse in the original token order, idx_out in the block
 *      layouts: query block I of the perm_q order routed to key blocks of the perm_k order).
 * workspace: at least spark_attn_workspace_size(p, (perm_q || perm_k) ? 2 : 0) bytes.
 * spark_attn_forward(p, Q, K, V, perm, ...) equals spark_attn_forward_kv(p, Q, K, V, perm, perm, ...).
 */
int spark_attn_forward_kv(const spark_attn_params *p, const void *Q, const void *K, const void *V,
                          const int32_t *perm_q, const int32_t *perm_k, void *O, float *lse,
                          int32_t *idx_out, void *workspace, size_t ws_bytes, void *stream);

/*
 * Spark-Reblock partition (Spark-H3 page, "Spark-Attnが変えるもの", Spark-Reblock bullet) of the
 * video queries of every (batch, head), with the metric Sigma = K^T K / N_v of the video keys:
 *  - Sigma is summed exactly in 64-bit fixed point; n_i = sqrt(q_i^T Sigma q_i);
 *  - a group holding c leaves splits (c > 1): pivot P0 = its lowest token; A = the token with
 *    the smallest Sigma-cosine to P0, B = the one with the smallest to A (ties: lower index);
 *    tokens ordered by cos(.,A) - cos(.,B) descending (then index ascending); the first
 *    ceil(c/2)*block tokens form the left child, the rest the right child;
 *  - perm lists leaves left to right, each leaf in ascending token order.
 * All decisions are taken in binary64 with a fixed operation order, so the result is exact and
 * reproducible.
 * In:  Q, K [B,H,N,d] (only video rows are read).
 * Out: perm [B,H,N_v] int32.
 * workspace: at least spark_attn_workspace_size(p, 1) bytes.
 */
int spark_attn_reblock(const spark_attn_params *p, const void *Q, const void *K, int32_t *perm,
                       void *workspace, size_t ws_bytes, void *stream);

/*
 * FP8 carriers (H3 Optimizations README, section "Manual Sparse Sage recovery": the FP8
 * FlexAttention fallback stores Q/K/V as per-head-scaled E4M3, restores the Q/K scale before the
 * softmax, returns the output in the original floating type and consumes the same route).
 * E4M3 is the OCP 8-bit float (4 exponent bits, bias 7, 3 mantissa bits, largest value 448).
 * Per (batch, head) and tensor, amax = max |x| over all N rows; r = 448/amax and s = amax/448
 * (binary32, both 1 when amax = 0); the carrier of x is e4m3(x * r), rounded to nearest even.
 * Keys' and values' scales also carry the compressed pseudo-keys.  Every logit is
 * scale * s_Q * s_K * (q8 . k8) (+ the pseudo-key bias), every value s_V * v8; the probabilities
 * are rounded to E4M3 for the value product, the normaliser sums them unrounded.
 *
 * spark_attn_fp8_scales: amax [B,H,3] fp32 (Q, K, V), written with atomics after a clear.
 * spark_attn_pool_fp8_scales: spark_attn_pool and spark_attn_fp8_scales with Q, K, V read once
 *   (the pooling kernels take the maxima of the video rows); the same outputs, every pointer
 *   required.
 * spark_attn_pack_fp8: the tiles of spark_attn_pack on E4M3 carriers (same tile list and fp32
 *   bias rows; a tile is 64 key rows of d bytes, then d value rows of 64 bytes); `packed` holds
 *   spark_attn_workspace_size(p, 9) bytes.
 * spark_attn_attend_fp8: spark_attn_attend on those tiles; idx [B,H,M,K] (ascending rows), perm as
 *   in spark_attn_attend; amax as written by spark_attn_fp8_scales for the same Q, K, V.  Like
 *   spark_attn_attend it writes eight tile counters the library keeps at the end of `packed`:
 *   calls that share one packed buffer must not overlap in time.
 * spark_attn_forward_fp8: [gather by perm] -> pool+scales -> select -> pack_fp8 -> attend_fp8;
 *   pooling and selection see the unquantized inputs (the route equals spark_attn_forward's);
 *   amax_out [B,H,3] or NULL; workspace of spark_attn_workspace_size(p, perm ? 8 : 7) bytes.
 * Errors and ownership as for the bf16 calls; every pointer is device memory.
 */
int spark_attn_fp8_scales(const spark_attn_params *p, const void *Q, const void *K, const void *V,
                          float *amax, void *stream);
int spark_attn_pool_fp8_scales(const spark_attn_params *p, const void *Q, const void *K,
                               const void *V, float *q_mean, float *k_mean, float *k_sum,
                               float *v_sum, float *bias, float *anchor, float *amax, void *stream);
int spark_attn_pack_fp8(const spark_attn_params *p, const void *K, const void *V, const float *k_sum,
                        const float *v_sum, const float *bias, const float *amax, void *packed,
                        size_t packed_bytes, void *stream);
int spark_attn_attend_fp8(const spark_attn_params *p, const void *Q, const void *packed,
                          size_t packed_bytes, const int32_t *idx, const int32_t *perm,
                          const float *amax, void *O, float *lse, void *stream);
int spark_attn_forward_fp8(const spark_attn_params *p, const void *Q, const void *K, const void *V,
                           const int32_t *perm, void *O, float *lse, int32_t *idx_out,
                           float *amax_out, void *workspace, size_t ws_bytes, void *stream);

/*
 * Row gather used for the q_reuse_k layout: for every (batch, head), Y row q = X row perm[q]
 * for q < N_v; sink rows are copied unchanged.  X, Y [B,H,N,d] in p->dtype, distinct buffers.
 */
int spark_attn_gather_rows(const spark_attn_params *p, const void *X, const int32_t *perm,
                           void *Y, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* SPARK_ATTN_H */
