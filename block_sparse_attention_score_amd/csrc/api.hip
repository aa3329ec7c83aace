// C ABI of the library: argument validation, workspace layout and the launch sequence on the
// caller's stream.  No allocation, no synchronisation, no fallback path.
#include <math.h>
#include <string.h>

#include <mutex>

#include "kernels.hpp"

// Scratch of spark_attn_select_noalloc: the score matrix, in a static device array each device
// holds until the process ends.  In host code `scratch` is only a stand-in for the symbol: its
// device address (per device) comes from hipGetSymbolAddress, and only that address is used.
static __device__ __align__(256) unsigned char scratch[SPARK_ATTN_NOALLOC_SCRATCH_BYTES];

namespace spark {

static bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

static int topk_count(int M, float ratio) {
    if (M < 1 || !(ratio > 0.f) || !(ratio <= 1.f)) return SPARK_ATTN_INVALID_ARGUMENT;
    double k = floor((double)ratio * (double)M + 0.5);
    if (k < 1.0) k = 1.0;
    if (k > (double)M) k = (double)M;
    return (int)k;
}

static int make_ctx(const spark_attn_params* p, void* stream, LaunchCtx* L) {
    if (!p) return SPARK_ATTN_INVALID_ARGUMENT;
    if (p->B < 1 || p->H < 1 || p->N < 1 || p->n_sink < 0 || p->n_sink >= p->N || p->block < 1 || p->d < 1)
        return SPARK_ATTN_INVALID_ARGUMENT;
    if (!(p->topk_ratio > 0.f) || !(p->topk_ratio <= 1.f)) return SPARK_ATTN_INVALID_ARGUMENT;
    if (p->pool_mode != SPARK_ATTN_POOL_MEAN && p->pool_mode != SPARK_ATTN_POOL_REWEIGHT)
        return SPARK_ATTN_INVALID_ARGUMENT;
    if (!(p->scale >= 0.f) || isinf(p->scale)) return SPARK_ATTN_INVALID_ARGUMENT;
    if (p->d != 64 && p->d != 128) return SPARK_ATTN_UNSUPPORTED;
    if (p->block != 64 && p->block != 128) return SPARK_ATTN_UNSUPPORTED;
    if (p->block_k < 0) return SPARK_ATTN_INVALID_ARGUMENT;
    if (p->block_k != 0 && p->block_k != 64 && p->block_k != 128) return SPARK_ATTN_UNSUPPORTED;
    if (p->dtype != SPARK_ATTN_BF16 && p->dtype != SPARK_ATTN_FP32) return SPARK_ATTN_UNSUPPORTED;
    const long long elems = (long long)p->B * p->H * p->N * p->d;
    if (elems >= (1LL << 31)) return SPARK_ATTN_UNSUPPORTED;
    L->B = p->B;
    L->H = p->H;
    L->BH = p->B * p->H;
    L->N = p->N;
    L->n_sink = p->n_sink;
    L->Nv = p->N - p->n_sink;
    L->d = p->d;
    L->block = p->block;
    L->M = (L->Nv + p->block - 1) / p->block;
    L->block_k = p->block_k ? p->block_k : p->block;
    L->Mk = (L->Nv + L->block_k - 1) / L->block_k;
    if (L->M > kMaxBlocks || L->Mk > kMaxBlocks) return SPARK_ATTN_UNSUPPORTED;
    L->K = topk_count(L->Mk, p->topk_ratio);
    L->pool_mode = p->pool_mode;
    L->dtype = p->dtype;
    L->scale = p->scale != 0.f ? p->scale : 1.0f / sqrtf((float)p->d);
    L->stream = (hipStream_t)stream;
    return SPARK_ATTN_OK;
}

// Device address of `scratch` on the current device, looked up once per device.
constexpr int kMaxDevices = 64;
static std::once_flag g_scratch_once[kMaxDevices];
static void* g_scratch_ptr[kMaxDevices];
static hipError_t g_scratch_err[kMaxDevices];

static int scratch_on_current_device(void** out) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return SPARK_ATTN_HIP_ERROR;
    if (dev < 0 || dev >= kMaxDevices) return SPARK_ATTN_UNSUPPORTED;
    std::call_once(g_scratch_once[dev], [dev] {
        g_scratch_err[dev] = hipGetSymbolAddress(&g_scratch_ptr[dev], HIP_SYMBOL(scratch));
    });
    if (g_scratch_err[dev] != hipSuccess || !g_scratch_ptr[dev]) return SPARK_ATTN_HIP_ERROR;
    *out = g_scratch_ptr[dev];
    return SPARK_ATTN_OK;
}

static int launch_status() {
    const hipError_t e = hipGetLastError();
    return e == hipSuccess ? SPARK_ATTN_OK : SPARK_ATTN_HIP_ERROR;
}

struct FwdWorkspace {
    size_t q_mean, k_mean, k_sum, v_sum, bias, anchor, idx, scores, packed, qp, kp, vp, total;
};

static FwdWorkspace fwd_layout(const LaunchCtx& L, bool with_perm) {
    FwdWorkspace w;
    const size_t md = (size_t)L.BH * L.M * L.d * 4, mkd = (size_t)L.BH * L.Mk * L.d * 4;
    size_t o = 0;
    w.q_mean = o; o = align256(o + md);
    w.k_mean = o; o = align256(o + mkd);
    w.k_sum = o; o = align256(o + mkd);
    w.v_sum = o; o = align256(o + mkd);
    w.bias = o; o = align256(o + (size_t)L.BH * L.Mk * 4);
    w.anchor = o; o = align256(o + (size_t)L.BH * L.d * 4);
    w.idx = o; o = align256(o + (size_t)L.BH * L.M * L.K * 4);
    w.scores = o; o = align256(o + select_workspace_bytes(L));
    w.packed = o; o = align256(o + pack_geom(L).bytes);
    w.qp = w.kp = w.vp = 0;
    if (with_perm) {
        const size_t x = (size_t)L.BH * L.N * L.d * (L.dtype == SPARK_ATTN_BF16 ? 2 : 4);
        w.qp = o; o = align256(o + x);
        w.kp = o; o = align256(o + x);
        w.vp = o; o = align256(o + x);
    }
    w.total = o;
    return w;
}

// workspace of spark_attn_select_tau: the score matrix, then the per-head partial sums
static size_t tau_select_bytes(const LaunchCtx& L) {
    return align256(select_workspace_bytes(L)) + tau_partials_bytes(L);
}

struct TauWorkspace {
    size_t q_mean, k_mean, k_sum, v_sum, bias, anchor, idx, counts, scores, partials, packed, total;
};

static TauWorkspace tau_layout(const LaunchCtx& L) {
    TauWorkspace w;
    const size_t md = (size_t)L.BH * L.M * L.d * 4;
    size_t o = 0;
    w.q_mean = o; o = align256(o + md);
    w.k_mean = o; o = align256(o + md);
    w.k_sum = o; o = align256(o + md);
    w.v_sum = o; o = align256(o + md);
    w.bias = o; o = align256(o + (size_t)L.BH * L.M * 4);
    w.anchor = o; o = align256(o + (size_t)L.BH * L.d * 4);
    w.idx = o; o = align256(o + (size_t)L.BH * L.M * L.M * 4);
    w.counts = o; o = align256(o + (size_t)L.BH * L.M * 4);
    w.scores = o; o = align256(o + select_workspace_bytes(L));
    w.partials = o; o = align256(o + tau_partials_bytes(L));
    w.packed = o; o = align256(o + pack_geom(L).bytes);
    w.total = o;
    return w;
}

struct Fp8Workspace {
    size_t q_mean, k_mean, k_sum, v_sum, bias, anchor, idx, scores, amax, packed, qp, kp, vp, total;
};

static Fp8Workspace fp8_layout(const LaunchCtx& L, bool with_perm) {
    Fp8Workspace w;
    const size_t md = (size_t)L.BH * L.M * L.d * 4, mkd = (size_t)L.BH * L.Mk * L.d * 4;
    size_t o = 0;
    w.q_mean = o; o = align256(o + md);
    w.k_mean = o; o = align256(o + mkd);
    w.k_sum = o; o = align256(o + mkd);
    w.v_sum = o; o = align256(o + mkd);
    w.bias = o; o = align256(o + (size_t)L.BH * L.Mk * 4);
    w.anchor = o; o = align256(o + (size_t)L.BH * L.d * 4);
    w.idx = o; o = align256(o + (size_t)L.BH * L.M * L.K * 4);
    w.scores = o; o = align256(o + select_workspace_bytes(L));
    w.amax = o; o = align256(o + (size_t)L.BH * 3 * 4);
    w.packed = o; o = align256(o + pack_geom_fp8(L).bytes);
    w.qp = w.kp = w.vp = 0;
    if (with_perm) {
        const size_t x = (size_t)L.BH * L.N * L.d * (L.dtype == SPARK_ATTN_BF16 ? 2 : 4);
        w.qp = o; o = align256(o + x);
        w.kp = o; o = align256(o + x);
        w.vp = o; o = align256(o + x);
    }
    w.total = o;
    return w;
}

}  // namespace spark

using namespace spark;

extern "C" {

int spark_attn_num_blocks(const spark_attn_params* p) {
    LaunchCtx L;
    const int s = make_ctx(p, nullptr, &L);
    return s < 0 ? s : L.M;
}

int spark_attn_num_key_blocks(const spark_attn_params* p) {
    LaunchCtx L;
    const int s = make_ctx(p, nullptr, &L);
    return s < 0 ? s : L.Mk;
}

int spark_attn_topk_count(int M, float ratio) { return topk_count(M, ratio); }

size_t spark_attn_workspace_size(const spark_attn_params* p, int what) {
    LaunchCtx L;
    if (make_ctx(p, nullptr, &L) < 0) return 0;
    if (what == 1) return reblock_workspace_bytes(L);
    if (what == 0 || what == 2) return fwd_layout(L, what == 2).total;
    if (what == 3) return select_workspace_bytes(L);
    if (what == 4) return pack_geom(L).bytes;
    if (what == 5) return tau_select_bytes(L);
    if (what == 6) return tau_layout(L).total;
    if (what == 7 || what == 8) return fp8_layout(L, what == 8).total;
    if (what == 9) return pack_geom_fp8(L).bytes;
    return 0;
}

const char* spark_attn_status_str(int status) {
    switch (status) {
        case SPARK_ATTN_OK: return "ok";
        case SPARK_ATTN_INVALID_ARGUMENT: return "invalid argument";
        case SPARK_ATTN_UNSUPPORTED: return "unsupported shape or dtype";
        case SPARK_ATTN_WORKSPACE_TOO_SMALL: return "workspace too small";
        case SPARK_ATTN_HIP_ERROR: return "HIP launch error";
        case SPARK_ATTN_MISALIGNED: return "pointer not 16-byte aligned";
        case SPARK_ATTN_SCRATCH_TOO_SMALL: return "problem exceeds the library's static scratch";
        default: return "unknown status";
    }
}

int spark_attn_pool(const spark_attn_params* p, const void* Q, const void* K, const void* V, float* q_mean,
                    float* k_mean, float* k_sum, float* v_sum, float* bias, float* anchor, void* stream) {
    LaunchCtx L;
    int s = make_ctx(p, stream, &L);
    if (s < 0) return s;
    if (!Q || !K || !V || !q_mean || !k_mean || !k_sum || !v_sum || !bias || !anchor)
        return SPARK_ATTN_INVALID_ARGUMENT;
    if (!aligned16(Q) || !aligned16(K) || !aligned16(V) || !aligned16(q_mean) || !aligned16(k_mean) ||
        !aligned16(k_sum) || !aligned16(v_sum) || !aligned16(anchor))
        return SPARK_ATTN_MISALIGNED;
    launch_pool(L, Q, K, V, q_mean, k_mean, k_sum, v_sum, bias, anchor);
    return launch_status();
}

int spark_attn_select(const spark_attn_params* p, const float* q_mean, const float* k_mean, int32_t* idx,
                      float* scores, void* workspace, size_t ws_bytes, void* stream) {
    LaunchCtx L;
    int s = make_ctx(p, stream, &L);
    if (s < 0) return s;
    if (!q_mean || !k_mean || !idx) return SPARK_ATTN_INVALID_ARGUMENT;
    if (!aligned16(q_mean) || !aligned16(k_mean) || !aligned16(scores) || !aligned16(workspace))
        return SPARK_ATTN_MISALIGNED;
    float* S = scores;
    if (!S) {
        if (!workspace || ws_bytes < select_workspace_bytes(L)) return SPARK_ATTN_WORKSPACE_TOO_SMALL;
        S = (float*)workspace;
    }
    launch_select(L, q_mean, k_mean, idx, S);
    return launch_status();
}

int spark_attn_select_noalloc(const spark_attn_params* p, const float* q_mean, const float* k_mean,
                              int32_t* idx, void* stream) {
    LaunchCtx L;
    int s = make_ctx(p, stream, &L);
    if (s < 0) return s;
    if (!q_mean || !k_mean || !idx) return SPARK_ATTN_INVALID_ARGUMENT;
    if (!aligned16(q_mean) || !aligned16(k_mean)) return SPARK_ATTN_MISALIGNED;
    if (select_workspace_bytes(L) > SPARK_ATTN_NOALLOC_SCRATCH_BYTES) return SPARK_ATTN_SCRATCH_TOO_SMALL;
    void* ws = nullptr;
    s = scratch_on_current_device(&ws);
    if (s < 0) return s;
    launch_select(L, q_mean, k_mean, idx, (float*)ws);
    return launch_status();
}

int spark_attn_pack(const spark_attn_params* p, const void* K, const void* V, const float* k_sum, const float* v_sum,
                    const float* bias, void* packed, size_t packed_bytes, void* stream) {
    LaunchCtx L;
    int s = make_ctx(p, stream, &L);
    if (s < 0) return s;
    if (!K || !V || !k_sum || !v_sum || !bias) return SPARK_ATTN_INVALID_ARGUMENT;
    if (!aligned16(K) || !aligned16(V) || !aligned16(k_sum) || !aligned16(v_sum) || !aligned16(packed))
        return SPARK_ATTN_MISALIGNED;
    if (!packed || packed_bytes < pack_geom(L).bytes) return SPARK_ATTN_WORKSPACE_TOO_SMALL;
    launch_pack(L, K, V, k_sum, v_sum, bias, packed);
    return launch_status();
}

int spark_attn_pool_pack(const spark_attn_params* p, const void* Q, const void* K, const void* V, float* q_mean,
                         float* k_mean, float* k_sum, float* v_sum, float* bias, float* anchor, void* packed,
                         size_t packed_bytes, void* stream) {
    LaunchCtx L;
    int s = make_ctx(p, stream, &L);
    if (s < 0) return s;
    if (!Q || !K || !V || !q_mean || !k_mean || !k_sum || !v_sum || !bias || !anchor)
        return SPARK_ATTN_INVALID_ARGUMENT;
    if (!aligned16(Q) || !aligned16(K) || !aligned16(V) || !aligned16(q_mean) || !aligned16(k_mean) ||
        !aligned16(k_sum) || !aligned16(v_sum) || !aligned16(anchor) || !aligned16(packed))
        return SPARK_ATTN_MISALIGNED;
    if (!packed || packed_bytes < pack_geom(L).bytes) return SPARK_ATTN_WORKSPACE_TOO_SMALL;
    launch_pool_pack(L, Q, K, V, q_mean, k_mean, k_sum, v_sum, bias, anchor, packed);
    return launch_status();
}

int spark_attn_attend(const spark_attn_params* p, const void* Q, const void* packed, size_t packed_bytes,
                      const int32_t* idx, const int32_t* perm, void* O, float* lse, void* stream) {
    LaunchCtx L;
    int s = make_ctx(p, stream, &L);
    if (s < 0) return s;
    if (!Q || !idx || !O) return SPARK_ATTN_INVALID_ARGUMENT;
    if (!aligned16(Q) || !aligned16(packed) || !aligned16(O)) return SPARK_ATTN_MISALIGNED;
    if (!packed || packed_bytes < pack_geom(L).bytes) return SPARK_ATTN_WORKSPACE_TOO_SMALL;
    launch_attend(L, Q, packed, idx, nullptr, perm, O, lse);
    return launch_status();
}

int spark_attn_attend_var(const spark_attn_params* p, const void* Q, const void* packed, size_t packed_bytes,
                          const int32_t* idx, const int32_t* counts, const int32_t* perm, void* O, float* lse,
                          void* stream) {
    LaunchCtx L;
    int s = make_ctx(p, stream, &L);
    if (s < 0) return s;
    if (L.Mk != L.M) return SPARK_ATTN_UNSUPPORTED;  // adaptive tau: equal query and key blocks
    if (!Q || !idx || !counts || !O) return SPARK_ATTN_INVALID_ARGUMENT;
    if (!aligned16(Q) || !aligned16(packed) || !aligned16(O)) return SPARK_ATTN_MISALIGNED;
    if (!packed || packed_bytes < pack_geom(L).bytes) return SPARK_ATTN_WORKSPACE_TOO_SMALL;
    launch_attend(L, Q, packed, idx, counts, perm, O, lse);
    return launch_status();
}

int spark_attn_select_tau(const spark_attn_params* p, float tau, const float* q_mean, const float* k_mean,
                          int32_t* idx, int32_t* counts, float* stats, void* workspace, size_t ws_bytes,
                          void* stream) {
    LaunchCtx L;
    int s = make_ctx(p, stream, &L);
    if (s < 0) return s;
    if (L.Mk != L.M) return SPARK_ATTN_UNSUPPORTED;  // adaptive tau: equal query and key blocks
    if (!(tau == tau) || tau == INFINITY || tau == -INFINITY) return SPARK_ATTN_INVALID_ARGUMENT;
    if (!q_mean || !k_mean || !idx || !counts) return SPARK_ATTN_INVALID_ARGUMENT;
    if (!aligned16(q_mean) || !aligned16(k_mean) || !aligned16(workspace)) return SPARK_ATTN_MISALIGNED;
    if (!workspace || ws_bytes < tau_select_bytes(L)) return SPARK_ATTN_WORKSPACE_TOO_SMALL;
    char* ws = (char*)workspace;
    launch_select_tau(L, tau, q_mean, k_mean, idx, counts, stats, (float*)ws,
                      (double*)(ws + align256(select_workspace_bytes(L))));
    return launch_status();
}

int spark_attn_forward_tau(const spark_attn_params* p, float tau, const void* Q, const void* K, const void* V,
                           void* O, float* lse, int32_t* idx_out, int32_t* counts_out, void* workspace,
                           size_t ws_bytes, void* stream) {
    LaunchCtx L;
    int s = make_ctx(p, stream, &L);
    if (s < 0) return s;
    if (L.Mk != L.M) return SPARK_ATTN_UNSUPPORTED;  // adaptive tau: equal query and key blocks
    if (!(tau == tau) || tau == INFINITY || tau == -INFINITY) return SPARK_ATTN_INVALID_ARGUMENT;
    if (!Q || !K || !V || !O) return SPARK_ATTN_INVALID_ARGUMENT;
    if (!aligned16(Q) || !aligned16(K) || !aligned16(V) || !aligned16(O) || !aligned16(workspace))
        return SPARK_ATTN_MISALIGNED;
    const TauWorkspace w = tau_layout(L);
    if (!workspace || ws_bytes < w.total) return SPARK_ATTN_WORKSPACE_TOO_SMALL;
    char* ws = (char*)workspace;
    float* q_mean = (float*)(ws + w.q_mean);
    float* k_mean = (float*)(ws + w.k_mean);
    float* k_sum = (float*)(ws + w.k_sum);
    float* v_sum = (float*)(ws + w.v_sum);
    float* bias = (float*)(ws + w.bias);
    float* anchor = (float*)(ws + w.anchor);
    int32_t* idx = idx_out ? idx_out : (int32_t*)(ws + w.idx);
    int32_t* counts = counts_out ? counts_out : (int32_t*)(ws + w.counts);
    launch_pool_pack(L, Q, K, V, q_mean, k_mean, k_sum, v_sum, bias, anchor, ws + w.packed);
    launch_select_tau(L, tau, q_mean, k_mean, idx, counts, nullptr, (float*)(ws + w.scores),
                      (double*)(ws + w.partials));
    launch_attend(L, Q, ws + w.packed, idx, counts, nullptr, O, lse);
    return launch_status();
}

int spark_attn_gather_rows(const spark_attn_params* p, const void* X, const int32_t* perm, void* Y, void* stream) {
    LaunchCtx L;
    int s = make_ctx(p, stream, &L);
    if (s < 0) return s;
    if (!X || !perm || !Y || X == Y) return SPARK_ATTN_INVALID_ARGUMENT;
    if (!aligned16(X) || !aligned16(Y)) return SPARK_ATTN_MISALIGNED;
    launch_gather_rows(L, X, perm, Y);
    return launch_status();
}

int spark_attn_forward_kv(const spark_attn_params* p, const void* Q, const void* K, const void* V,
                          const int32_t* perm_q, const int32_t* perm_k, void* O, float* lse, int32_t* idx_out,
                          void* workspace, size_t ws_bytes, void* stream) {
    LaunchCtx L;
    int s = make_ctx(p, stream, &L);
    if (s < 0) return s;
    if (!Q || !K || !V || !O) return SPARK_ATTN_INVALID_ARGUMENT;
    if (!aligned16(Q) || !aligned16(K) || !aligned16(V) || !aligned16(O) || !aligned16(workspace))
        return SPARK_ATTN_MISALIGNED;
    const FwdWorkspace w = fwd_layout(L, perm_q != nullptr || perm_k != nullptr);
    if (!workspace || ws_bytes < w.total) return SPARK_ATTN_WORKSPACE_TOO_SMALL;
    char* ws = (char*)workspace;
    const void *q = Q, *k = K, *v = V;
    if (perm_q) {
        launch_gather_rows(L, Q, perm_q, ws + w.qp);
        q = ws + w.qp;
    }
    if (perm_k) {
        launch_gather_rows(L, K, perm_k, ws + w.kp);
        launch_gather_rows(L, V, perm_k, ws + w.vp);
        k = ws + w.kp;
        v = ws + w.vp;
    }
    float* q_mean = (float*)(ws + w.q_mean);
    float* k_mean = (float*)(ws + w.k_mean);
    float* k_sum = (float*)(ws + w.k_sum);
    float* v_sum = (float*)(ws + w.v_sum);
    float* bias = (float*)(ws + w.bias);
    float* anchor = (float*)(ws + w.anchor);
    int32_t* idx = idx_out ? idx_out : (int32_t*)(ws + w.idx);
    launch_pool_pack(L, q, k, v, q_mean, k_mean, k_sum, v_sum, bias, anchor, ws + w.packed);
    launch_select(L, q_mean, k_mean, idx, (float*)(ws + w.scores));
    launch_attend(L, q, ws + w.packed, idx, nullptr, perm_q, O, lse);
    return launch_status();
}

int spark_attn_forward(const spark_attn_params* p, const void* Q, const void* K, const void* V, const int32_t* perm,
                       void* O, float* lse, int32_t* idx_out, void* workspace, size_t ws_bytes, void* stream) {
    return spark_attn_forward_kv(p, Q, K, V, perm, perm, O, lse, idx_out, workspace, ws_bytes, stream);
}

int spark_attn_fp8_scales(const spark_attn_params* p, const void* Q, const void* K, const void* V, float* amax,
                          void* stream) {
    LaunchCtx L;
    int s = make_ctx(p, stream, &L);
    if (s < 0) return s;
    if (!Q || !K || !V || !amax) return SPARK_ATTN_INVALID_ARGUMENT;
    if (!aligned16(Q) || !aligned16(K) || !aligned16(V)) return SPARK_ATTN_MISALIGNED;
    launch_fp8_scales(L, Q, K, V, (uint32_t*)amax);
    return launch_status();
}

int spark_attn_pool_fp8_scales(const spark_attn_params* p, const void* Q, const void* K, const void* V,
                               float* q_mean, float* k_mean, float* k_sum, float* v_sum, float* bias, float* anchor,
                               float* amax, void* stream) {
    LaunchCtx L;
    int s = make_ctx(p, stream, &L);
    if (s < 0) return s;
    if (!Q || !K || !V || !q_mean || !k_mean || !k_sum || !v_sum || !bias || !anchor || !amax)
        return SPARK_ATTN_INVALID_ARGUMENT;
    if (!aligned16(Q) || !aligned16(K) || !aligned16(V) || !aligned16(q_mean) || !aligned16(k_mean) ||
        !aligned16(k_sum) || !aligned16(v_sum) || !aligned16(anchor))
        return SPARK_ATTN_MISALIGNED;
    launch_pool_fp8_scales(L, Q, K, V, q_mean, k_mean, k_sum, v_sum, bias, anchor, (uint32_t*)amax);
    return launch_status();
}

int spark_attn_pack_fp8(const spark_attn_params* p, const void* K, const void* V, const float* k_sum,
                        const float* v_sum, const float* bias, const float* amax, void* packed, size_t packed_bytes,
                        void* stream) {
    LaunchCtx L;
    int s = make_ctx(p, stream, &L);
    if (s < 0) return s;
    if (!K || !V || !k_sum || !v_sum || !bias || !amax) return SPARK_ATTN_INVALID_ARGUMENT;
    if (!aligned16(K) || !aligned16(V) || !aligned16(k_sum) || !aligned16(v_sum) || !aligned16(packed))
        return SPARK_ATTN_MISALIGNED;
    if (!packed || packed_bytes < pack_geom_fp8(L).bytes) return SPARK_ATTN_WORKSPACE_TOO_SMALL;
    launch_pack_fp8(L, K, V, k_sum, v_sum, bias, (const uint32_t*)amax, packed);
    return launch_status();
}

int spark_attn_attend_fp8(const spark_attn_params* p, const void* Q, const void* packed, size_t packed_bytes,
                          const int32_t* idx, const int32_t* perm, const float* amax, void* O, float* lse,
                          void* stream) {
    LaunchCtx L;
    int s = make_ctx(p, stream, &L);
    if (s < 0) return s;
    if (!Q || !idx || !amax || !O) return SPARK_ATTN_INVALID_ARGUMENT;
    if (!aligned16(Q) || !aligned16(packed) || !aligned16(O)) return SPARK_ATTN_MISALIGNED;
    if (!packed || packed_bytes < pack_geom_fp8(L).bytes) return SPARK_ATTN_WORKSPACE_TOO_SMALL;
    launch_attend_fp8(L, Q, packed, idx, perm, (const uint32_t*)amax, O, lse);
    return launch_status();
}

int spark_attn_forward_fp8(const spark_attn_params* p, const void* Q, const void* K, const void* V,
                           const int32_t* perm, void* O, float* lse, int32_t* idx_out, float* amax_out,
                           void* workspace, size_t ws_bytes, void* stream) {
    LaunchCtx L;
    int s = make_ctx(p, stream, &L);
    if (s < 0) return s;
    if (!Q || !K || !V || !O) return SPARK_ATTN_INVALID_ARGUMENT;
    if (!aligned16(Q) || !aligned16(K) || !aligned16(V) || !aligned16(O) || !aligned16(workspace))
        return SPARK_ATTN_MISALIGNED;
    const Fp8Workspace w = fp8_layout(L, perm != nullptr);
    if (!workspace || ws_bytes < w.total) return SPARK_ATTN_WORKSPACE_TOO_SMALL;
    char* ws = (char*)workspace;
    const void *q = Q, *k = K, *v = V;
    if (perm) {
        launch_gather_rows(L, Q, perm, ws + w.qp);
        launch_gather_rows(L, K, perm, ws + w.kp);
        launch_gather_rows(L, V, perm, ws + w.vp);
        q = ws + w.qp;
        k = ws + w.kp;
        v = ws + w.vp;
    }
    float* q_mean = (float*)(ws + w.q_mean);
    float* k_mean = (float*)(ws + w.k_mean);
    float* k_sum = (float*)(ws + w.k_sum);
    float* v_sum = (float*)(ws + w.v_sum);
    float* bias = (float*)(ws + w.bias);
    float* anchor = (float*)(ws + w.anchor);
    int32_t* idx = idx_out ? idx_out : (int32_t*)(ws + w.idx);
    uint32_t* amax = amax_out ? (uint32_t*)amax_out : (uint32_t*)(ws + w.amax);
    launch_pool_fp8_scales(L, q, k, v, q_mean, k_mean, k_sum, v_sum, bias, anchor, amax);
    launch_select(L, q_mean, k_mean, idx, (float*)(ws + w.scores));
    launch_pack_fp8(L, k, v, k_sum, v_sum, bias, amax, ws + w.packed);
    launch_attend_fp8(L, q, ws + w.packed, idx, perm, amax, O, lse);
    return launch_status();
}

int spark_attn_reblock(const spark_attn_params* p, const void* Q, const void* K, int32_t* perm, void* workspace,
                       size_t ws_bytes, void* stream) {
    LaunchCtx L;
    int s = make_ctx(p, stream, &L);
    if (s < 0) return s;
    if (!Q || !K || !perm) return SPARK_ATTN_INVALID_ARGUMENT;
    if (!aligned16(Q) || !aligned16(K) || !aligned16(workspace)) return SPARK_ATTN_MISALIGNED;
    const size_t need = reblock_workspace_bytes(L);
    if (need == 0) return SPARK_ATTN_UNSUPPORTED;
    if (!workspace || ws_bytes < need) return SPARK_ATTN_WORKSPACE_TOO_SMALL;
    launch_reblock(L, Q, K, perm, workspace);
    return launch_status();
}

}  // extern "C"
