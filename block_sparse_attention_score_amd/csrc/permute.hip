// Row gather for the adaptive block layout (Spark-H3 page, section "ワークフロー":
// reblock_layout=q_reuse_k, keys and values follow the query partition).  For each (batch, head)
// row q < N_v of Y is row perm[q] of X; sink rows are copied as they are.  Pure HBM traffic:
// one thread per 16-byte chunk, rows read whole, so every access is a full coalesced row.
#include "kernels.hpp"

namespace spark {

template <int CPR>  // 16-byte chunks per row
__global__ __launch_bounds__(256) void gather_rows_kernel(const u32x4* __restrict__ X, const int32_t* __restrict__ perm,
                                                          u32x4* __restrict__ Y, int N, int Nv, size_t total) {
    for (size_t e = (size_t)blockIdx.x * 256 + threadIdx.x; e < total; e += (size_t)gridDim.x * 256) {
        const size_t row = e / CPR;
        const int c = (int)(e % CPR);
        const size_t bh = row / N;
        const int r = (int)(row % N);
        // a permutation entry out of range is clamped to the video rows (no read out of bounds)
        const int src = r < Nv ? min(max(perm[bh * Nv + r], 0), Nv - 1) : r;
        Y[e] = X[(bh * N + src) * CPR + c];
    }
}

void launch_gather_rows(const LaunchCtx& L, const void* X, const int32_t* perm, void* Y) {
    const int row_bytes = L.d * (L.dtype == SPARK_ATTN_BF16 ? 2 : 4);
    const int cpr = row_bytes / 16;
    const size_t total = (size_t)L.BH * L.N * cpr;
    size_t blocks = (total + 255) / 256;
    if (blocks > 65536) blocks = 65536;
    const u32x4* x = (const u32x4*)X;
    u32x4* y = (u32x4*)Y;
    switch (cpr) {
        case 8: hipLaunchKernelGGL((gather_rows_kernel<8>), dim3(blocks), dim3(256), 0, L.stream, x, perm, y, L.N, L.Nv, total); break;
        case 16: hipLaunchKernelGGL((gather_rows_kernel<16>), dim3(blocks), dim3(256), 0, L.stream, x, perm, y, L.N, L.Nv, total); break;
        case 32: hipLaunchKernelGGL((gather_rows_kernel<32>), dim3(blocks), dim3(256), 0, L.stream, x, perm, y, L.N, L.Nv, total); break;
        default: break;  // d in {64, 128} x {2, 4} bytes always gives 8, 16 or 32
    }
}

}  // namespace spark
