// Block representatives: mean pooling of contiguous key blocks.
//
// Mean pooling of contiguous blocks of B keys is how the pages build the
// coarse-stage block representatives (gptget.net English summary,
// "Methodology"; Chinese summary, method details).  The representative is
// bf16 so that the block stage feeds the same bf16 matrix-core scorer as the
// token stage; it is rounded once from the exact-order fp64 sum:
//     mean = bf16_RNE( fp32_RNE( (sum over rows, increasing row, in fp64) / count ) ).
// One thread owns one column of one block: the 64 lanes of a wave read 64
// consecutive bf16 of a key row (128 coalesced bytes) per step.

#include "hisa_internal.h"

namespace hisa {
namespace {

__device__ __forceinline__ uint16_t column_mean(const uint16_t *__restrict__ col, int64_t rows,
                                                int d) {
    double sum = 0.0;
    for (int64_t j = 0; j < rows; ++j)
        sum += static_cast<double>(bf16_to_f32(col[j * d]));
    const float mean = static_cast<float>(sum / static_cast<double>(rows));
    return f32_to_bf16_rne(mean);
}

// grid: (nblk, S), block: d threads.  Recomputes blocks [blk0, blk0 + nblk).
__global__ void pool_append_kernel(const uint16_t *__restrict__ K, int64_t k_seq_stride, int d,
                                   int B, int64_t blk0, int64_t L_new,
                                   uint16_t *__restrict__ pool, int64_t pool_seq_stride) {
    const int s = blockIdx.y;
    const int64_t b = blk0 + blockIdx.x;
    const int c = threadIdx.x;
    const int64_t r0 = b * B;
    const int64_t r1 = (r0 + B < L_new) ? r0 + B : L_new;
    const uint16_t *col = K + s * k_seq_stride + r0 * d + c;
    pool[s * pool_seq_stride + b * d + c] = column_mean(col, r1 - r0, d);
}

// grid: (S*T), block: d threads.  For a query at t whose own block
// b_t = floor(t/B) is not exactly covered by the pool entry (the entry covers
// rows [b_t*B, min(b_t*B + B, L)), the query needs [b_t*B, t]), writes the
// mean of rows [b_t*B, t] to own_rep[qi].
__global__ void own_mean_kernel(const uint16_t *__restrict__ K, int64_t k_seq_stride,
                                const int32_t *__restrict__ qpos, int64_t L, int T, int d, int B,
                                uint16_t *__restrict__ own_rep) {
    const int qi = blockIdx.x;
    const int s = qi / T;
    const int i = qi - s * T;
    const int64_t t = query_pos(qpos, qi, i, L, T);
    if (t < 0) return;
    const int64_t r0 = (t / B) * B;
    const int64_t covered = (r0 + B < L) ? r0 + B : L;
    if (covered == t + 1) return;
    const int c = threadIdx.x;
    const uint16_t *col = K + s * k_seq_stride + r0 * d + c;
    own_rep[static_cast<int64_t>(qi) * d + c] = column_mean(col, t + 1 - r0, d);
}

}  // namespace

hipError_t launch_pool_append(const uint16_t *K, int64_t k_seq_stride, int S, int d, int B,
                              int64_t blk0, int64_t nblk, int64_t L_new, uint16_t *pool,
                              int64_t pool_seq_stride, hipStream_t st) {
    prof_begin(kKindPoolAppend, st);
    hipLaunchKernelGGL(pool_append_kernel, dim3(static_cast<uint32_t>(nblk), S), dim3(d), 0, st,
                       K, k_seq_stride, d, B, blk0, L_new, pool, pool_seq_stride);
    prof_end(kKindPoolAppend, st);
    return hipGetLastError();
}

hipError_t launch_own_mean(const uint16_t *K, int64_t k_seq_stride, const int32_t *qpos,
                           int64_t L, int S, int T, int d, int B, uint16_t *own_rep,
                           hipStream_t st) {
    prof_begin(kKindOwnMean, st);
    hipLaunchKernelGGL(own_mean_kernel, dim3(S * T), dim3(d), 0, st, K, k_seq_stride, qpos, L, T,
                       d, B, own_rep);
    prof_end(kKindOwnMean, st);
    return hipGetLastError();
}

}  // namespace hisa
