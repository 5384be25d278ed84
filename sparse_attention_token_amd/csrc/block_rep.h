// Representative of a query's own block, computed inside a kernel from the
// block's rows staged in LDS -- the same arithmetic as the block pool
// (pool.hip): the mean bf16(fp32(fp64 sum in row order / n)), or the
// per-column maximum.  Shared by the fused two-level kernels and the
// three-level tree kernel.
#pragma once

#include "hisa_internal.h"

namespace hisa {

// Own-block representative over rows 0 .. n-1 (1 <= n <= 256) of the staged
// block s_own (row stride D), per column, into mean[0 .. D) and, when dst is
// not null, dst[0 .. D): the mean bf16(fp32(fp64 sum in row order / n)), or
// with MAX the largest value (the earliest row among equal values, +0 and
// -0).  One thread per column (the first D threads); ends with a barrier.
// Rows are read U at a time, all U reads issued before the first addition
// (U = 64, or 16 in 1024-thread workgroups, whose register budget is
// smaller); a round may read past row n-1, never past the staging buffer
// (its kFusedOwnElems / D rows are a multiple of U), and such rows are not
// used.
template <int D, int U, bool MAX>
__device__ __forceinline__ void own_rows_rep(const uint16_t *s_own, int n, uint16_t *mean, uint16_t *dst) {
    static_assert((kFusedOwnElems / D) % U == 0, "rounds stay inside the staging buffer");
    const int c = threadIdx.x;
    if (c < D) {
        double sum = 0.0;
        float bestf = -__builtin_huge_valf();
        uint16_t best = 0;
        for (int r0 = 0; r0 < n; r0 += U) {
            const uint16_t *col = s_own + r0 * D + c;
            uint16_t x[U];
#pragma unroll
            for (int j = 0; j < U; ++j) x[j] = col[j * D];
            auto take = [&](uint16_t h) {
                const float v = bf16_to_f32(h);
                if (MAX) {
                    if (v > bestf) {
                        bestf = v;
                        best = h;
                    }
                } else {
                    sum += static_cast<double>(v);
                }
            };
            if (r0 + U <= n) {           // full round: no per-row test in the chain
#pragma unroll
                for (int j = 0; j < U; ++j) take(x[j]);
            } else {
#pragma unroll
                for (int j = 0; j < U; ++j)
                    if (r0 + j < n) take(x[j]);
            }
        }
        const uint16_t mv = MAX ? best : f32_to_bf16_rne(static_cast<float>(sum / static_cast<double>(n)));
        mean[c] = mv;
        if (dst) dst[c] = mv;
    }
    __syncthreads();
}

}  // namespace hisa

