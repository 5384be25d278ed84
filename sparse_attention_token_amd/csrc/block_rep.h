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

namespace hisa {

// Largest spread of binary exponents over which an fp64 sum of up to 256 bf16
// values is exact whatever the order.  A bf16 value of biased exponent e (1 for
// subnormals) is an integer multiple of 2^(e - 134) below 2^(e - 126) in
// magnitude; so every partial sum of n <= 256 such values with exponents in
// [emin, emax] is a multiple of 2^(emin - 134) below 2^(emax - 118), an
// integer of at most (emax - emin) + 16 bits, which fp64's 53-bit significand
// holds when emax - emin <= 37.
constexpr int kExactExpSpread = 37;

// LDS of own_rows_rep_par: kOwnParts partial results per column.
constexpr int kOwnParts = 4;
struct OwnRepScratch {
    double sum[kOwnParts][128];
    uint32_t aux[kOwnParts][128];   // mean: emin | emax << 16; max: the part's best bits
};

// As own_rows_rep, with the rows split among min(4, NT / D) threads per column
// and the same bits.  Each thread sums its run of rows in fp64 and records the
// smallest and largest exponent among the nonzero values; when the column's
// spread is at most kExactExpSpread every partial sum is exact, so their sum
// in any order is the exact sum -- the value the row-order sum also reaches --
// and the partial sums are added; otherwise the first thread of the column
// adds all rows in row order.  Max pooling takes the parts' maxima in row
// order, keeping the earliest among equal values.  NT threads; ends with a
// barrier.
template <int D, int NT, bool MAX>
__device__ __forceinline__ void own_rows_rep_par(const uint16_t *s_own, int n, uint16_t *mean, uint16_t *dst,
                                                 OwnRepScratch &sc) {
    constexpr int P = (NT / D) < kOwnParts ? (NT / D) : kOwnParts;
    static_assert(P >= 1 && D <= 128, "own-block representative layout");
    const int tid = threadIdx.x;
    const int c = tid % D, p = tid / D;
    if (p < P) {
        const int per = (n + P - 1) / P;
        const int r0 = p * per, r1 = (r0 + per < n) ? r0 + per : n;
        double sum = 0.0;
        uint32_t emin = 255u, emax = 0u;
        float bestf = -__builtin_huge_valf();
        uint16_t best = 0;
        constexpr int U = 16;                            // LDS reads in flight
        for (int r = r0; r < r1; r += U) {
            uint16_t x[U];
#pragma unroll
            for (int j = 0; j < U; ++j) x[j] = r + j < r1 ? s_own[(r + j) * D + c] : uint16_t{0};
#pragma unroll
            for (int j = 0; j < U; ++j) {
                if (r + j < r1) {
                    const uint16_t h = x[j];
                    const float v = bf16_to_f32(h);
                    if (MAX) {
                        if (v > bestf) {
                            bestf = v;
                            best = h;
                        }
                    } else {
                        sum += static_cast<double>(v);
                        if ((h & 0x7FFFu) != 0u) {
                            uint32_t e = (h >> 7) & 0xFFu;
                            e = e == 0u ? 1u : e;
                            emin = e < emin ? e : emin;
                            emax = e > emax ? e : emax;
                        }
                    }
                }
            }
        }
        sc.sum[p][c] = sum;
        sc.aux[p][c] = MAX ? (r0 < r1 ? static_cast<uint32_t>(best) | 0x10000u : 0u) : (emin | (emax << 16));
    }
    __syncthreads();
    if (tid < D) {
        uint16_t mv;
        if (MAX) {
            float bf = -__builtin_huge_valf();
            uint16_t b = 0;
#pragma unroll
            for (int q = 0; q < P; ++q) {
                const uint32_t a = sc.aux[q][c];
                if (a & 0x10000u) {                      // the part held rows
                    const uint16_t h = static_cast<uint16_t>(a & 0xFFFFu);
                    const float v = bf16_to_f32(h);
                    if (v > bf) {
                        bf = v;
                        b = h;
                    }
                }
            }
            mv = b;
        } else {
            uint32_t emin = 255u, emax = 0u;
            double total = 0.0;
#pragma unroll
            for (int q = 0; q < P; ++q) {
                const uint32_t a = sc.aux[q][c];
                emin = (a & 0xFFFFu) < emin ? (a & 0xFFFFu) : emin;
                emax = (a >> 16) > emax ? (a >> 16) : emax;
                total += sc.sum[q][c];
            }
            if (emax > emin && emax - emin > static_cast<uint32_t>(kExactExpSpread)) {
                total = 0.0;                             // the sum may round: rows in row order
                for (int r = 0; r < n; ++r) total += static_cast<double>(bf16_to_f32(s_own[r * D + c]));
            }
            mv = f32_to_bf16_rne(static_cast<float>(total / static_cast<double>(n)));
        }
        mean[c] = mv;
        if (dst) dst[c] = mv;
    }
    __syncthreads();
}

}  // namespace hisa
