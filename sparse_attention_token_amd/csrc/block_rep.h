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


// Largest spread of binary exponents over which an fp64 sum of up to 256 bf16
// values is exact in any order.  A bf16 value of biased exponent e (1 for
// subnormals) is an integer multiple of 2^(e - 134) below 2^(e - 126) in
// magnitude, so every partial sum of n <= 256 values with exponents in
// [emin, emax] is a multiple of 2^(emin - 134) below 2^(emax - 118): an
// integer of at most emax - emin + 16 bits, which fp64's 53-bit significand
// holds while emax - emin <= 37.  The row-order sum is then also the exact
// sum, so partial sums added in any grouping give its bits.
constexpr int kExactExpSpread = 37;

typedef unsigned short own_u16x2 __attribute__((ext_vector_type(2)));

// The own-block representative spread over all NT threads of a workgroup:
// thread (p, cp) takes column pair cp (columns 2cp, 2cp+1: one 32-bit word of
// each row) over part p of the rows -- rows [p*rp, p*rp + rp), rp =
// ceil(n / P) -- straight from global memory (each row is one coalesced
// access across the part's lanes), so the rows are never staged in LDS.
// Mean: each part sums its rows in row order in fp64 and records the smallest
// and largest nonzero magnitude; when a column's exponent spread is at most
// kExactExpSpread, the parts' sums added in part order are the exact sum --
// the bits of the row-order sum -- and otherwise the column's thread adds its
// rows in row order itself.  Max: each part keeps its first largest value;
// the parts are taken in order and a later part wins only with a larger value.
// Usage: load() early (the loads stay in flight), partial() once the rows are
// needed (writes the parts to the scratch), a workgroup barrier, then
// combine() on threads c < D.
template <int D, int NT>
struct OwnRowsPar {
    static constexpr int CP = D / 2;                         // column pairs
    static constexpr int P = NT / CP;                        // row parts
    static constexpr int MAXR = kFusedOwnElems / D / P;      // rows per part at most (n <= kFusedOwnElems / D)
    static_assert(NT % CP == 0 && MAXR >= 1, "own-block thread layout");
    struct Scratch {
        double sum[P][D];
        uint32_t lo[P][CP];     // mean: smallest nonzero magnitude - 1 per column (u16 pair); max: unused
        uint32_t hi[P][CP];     // mean: largest magnitude per column (u16 pair)
        uint32_t best[P][D];    // max: the part's first largest bf16 | 0x10000, or 0 for an empty part
    };
    uint32_t v[MAXR];

    // Every load is issued (rows past the part read row n-1, masked out by
    // partial()): a load under a branch can make the wave wait for it at once.
    __device__ __forceinline__ void load(const uint16_t *rows, int n, int tid) {
        const int cp = tid % CP, p = tid / CP;
        const int rp = (n + P - 1) / P;
#pragma unroll
        for (int j = 0; j < MAXR; ++j) {
            const int r = p * rp + j;
            const int rc = (j < rp && r < n) ? r : n - 1;
            v[j] = reinterpret_cast<const uint32_t *>(rows + static_cast<int64_t>(rc) * D)[cp];
        }
    }

    template <bool MAX>
    __device__ __forceinline__ void partial(int n, int tid, Scratch &sc) const {
        const int cp = tid % CP, p = tid / CP;
        const int rp = (n + P - 1) / P;
        if (MAX) {
            float b0 = -__builtin_huge_valf(), b1 = -__builtin_huge_valf();
            uint32_t h0 = 0u, h1 = 0u;
#pragma unroll
            for (int j = 0; j < MAXR; ++j) {
                if (j < rp && p * rp + j < n) {
                    const float x0 = __uint_as_float(v[j] << 16), x1 = __uint_as_float(v[j] & 0xFFFF0000u);
                    if (x0 > b0) { b0 = x0; h0 = (v[j] & 0xFFFFu) | 0x10000u; }
                    if (x1 > b1) { b1 = x1; h1 = (v[j] >> 16) | 0x10000u; }
                }
            }
            sc.best[p][2 * cp] = h0;
            sc.best[p][2 * cp + 1] = h1;
        } else {
            double s0 = 0.0, s1 = 0.0;
            own_u16x2 lo = {0xFFFFu, 0xFFFFu}, hi = {0u, 0u};
            const own_u16x2 one = {1u, 1u};
#pragma unroll
            for (int j = 0; j < MAXR; ++j) {      // rows past the part count as zero: +0, no magnitude
                const uint32_t x = (j < rp && p * rp + j < n) ? v[j] : 0u;
                const own_u16x2 mag = __builtin_bit_cast(own_u16x2, x & 0x7FFF7FFFu);
                lo = __builtin_elementwise_min(lo, mag - one);     // a zero wraps to 0xFFFF
                hi = __builtin_elementwise_max(hi, mag);
                s0 += static_cast<double>(__uint_as_float(x << 16));
                s1 += static_cast<double>(__uint_as_float(x & 0xFFFF0000u));
            }
            sc.sum[p][2 * cp] = s0;
            sc.sum[p][2 * cp + 1] = s1;
            sc.lo[p][cp] = __builtin_bit_cast(uint32_t, lo);
            sc.hi[p][cp] = __builtin_bit_cast(uint32_t, hi);
        }
    }

    // Thread c < D: the representative of column c, into mean[c] and dst[c]
    // (either may be null).  rows: as for load().
    template <bool MAX>
    __device__ __forceinline__ void combine(const uint16_t *rows, int n, int c, const Scratch &sc, uint16_t *mean,
                                            uint16_t *dst) const {
        uint16_t mv;
        if (MAX) {
            float bf = -__builtin_huge_valf();
            uint16_t b = 0;
#pragma unroll
            for (int q = 0; q < P; ++q) {
                const uint32_t x = sc.best[q][c];
                if (x & 0x10000u) {
                    const float f = __uint_as_float(x << 16);
                    if (f > bf) { bf = f; b = static_cast<uint16_t>(x & 0xFFFFu); }
                }
            }
            mv = b;
        } else {
            const int cp = c >> 1, sh = (c & 1) * 16;
            double total = 0.0;
            uint32_t lo = 0xFFFFu, hi = 0u;
#pragma unroll
            for (int q = 0; q < P; ++q) {
                total += sc.sum[q][c];
                const uint32_t l = (sc.lo[q][cp] >> sh) & 0xFFFFu, h = (sc.hi[q][cp] >> sh) & 0xFFFFu;
                lo = l < lo ? l : lo;
                hi = h > hi ? h : hi;
            }
            if (lo != 0xFFFFu) {                   // some nonzero value: check the spread
                const uint32_t emin = ((lo + 1u) >> 7) > 1u ? ((lo + 1u) >> 7) : 1u;
                const uint32_t emax = (hi >> 7) > 1u ? (hi >> 7) : 1u;
                if (emax - emin > static_cast<uint32_t>(kExactExpSpread)) {
                    total = 0.0;                   // the sum may round: add the rows in row order
                    for (int r = 0; r < n; ++r)
                        total += static_cast<double>(__uint_as_float(static_cast<uint32_t>(rows[static_cast<int64_t>(r) * D + c]) << 16));
                }
            }
            mv = f32_to_bf16_rne(static_cast<float>(total / static_cast<double>(n)));
        }
        if (mean) mean[c] = mv;
        if (dst) dst[c] = mv;
    }
};

}  // namespace hisa

