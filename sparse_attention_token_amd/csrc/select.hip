// Exact top-k selection over per-query candidate keys.
//
// Both stages of the pages' method end in a "keep the best" step -- the top m
// blocks after block scoring, then the final top k tokens of the refinement
// (gptget.net English summary, "Methodology"; Chinese summary, method
// details) -- and the flat indexer ends in a top k over the whole prefix.
// This kernel implements all three with one rule: rank by (score desc,
// index asc), keep min(k, #candidates), pad with -1.
//
// Scores arrive as order-preserving uint32 keys (0 = no candidate).  One
// workgroup of 1024 threads owns one query:
//   1. Radix select, most significant byte first (4 passes of 8 bits):
//      an LDS histogram of the next byte over keys that still match the
//      prefix, then one wave scans the 256 bins from the top to find the byte
//      holding the rank still needed.  After 4 passes the exact 32-bit key
//      K* of the k-th best candidate is known, together with the number of
//      candidates strictly above it.  (The first pass also counts the
//      candidates, which fixes k_eff.)
//   2. Compaction in position order: thread i owns positions
//      [i*16, i*16 + 16) of each 16384-position chunk; one block-wide scan of
//      the packed pair (#keys > K*, #keys == K*) gives every kept key its
//      output slot, where keys equal to K* are kept lowest position first up
//      to the count still needed.
// Positions are laid out in increasing candidate index (block ids, or token
// ids of the kept blocks taken in ascending block order), so "lowest
// position first" is the index-ascending tie rule, and every output row comes
// out sorted by index.

#include "hisa_internal.h"

namespace hisa {
namespace {

constexpr int kThreads = 1024;
constexpr int kWavesSel = kThreads / 64;
constexpr int kR = 16;
constexpr int64_t kChunk = static_cast<int64_t>(kThreads) * kR;   // 16384 < 2^16

template <int MODE>
__device__ __forceinline__ int32_t position_to_id(const SelectArgs &a, int qi, int64_t p) {
    if (MODE == kScoreRefine) {
        const int64_t slot = p / a.B;
        return static_cast<int32_t>(
            static_cast<int64_t>(a.sel_blk[static_cast<int64_t>(qi) * a.m + slot]) * a.B + (p - slot * a.B));
    }
    return static_cast<int32_t>(p);
}

template <int MODE>
__global__ __launch_bounds__(kThreads) void select_kernel(SelectArgs a) {
    __shared__ uint32_t hist[256];
    __shared__ uint32_t wave_tot[kWavesSel];
    __shared__ uint32_t sh_digit, sh_above, sh_keff;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int qi = blockIdx.x;
    const int s = qi / a.T;
    const int i = qi - s * a.T;
    const int64_t t = query_pos(a.qpos, qi, i, a.L, a.T);
    int64_t n = 0;
    if (t >= 0) {
        const int64_t bt = t / a.B;
        if (MODE == kScoreBlocks) n = bt + 1;
        else if (MODE == kScoreRefine) n = ((a.m < bt + 1) ? a.m : bt + 1) * a.B;
        else n = t + 1;
    }
    const uint32_t *keys = a.keys + static_cast<int64_t>(qi) * a.keys_stride;
    int32_t *out = a.out_id + static_cast<int64_t>(qi) * a.kout;
    float *osc = a.out_score ? a.out_score + static_cast<int64_t>(qi) * a.kout : nullptr;
    int32_t *out2 = a.out_id_copy ? a.out_id_copy + static_cast<int64_t>(qi) * a.kout : nullptr;

    // ---------------- 1. radix select of the k-th best key
    uint32_t prefix = 0, mask = 0;
    uint32_t need = 0, keff = 0;
    for (int pass = 0; pass < 4 && n > 0; ++pass) {
        const int shift = 24 - 8 * pass;
        if (tid < 256) hist[tid] = 0;
        __syncthreads();
        for (int64_t c0 = 0; c0 < n; c0 += kChunk) {
            const int64_t base = c0 + static_cast<int64_t>(tid) * kR;
#pragma unroll
            for (int r = 0; r < kR; ++r) {
                const int64_t p = base + r;
                if (p < n) {
                    const uint32_t key = keys[p];
                    if (key != kNoCandidate && (key & mask) == prefix)
                        atomicAdd(&hist[(key >> shift) & 255u], 1u);
                }
            }
        }
        __syncthreads();
        if (wave == 0) {
            const uint32_t h0 = hist[4 * lane + 0], h1 = hist[4 * lane + 1];
            const uint32_t h2 = hist[4 * lane + 2], h3 = hist[4 * lane + 3];
            const uint32_t c = h0 + h1 + h2 + h3;
            uint32_t suf = c;                                  // sum over lanes >= this lane
#pragma unroll
            for (int off = 1; off < 64; off <<= 1) {
                const uint32_t v = __shfl_down(suf, off);
                if (lane + off < 64) suf += v;
            }
            // rank still needed among keys matching the prefix; on the first
            // pass the histogram holds every candidate, which fixes k_eff
            uint32_t rank = need;
            if (pass == 0) {
                const uint32_t total = __shfl(suf, 0);
                rank = total < static_cast<uint32_t>(a.kout) ? total : static_cast<uint32_t>(a.kout);
                if (lane == 0) sh_keff = rank;
            }
            uint32_t above = suf - c;
            const uint32_t hb[4] = {h0, h1, h2, h3};
#pragma unroll
            for (int b = 3; b >= 0; --b) {
                if (rank > 0 && above < rank && above + hb[b] >= rank) {
                    sh_digit = static_cast<uint32_t>(4 * lane + b);
                    sh_above = above;
                }
                above += hb[b];
            }
        }
        __syncthreads();
        if (pass == 0) {
            keff = sh_keff;
            need = keff;
            if (keff == 0) break;
        }
        prefix |= sh_digit << shift;
        mask |= 0xFFu << shift;
        need -= sh_above;
        __syncthreads();   // sh_digit / sh_above / hist are rewritten next pass
    }
    const uint32_t kstar = prefix;
    const uint32_t need_eq = need;   // >= 1 when keff > 0

    // ---------------- 2. compaction in position order
    if (keff > 0) {
        uint32_t run_gt = 0, run_eq = 0;
        for (int64_t c0 = 0; c0 < n; c0 += kChunk) {
            const int64_t base = c0 + static_cast<int64_t>(tid) * kR;
            uint32_t kv[kR];
            uint32_t cg = 0, ce = 0;
#pragma unroll
            for (int r = 0; r < kR; ++r) {
                const int64_t p = base + r;
                kv[r] = p < n ? keys[p] : kNoCandidate;
                cg += kv[r] > kstar;
                ce += kv[r] == kstar;
            }
            const uint32_t v = (cg << 16) | ce;
            uint32_t incl = v;
#pragma unroll
            for (int off = 1; off < 64; off <<= 1) {
                const uint32_t y = __shfl_up(incl, off);
                if (lane >= off) incl += y;
            }
            if (lane == 63) wave_tot[wave] = incl;
            __syncthreads();
            uint32_t ex_wave = 0, tot = 0;
#pragma unroll
            for (int wv = 0; wv < kWavesSel; ++wv) {
                const uint32_t x = wave_tot[wv];
                ex_wave += wv < wave ? x : 0u;
                tot += x;
            }
            const uint32_t ex = ex_wave + incl - v;
            uint32_t gt_before = run_gt + (ex >> 16);
            uint32_t eq_before = run_eq + (ex & 0xFFFFu);
#pragma unroll
            for (int r = 0; r < kR; ++r) {
                const uint32_t key = kv[r];
                uint32_t op = 0xFFFFFFFFu;
                if (key > kstar) {
                    op = gt_before + (eq_before < need_eq ? eq_before : need_eq);
                    ++gt_before;
                } else if (key == kstar) {
                    if (eq_before < need_eq) op = gt_before + eq_before;
                    ++eq_before;
                }
                if (op < keff) {   // always true for a correct threshold; guards the write
                    const int32_t id = position_to_id<MODE>(a, qi, base + r);
                    out[op] = id;
                    if (osc) osc[op] = key_to_score(key);
                    if (out2) out2[op] = id;
                }
            }
            run_gt += tot >> 16;
            run_eq += tot & 0xFFFFu;
            __syncthreads();   // wave_tot is rewritten by the next chunk
        }
    }

    // ---------------- 3. padding
    for (int j = static_cast<int>(keff) + tid; j < a.kout; j += kThreads) {
        out[j] = -1;
        if (osc) osc[j] = -__builtin_huge_valf();
        if (out2) out2[j] = -1;
    }
}

}  // namespace

hipError_t launch_select(ScoreMode mode, const SelectArgs &a, int nq, hipStream_t st) {
    const KernelKind kind = mode == kScoreBlocks ? kKindSelectBlocks
                          : mode == kScoreRefine ? kKindSelectRefine : kKindSelectFlat;
    prof_begin(kind, st);
    if (mode == kScoreBlocks)
        hipLaunchKernelGGL(select_kernel<kScoreBlocks>, dim3(nq), dim3(kThreads), 0, st, a);
    else if (mode == kScoreRefine)
        hipLaunchKernelGGL(select_kernel<kScoreRefine>, dim3(nq), dim3(kThreads), 0, st, a);
    else
        hipLaunchKernelGGL(select_kernel<kScoreFlat>, dim3(nq), dim3(kThreads), 0, st, a);
    prof_end(kind, st);
    return hipGetLastError();
}

}  // namespace hisa
