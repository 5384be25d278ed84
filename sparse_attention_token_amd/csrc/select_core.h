// Exact top-k of register-resident keys for one workgroup (device code).
//
// Ranks by (key descending, position ascending), keeps min(kout, #candidates)
// and hands every kept key to emit(slot, position, key) with slots
// 0..k_eff-1 assigned in increasing position order.  Key 0 = no candidate.
// Thread t owns positions [t*R, t*R + R) and holds their keys in registers.
//
//   1. Radix select over digits of 11, 11 and 10 bits (three LDS histograms,
//      cleared together up front).  After each histogram the whole block
//      scans the bins from the top: thread t owns a contiguous run of bins in
//      descending order, reads it with 16-byte LDS loads, and a DPP prefix sum
//      within each wave plus one exchange of wave totals gives every thread
//      the count of keys in higher bins; the thread whose run holds the rank
//      still needed records the digit.  Three passes give the exact key K* of
//      the k-th best candidate and the count of keys above it; the passes stop
//      early when every key of the cutoff bin is kept (the kept set is then
//      every key at or above the bin's lowest value).
//   2. Compaction: a DPP prefix sum over the packed pair (#keys > K*,
//      #keys == K*) per thread gives each kept key its slot; keys equal to K*
//      are kept lowest position first.
//
// Costs on gfx950 that shaped this: LDS atomics to one address from many lanes
// serialize (about 16x a conflict-free one), cross-lane shuffles through LDS
// cost about 75 cycles each while DPP row operations cost a few, and 16-byte
// LDS reads whose lanes stride by 128 bytes conflict on every bank.
#pragma once

#include "hisa_internal.h"

namespace hisa {

typedef uint32_t sel_u32x4 __attribute__((ext_vector_type(4)));

// Inclusive prefix sum across a 64-lane wave with DPP row shifts and row
// broadcasts (lanes beyond a row edge contribute 0).
__device__ __forceinline__ uint32_t wave_prefix_incl(uint32_t x) {
    x += static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(x), 0x111, 0xf, 0xf, false));  // row_shr:1
    x += static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(x), 0x112, 0xf, 0xf, false));  // row_shr:2
    x += static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(x), 0x114, 0xf, 0xf, false));  // row_shr:4
    x += static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(x), 0x118, 0xf, 0xf, false));  // row_shr:8
    x += static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(x), 0x142, 0xa, 0xf, false));  // row_bcast:15
    x += static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(x), 0x143, 0xc, 0xf, false));  // row_bcast:31
    return x;
}

constexpr int kCoreBins0 = 2048, kCoreBins1 = 2048, kCoreBins2 = 1024;

struct SelectScratch {
    uint32_t hist[kCoreBins0 + kCoreBins1 + kCoreBins2];
    uint32_t wave_tot[16];
    uint32_t digit, above, count;
};

// Block-wide exclusive prefix over threads of a per-thread count; also returns
// the block total.  Uses sc.wave_tot; ends with the wave totals consumed.
template <int NT>
__device__ __forceinline__ uint32_t block_exclusive(uint32_t v, uint32_t &total, SelectScratch &sc) {
    constexpr int NW = NT / 64;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const uint32_t incl = wave_prefix_incl(v);
    if (lane == 63) sc.wave_tot[wave] = incl;
    __syncthreads();
    uint32_t before = 0, tot = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
        const uint32_t x = sc.wave_tot[w];
        before += w < wave ? x : 0u;
        tot += x;
    }
    total = tot;
    return before + incl - v;
}

struct SelectResult {
    uint32_t kstar;      // key of the k_eff-th best candidate
    uint32_t need_eq;    // how many keys equal to kstar are kept
    uint32_t keff;       // number of kept keys
};

template <int NT, int R>
__device__ __forceinline__ SelectResult block_radix_select(const uint32_t (&kv)[R], uint32_t kout,
                                                           SelectScratch &sc) {
    const int tid = threadIdx.x;
    for (int b = tid * 4; b < kCoreBins0 + kCoreBins1 + kCoreBins2; b += NT * 4)
        *reinterpret_cast<sel_u32x4 *>(&sc.hist[b]) = sel_u32x4{0u, 0u, 0u, 0u};
    __syncthreads();
    uint32_t prefix = 0, mask = 0, need = 0, keff = 0;
#pragma unroll
    for (int pass = 0; pass < 3; ++pass) {
        const int shift = pass == 0 ? 21 : (pass == 1 ? 10 : 0);
        constexpr int kNB[3] = {kCoreBins0, kCoreBins1, kCoreBins2};
        const int nb = kNB[pass];
        uint32_t *h = sc.hist + (pass == 0 ? 0 : (pass == 1 ? kCoreBins0 : kCoreBins0 + kCoreBins1));
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const uint32_t key = kv[r];
            if (key != kNoCandidate && (key & mask) == prefix)
                atomicAdd(&h[(key >> shift) & static_cast<uint32_t>(nb - 1)], 1u);
        }
        __syncthreads();
        // thread t owns bins [nb - (t+1)*bpt, nb - t*bpt): descending ownership
        const int bpt = nb / NT;                      // 2, 4 or 8
        const int b0 = nb - (tid + 1) * bpt;
        uint32_t hb[8];
        uint32_t c = 0;
        if (bpt >= 4) {
#pragma unroll
            for (int v = 0; v < 2; ++v) {
                if (v * 4 < bpt) {
                    const sel_u32x4 x = *reinterpret_cast<const sel_u32x4 *>(&h[b0 + 4 * v]);
                    hb[4 * v + 0] = x[0]; hb[4 * v + 1] = x[1]; hb[4 * v + 2] = x[2]; hb[4 * v + 3] = x[3];
                }
            }
        } else {
#pragma unroll
            for (int j = 0; j < 2; ++j) hb[j] = j < bpt ? h[b0 + j] : 0u;
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) c += j < bpt ? hb[j] : 0u;
        uint32_t total;
        const uint32_t above_me = block_exclusive<NT>(c, total, sc);
        if (pass == 0) {
            keff = total < kout ? total : kout;
            need = keff;
        }
        if (keff == 0) {
            __syncthreads();
            return SelectResult{0u, 0u, 0u};
        }
        if (above_me < need && above_me + c >= need) {
            uint32_t above = above_me;
            bool done = false;
#pragma unroll
            for (int j = 7; j >= 0; --j) {
                if (j < bpt && !done) {
                    if (above + hb[j] >= need) {
                        sc.digit = static_cast<uint32_t>(b0 + j);
                        sc.above = above;
                        sc.count = hb[j];
                        done = true;
                    } else {
                        above += hb[j];
                    }
                }
            }
        }
        __syncthreads();
        prefix |= sc.digit << shift;
        mask |= static_cast<uint32_t>(nb - 1) << shift;
        need -= sc.above;
        const uint32_t in_bin = sc.count;
        __syncthreads();   // digit/above/count and wave_tot are rewritten by the next pass
        // every key of the cutoff bin is kept: the kept set is exactly the keys
        // >= prefix (low bits still open), i.e. the keys > prefix - 1, with
        // none kept at equality -- no further pass needed
        if (pass < 2 && need == in_bin) return SelectResult{prefix == 0u ? 0u : prefix - 1u, 0u, keff};
    }
    return SelectResult{prefix, need, keff};
}

// Hands the thread's kept keys to emit(slot, r, key) (r = index into its
// run), given the counts of keys above K* and equal to K* in earlier runs.  A
// key above K* is kept at slot gt_before + min(eq_before, need_eq); a key
// equal to K* is kept while eq_before < need_eq, at slot gt_before + eq_before
// (the same expression).  Only the store is predicated.
template <int R, typename Emit>
__device__ __forceinline__ void emit_kept(const uint32_t (&kv)[R], const SelectResult &res, uint32_t gt_before,
                                          uint32_t eq_before, Emit &&emit) {
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const uint32_t key = kv[r];
        const bool gt = key > res.kstar, eq = key == res.kstar;
        const uint32_t op = gt_before + (eq_before < res.need_eq ? eq_before : res.need_eq);
        const bool keep = gt || (eq && eq_before < res.need_eq);
        gt_before += gt ? 1u : 0u;
        eq_before += eq ? 1u : 0u;
        if (keep && op < res.keff) emit(op, r, key);   // op < keff always holds for a kept key; guards the write
    }
}

// Slots for the kept keys, in position order; calls emit(slot, r, key) for
// the thread's kept keys (r = index into its run).
template <int NT, int R, typename Emit>
__device__ __forceinline__ void block_compact(const uint32_t (&kv)[R], const SelectResult &res,
                                              SelectScratch &sc, Emit &&emit) {
    uint32_t cg = 0, ce = 0;
#pragma unroll
    for (int r = 0; r < R; ++r) {
        cg += kv[r] > res.kstar;
        ce += kv[r] == res.kstar;
    }
    const uint32_t v = (cg << 16) | ce;                // per-block counts stay below 2^16
    uint32_t total;
    const uint32_t ex = block_exclusive<NT>(v, total, sc);
    emit_kept<R>(kv, res, ex >> 16, ex & 0xFFFFu, emit);
}

// ---------------------------------------------------------------- one wave
// Exact select for short rows (n <= 64*R), run by a single wave with no
// workgroup barriers and no LDS: lane l holds positions [l*Rd, l*Rd + Rd) of
// the row in kv[0..Rd).  The cutoff key K* (the largest v with
// #{key >= v} >= k_eff) is found bit by bit from the top: for each candidate
// prefix the wave counts the keys at or above it with one ballot and one
// population count per register, all on scalar registers -- at most 32
// short dependent steps instead of histogram passes through LDS.  The search
// stops as soon as exactly k_eff keys lie at or above the candidate.
template <int R>
__device__ __forceinline__ SelectResult wave_ballot_select(const uint32_t (&kv)[R], uint32_t kout) {
    uint32_t nvalid = 0;
#pragma unroll
    for (int r = 0; r < R; ++r) nvalid += static_cast<uint32_t>(__popcll(__ballot(kv[r] != kNoCandidate)));
    const uint32_t keff = nvalid < kout ? nvalid : kout;
    if (keff == 0) return SelectResult{0u, 0u, 0u};
    uint32_t prefix = 0;
    for (int bit = 31; bit >= 0; --bit) {
        const uint32_t cand = prefix | (1u << bit);
        uint32_t cnt = 0;
#pragma unroll
        for (int r = 0; r < R; ++r) cnt += static_cast<uint32_t>(__popcll(__ballot(kv[r] >= cand)));
        // exactly k_eff keys at or above cand: they are the kept set (keys > cand - 1)
        if (cnt == keff) return SelectResult{cand - 1u, 0u, keff};
        if (cnt > keff) prefix = cand;
    }
    uint32_t gt = 0;
#pragma unroll
    for (int r = 0; r < R; ++r) gt += static_cast<uint32_t>(__popcll(__ballot(kv[r] > prefix)));
    return SelectResult{prefix, keff - gt, keff};
}

template <int R, typename Emit>
__device__ __forceinline__ void wave_compact(const uint32_t (&kv)[R], const SelectResult &res,
                                             Emit &&emit) {
    uint32_t cg = 0, ce = 0;
#pragma unroll
    for (int r = 0; r < R; ++r) {
        cg += kv[r] > res.kstar;
        ce += kv[r] == res.kstar;
    }
    const uint32_t v = (cg << 16) | ce;
    const uint32_t ex = wave_prefix_incl(v) - v;
    emit_kept<R>(kv, res, ex >> 16, ex & 0xFFFFu, emit);
}

}  // namespace hisa
