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
// One wave alone (top m over at most 2048 block keys): wave_ballot_select
// finds K* bit by bit with ballots (about 110 cycles a round, 32 rounds), and
// wave_window_select takes one LDS histogram over the four binades below the
// best key instead, which costs less once a lane holds more than 4 keys.
//
// Costs on gfx950 that shaped this: LDS atomics to one address from many lanes
// serialize (about 16x a conflict-free one), cross-lane shuffles through LDS
// cost about 75 cycles each while DPP row operations cost a few, and 16-byte
// LDS reads whose lanes stride by 128 bytes conflict on every bank.  A
// workgroup's select over 8192 keys is bound by its one CU's vector ALUs and
// LDS (some 30 operations a key): a histogram range fitted to the keys
// measured no faster there (its extra reduction and barrier cost what the
// avoided contention saved); copies of the first histogram (NC) cut the
// contention without either.
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
// After the exchange each wave reads the NW wave totals with one lane-parallel
// LDS load (lane w takes wave w's) and scans them with DPP, rather than every
// thread reading all NW of them.
template <int NT>
__device__ __forceinline__ uint32_t block_exclusive(uint32_t v, uint32_t &total, SelectScratch &sc) {
    constexpr int NW = NT / 64;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const uint32_t incl = wave_prefix_incl(v);
    if (lane == 63) sc.wave_tot[wave] = incl;
    __syncthreads();
    const uint32_t wt = wave_prefix_incl(lane < NW ? sc.wave_tot[lane] : 0u);
    const uint32_t before =
        wave == 0 ? 0u : static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(wt), wave - 1));
    total = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(wt), NW - 1));
    return before + incl - v;
}

struct SelectResult {
    uint32_t kstar;      // key of the k_eff-th best candidate
    uint32_t need_eq;    // how many keys equal to kstar are kept
    uint32_t keff;       // number of kept keys
};

// The first digit's histogram in NC copies (NC = 1, 2 or 4), lane l adding
// into copy l % NC: the top 11 bits of clustered scores fall into a handful
// of bins, and LDS atomics of one wave to one address serialize, so spreading
// a bin over NC addresses (in different banks: copies kCopyStride words
// apart) divides that wait by up to NC.  h0 holds NC * kCopyStride words
// (unused when NC = 1: sc.hist serves).
constexpr int kCopyStride = kCoreBins0 + 16;

template <int NT, int R, int NC = 1>
__device__ __forceinline__ SelectResult block_radix_select(const uint32_t (&kv)[R], uint32_t kout,
                                                           SelectScratch &sc, uint32_t *h0 = nullptr) {
    static_assert(NC == 1 || NC == 2 || NC == 4, "histogram copies");
    const int tid = threadIdx.x;
    for (int b = tid * 4; b < kCoreBins0 + kCoreBins1 + kCoreBins2; b += NT * 4)
        *reinterpret_cast<sel_u32x4 *>(&sc.hist[b]) = sel_u32x4{0u, 0u, 0u, 0u};
    if (NC > 1)
        for (int b = tid * 4; b < NC * kCopyStride; b += NT * 4)
            *reinterpret_cast<sel_u32x4 *>(&h0[b]) = sel_u32x4{0u, 0u, 0u, 0u};
    __syncthreads();
    uint32_t prefix = 0, mask = 0, need = 0, keff = 0;
#pragma unroll
    for (int pass = 0; pass < 3; ++pass) {
        const int shift = pass == 0 ? 21 : (pass == 1 ? 10 : 0);
        constexpr int kNB[3] = {kCoreBins0, kCoreBins1, kCoreBins2};
        const int nb = kNB[pass];
        uint32_t *h = sc.hist + (pass == 0 ? 0 : (pass == 1 ? kCoreBins0 : kCoreBins0 + kCoreBins1));
        const int ncp = pass == 0 ? NC : 1;                // histogram copies of this pass
        if (pass == 0 && NC > 1) h = h0;
        uint32_t *ha = ncp > 1 ? h + (threadIdx.x & (ncp - 1)) * kCopyStride : h;
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const uint32_t key = kv[r];
            if (key != kNoCandidate && (key & mask) == prefix)
                atomicAdd(&ha[(key >> shift) & static_cast<uint32_t>(nb - 1)], 1u);
        }
        __syncthreads();
        // thread t owns bins [nb - (t+1)*bpt, nb - t*bpt): descending ownership
        const int bpt = nb / NT;                      // 2, 4 or 8
        const int b0 = nb - (tid + 1) * bpt;
        uint32_t hb[8];
        uint32_t c = 0;
#pragma unroll
        for (int j = 0; j < 8; ++j) hb[j] = 0u;
#pragma unroll
        for (int cp = 0; cp < (pass == 0 ? NC : 1); ++cp) {   // a bin's count: the sum over its copies
            const uint32_t *hc = h + cp * kCopyStride;
            if (bpt >= 4) {
#pragma unroll
                for (int v = 0; v < 2; ++v) {
                    if (v * 4 < bpt) {
                        const sel_u32x4 x = *reinterpret_cast<const sel_u32x4 *>(&hc[b0 + 4 * v]);
                        hb[4 * v + 0] += x[0]; hb[4 * v + 1] += x[1]; hb[4 * v + 2] += x[2]; hb[4 * v + 3] += x[3];
                    }
                }
            } else {
#pragma unroll
                for (int j = 0; j < 2; ++j) hb[j] += j < bpt ? hc[b0 + j] : 0u;
            }
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
        // No barrier here: the next pass rewrites wave_tot and digit/above/count
        // only after its histogram barrier, which every thread reaches after
        // these reads; after a return, block_compact rewrites only wave_tot,
        // whose reads all came before the barrier above.
        // every key of the cutoff bin is kept: the kept set is exactly the keys
        // >= prefix (low bits still open), i.e. the keys > prefix - 1, with
        // none kept at equality -- no further pass needed
        if (pass < 2 && need == in_bin) return SelectResult{prefix == 0u ? 0u : prefix - 1u, 0u, keff};
        // all 32 bits resolved: the bin holds the keys equal to K*; when every
        // one of them is kept the kept set is the keys > K* - 1 (K* >= 1: key 0
        // is no candidate), the form whose compaction needs no tie counts
        if (pass == 2 && need == in_bin) return SelectResult{prefix - 1u, 0u, keff};
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
    if (res.need_eq == 0) {
        // no key equal to K* is kept (block_radix_select returns every case
        // without a partial tie in this form): a key is kept iff it is > K*,
        // at slot = kept keys before it -- one compare a key instead of the
        // (greater, equal) pair below, the same slots
        uint32_t cg = 0;
#pragma unroll
        for (int r = 0; r < R; ++r) cg += kv[r] > res.kstar;
        uint32_t total;
        uint32_t op = block_exclusive<NT>(cg, total, sc);
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const uint32_t key = kv[r];
            if (key > res.kstar && op < res.keff) emit(op, r, key);   // op < keff always holds; guards the write
            op += key > res.kstar;
        }
        return;
    }
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

// Reduction across a 64-lane wave with DPP row shifts and row broadcasts;
// lanes past a row edge contribute `id`.  Every lane gets lane 63's result.
template <typename Op>
__device__ __forceinline__ uint32_t wave_reduce(uint32_t x, uint32_t id, Op op) {
    const int i = static_cast<int>(id);
    x = op(x, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(i, static_cast<int>(x), 0x111, 0xf, 0xf, false)));
    x = op(x, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(i, static_cast<int>(x), 0x112, 0xf, 0xf, false)));
    x = op(x, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(i, static_cast<int>(x), 0x114, 0xf, 0xf, false)));
    x = op(x, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(i, static_cast<int>(x), 0x118, 0xf, 0xf, false)));
    x = op(x, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(i, static_cast<int>(x), 0x142, 0xa, 0xf, false)));
    x = op(x, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(i, static_cast<int>(x), 0x143, 0xc, 0xf, false)));
    return static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(x), 63));
}

constexpr int kWindowWords = 2048 + 64;    // LDS words of one wave_window_select

// One-wave select with the contract of wave_ballot_select, through an LDS
// histogram fitted to the keys: no workgroup barrier, and a handful of short
// steps instead of up to 32 ballot rounds.
//   1. The largest key kmax (a DPP reduction).  The window [lo, kmax] with
//      lo = kmax - (4 << 23) holds the scores within a factor 16 of the
//      largest (subtracting 4 << 23 from a key divides a positive score by 16);
//      digit(key) = (key - lo) >> shift spreads it over 2048 bins.
//   2. A histogram of the window's keys (LDS atomics, spread over the bins);
//      lane l then owns 32 bins from the top, and a DPP prefix over the lanes'
//      counts gives the bin holding the k_eff-th key.
//   3. Every key of that bin kept, or the bin one key value: done.  Otherwise
//      its keys (at most 64) are gathered in LDS and ranked against each other,
//      one per lane.
// Fewer than k_eff keys in the window, or more than 64 in the cutoff bin: the
// ballot select does it instead.  lds: kWindowWords words of LDS that no
// other wave touches meanwhile.
template <int R>
__device__ __forceinline__ SelectResult wave_window_select(const uint32_t (&kv)[R], uint32_t kout, uint32_t *lds) {
    constexpr int kBins = 2048;
    const int lane = threadIdx.x & 63;
    uint32_t nvalid = 0, mx = 0u;
#pragma unroll
    for (int r = 0; r < R; ++r) {
        nvalid += static_cast<uint32_t>(__popcll(__ballot(kv[r] != kNoCandidate)));
        mx = kv[r] > mx ? kv[r] : mx;
    }
    const uint32_t keff = nvalid < kout ? nvalid : kout;
    if (keff == 0 || keff == nvalid) return SelectResult{0u, 0u, keff};   // nothing, or every key > 0
    const uint32_t kmax = wave_reduce(mx, 0u, [](uint32_t a, uint32_t b) { return a > b ? a : b; });
    constexpr uint32_t kWindow = 4u << 23;
    const uint32_t lo = kmax > kWindow ? kmax - kWindow : 1u;
    const int bits = 32 - __clz(kmax - lo);
    const int shift = bits > 11 ? bits - 11 : 0;
    uint32_t *hist = lds, *bin = lds + kBins;
#pragma unroll
    for (int i = 0; i < kBins / 256; ++i)
        *reinterpret_cast<sel_u32x4 *>(&hist[(i * 64 + lane) * 4]) = sel_u32x4{0u, 0u, 0u, 0u};
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
#pragma unroll
    for (int r = 0; r < R; ++r)
        if (kv[r] != kNoCandidate && kv[r] >= lo) atomicAdd(&hist[(kv[r] - lo) >> shift], 1u);
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
    // lane l owns bins [kBins - 32(l+1), kBins - 32 l), highest first
    uint32_t hb[32];
    const int b0 = kBins - 32 * (lane + 1);
#pragma unroll
    for (int v = 0; v < 8; ++v) {
        const sel_u32x4 x = *reinterpret_cast<const sel_u32x4 *>(&hist[b0 + 4 * v]);
        hb[4 * v + 0] = x[0]; hb[4 * v + 1] = x[1]; hb[4 * v + 2] = x[2]; hb[4 * v + 3] = x[3];
    }
    uint32_t c = 0;
#pragma unroll
    for (int j = 0; j < 32; ++j) c += hb[j];
    const uint32_t incl = wave_prefix_incl(c);
    const uint32_t total = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(incl), 63));
    if (total < keff) return wave_ballot_select<R>(kv, kout);    // the cutoff lies below the window
    const uint32_t above_me = incl - c;
    // the lane whose bins hold the k_eff-th key finds the bin
    uint32_t dig = 0, abv = 0, cnt = 0;
    const bool mine = above_me < keff && above_me + c >= keff;
    if (mine) {
        uint32_t above = above_me;
        bool done = false;
#pragma unroll
        for (int j = 31; j >= 0; --j) {
            if (!done) {
                if (above + hb[j] >= keff) {
                    dig = static_cast<uint32_t>(b0 + j);
                    abv = above;
                    cnt = hb[j];
                    done = true;
                } else {
                    above += hb[j];
                }
            }
        }
    }
    const int owner = __builtin_ctzll(__ballot(mine));
    const uint32_t dstar = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(dig), owner));
    const uint32_t need = keff - static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(abv), owner));
    const uint32_t in_bin = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(cnt), owner));
    const uint32_t blo = lo + (dstar << shift);
    if (need == in_bin) return SelectResult{blo - 1u, 0u, keff};   // the keys >= blo
    if (shift == 0) return SelectResult{blo, need, keff};         // the bin is one key value
    if (in_bin > 64u) return wave_ballot_select<R>(kv, kout);
    // gather the bin's keys into LDS (slots by ballot prefix), one per lane
    uint32_t base = 0;
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const bool inb = kv[r] != kNoCandidate && kv[r] >= lo && ((kv[r] - lo) >> shift) == dstar;
        const uint64_t bal = __ballot(inb);
        if (inb) bin[base + __builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(bal >> 32),
                                                      __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(bal), 0u))] = kv[r];
        base += static_cast<uint32_t>(__popcll(bal));
    }
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
    // lane j ranks bin key j against the others (broadcast from their lanes):
    // K* has fewer than `need` keys above it and at least `need` at or above it
    const uint32_t me = static_cast<uint32_t>(lane) < in_bin ? bin[lane] : 0u;
    uint32_t gt = 0, ge = 0;
    for (uint32_t i = 0; i < in_bin; ++i) {
        const uint32_t o = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(me), static_cast<int>(i)));
        gt += o > me ? 1u : 0u;
        ge += o >= me ? 1u : 0u;
    }
    const bool is_k = static_cast<uint32_t>(lane) < in_bin && gt < need && ge >= need;
    const int kl = __builtin_ctzll(__ballot(is_k));
    const uint32_t kstar = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(me), kl));
    const uint32_t gtk = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(gt), kl));
    return SelectResult{kstar, need - gtk, keff};
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
