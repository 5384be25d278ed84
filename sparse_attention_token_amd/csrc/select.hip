// Exact top-k selection over per-query candidate keys.
//
// Both stages of the pages' method end in a "keep the best" step -- the top m
// blocks after block scoring, then the final top k tokens of the refinement
// (gptget.net English summary, "Methodology"; Chinese summary, method
// details) -- and the flat indexer ends in a top k over the whole prefix.  All
// of them use one rule: rank by (score desc, index asc), keep
// min(k, #candidates), pad with -1.  Scores arrive as order-preserving uint32
// keys (0 = no candidate), laid out by increasing candidate index.
// The three-level tree adds one more such step: the top m blocks among those
// of its kept super-blocks (tree-blocks mode, ids mapped like refine mode's
// with the super-block table and G blocks per slot).
//
// One workgroup (1024 threads) selects over up to 32768 positions of one
// query: thread t holds positions [t*R, t*R + R) in registers and
// block_radix_select / block_compact (select_core.h) do the rest.  Longer rows
// are cut into chunks of 32768 positions; each chunk keeps its own top k as
// (key, id) pairs in position order, and the next stage selects over the
// concatenation.  This is exact: a member of the row's top k has fewer than k
// better keys in its chunk, so it survives its chunk's stage, and chunk
// outputs stay in increasing index order, so ties still resolve by index.

#include "hisa_internal.h"
#include "select_core.h"

namespace hisa {
namespace {

constexpr int kNT = 1024;
constexpr int kChunkMax = kNT * 32;
constexpr int kNarrowNT = 512;          // select workgroup size when there are many queries (prefill top k: 115 -> 99 us against 256)
constexpr int kManyQueries = 1024;

// number of candidate positions of query qi for a mode (0 for an invalid t)
template <int MODE>
__device__ __forceinline__ int64_t row_length(const SelectArgs &a, int qi) {
    const int s = qi / a.T;
    const int64_t t = query_pos(a.qpos, qi, qi - s * a.T, a.L, a.T);
    if (t < 0) return 0;
    const int64_t bt = t / a.B;
    if (MODE == kScoreBlocks) return bt + 1;
    if (MODE == kScoreRefine) return ((a.m < bt + 1) ? a.m : bt + 1) * a.B;
    if (MODE == kScoreTreeBlocks) {
        const int64_t ns = bt / a.G + 1;
        return (a.m < ns ? a.m : ns) * a.G;
    }
    return t + 1;
}

// Modes whose positions are slot*grp + r over a table of kept parents.
template <int MODE>
constexpr bool kMapped = MODE == kScoreRefine || MODE == kScoreTreeBlocks;

template <int MODE>
__device__ __forceinline__ int group_size(const SelectArgs &a) {
    return MODE == kScoreTreeBlocks ? a.G : a.B;
}

// Store to element `op` of a row through a 32-bit byte offset (op < 2^30
// always: rows hold at most k entries), which lets the base stay in scalar
// registers instead of forming a 64-bit address per element.
template <typename T>
__device__ __forceinline__ void put(T *row, uint32_t op, T v) {
    *reinterpret_cast<T *>(reinterpret_cast<char *>(row) + (op << 2)) = v;
}

template <int R>
__device__ __forceinline__ void load_run(const uint32_t *__restrict__ keys, int64_t base, int64_t n,
                                         uint32_t (&kv)[R]) {
    if constexpr (R >= 4) {
        // every load is issued (past the row end it reads the row's first
        // keys, masked below): a load under a branch can make the wave wait
        // for it at once
#pragma unroll
        for (int v = 0; v < R / 4; ++v) {
            const int64_t p = base + 4 * v;
            const sel_u32x4 x = *reinterpret_cast<const sel_u32x4 *>(keys + (p < n ? p : 0));   // rows are padded to 64 keys
#pragma unroll
            for (int e = 0; e < 4; ++e) kv[4 * v + e] = (p + e < n) ? x[e] : kNoCandidate;
        }
    } else {
#pragma unroll
        for (int r = 0; r < R; ++r) kv[r] = (base + r < n) ? keys[base + r] : kNoCandidate;
    }
}

// A thread's run of R keys, loaded from the row's address and stride alone:
// every load stays inside the row's padded stride (a multiple of 64 keys),
// so none waits for the row length, which comes from the argument struct;
// mask_run then marks positions >= n as no candidate.
template <int R>
__device__ __forceinline__ void load_run_early(const uint32_t *__restrict__ row, int64_t base, int64_t stride,
                                               uint32_t (&kv)[R]) {
    if constexpr (R >= 4) {
#pragma unroll
        for (int v = 0; v < R / 4; ++v) {
            const int64_t p = base + 4 * v;
            const sel_u32x4 x = *reinterpret_cast<const sel_u32x4 *>(row + (p < stride ? p : 0));
#pragma unroll
            for (int e = 0; e < 4; ++e) kv[4 * v + e] = x[e];
        }
    } else {
#pragma unroll
        for (int r = 0; r < R; ++r) kv[r] = row[base + r < stride ? base + r : 0];
    }
}

template <int R>
__device__ __forceinline__ void mask_run(int64_t base, int64_t n, uint32_t (&kv)[R]) {
#pragma unroll
    for (int r = 0; r < R; ++r) kv[r] = base + r < n ? kv[r] : kNoCandidate;
}

// Single-stage select: the whole row (n <= NT*R) in one workgroup of NT
// threads (1024 for latency with few queries, 512 for throughput with many).
// STAGE: the kept (id, key) pairs are first written to LDS at their slots,
// then the row is stored with consecutive threads on consecutive entries
// (kout <= kStageOut), instead of each thread storing its kept keys where
// they fall.  Same-box A/B: the prefill chunk's top k (4096 queries, 512
// threads each) 94 -> 66.5 us; decode 128K 9.5 -> 9.25 us; decode 32K
// unchanged.
constexpr int kStageOut = 2048;
// A kept entry staged in LDS: (id, key) in one 64-bit word, one LDS write per
// kept key rather than two.
typedef uint32_t stage_u32x2 __attribute__((ext_vector_type(2)));
// Workgroups of 1024 threads count the first digit into four histogram
// copies (block_radix_select's NC): the decode top k's first pass took 1,730
// cycles instead of 2,430.  512-thread workgroups (many queries) keep one
// copy, whose LDS lets more workgroups share a compute unit.
template <int NT>
constexpr int kFirstCopies = NT == 1024 ? 4 : 1;

// The key rows' address and stride come first among the arguments, which
// this file's build preloads into scalar registers at dispatch: the key loads
// issue at once instead of after a memory round trip for the arguments
// (1,230 cycles in the decode top k), and the rest of the struct arrives
// while they are in flight.
template <int MODE, int R, int NT, bool STAGE>
__global__ __launch_bounds__(NT) void select_kernel(const uint32_t *__restrict__ keys, int64_t keys_stride,
                                                    SelectArgs a) {
    __shared__ __attribute__((aligned(16))) SelectScratch sc;
    __shared__ int32_t s_sel[kSelMaxM];
    __shared__ stage_u32x2 s_out[STAGE ? kStageOut : 1];       // (id, key) by output slot
    __shared__ __attribute__((aligned(16))) uint32_t s_h0[kFirstCopies<NT> > 1 ? kFirstCopies<NT> * kCopyStride : 4];
    const int tid = threadIdx.x;
    const int qi = blockIdx.x;
    uint32_t kv[R];
    load_run_early<R>(keys + static_cast<int64_t>(qi) * keys_stride, static_cast<int64_t>(tid) * R, keys_stride, kv);
    const int64_t n = row_length<MODE>(a, qi);
    mask_run<R>(static_cast<int64_t>(tid) * R, n, kv);
    int32_t *out = a.out_id + static_cast<int64_t>(qi) * a.kout;
    float *osc = a.out_score ? a.out_score + static_cast<int64_t>(qi) * a.kout : nullptr;
    int32_t *out2 = a.out_id_copy ? a.out_id_copy + static_cast<int64_t>(qi) * a.kout : nullptr;
    const int grp = group_size<MODE>(a);
    if (kMapped<MODE>) {
        const int meff = static_cast<int>(n / grp);
        for (int j = tid; j < meff; j += NT) s_sel[j] = a.sel_blk[static_cast<int64_t>(qi) * a.m + j];
        // block_radix_select starts with a barrier, which also publishes s_sel
    }
    const SelectResult res = block_radix_select<NT, R, kFirstCopies<NT>>(kv, static_cast<uint32_t>(a.kout), sc, s_h0);
    if (res.keff > 0) {
        // mapped modes: R and the group size are powers of two, so with
        // R <= grp the thread's R positions lie in one slot and one lookup
        // serves them all; with R > grp each position looks up its slot
        const bool per_pos = kMapped<MODE> && R > grp;
        const int lg = __builtin_ctz(static_cast<unsigned>(grp));      // grp is a power of two
        int32_t id0 = tid * R;
        if (kMapped<MODE> && !per_pos && id0 < n) id0 = s_sel[id0 >> lg] * grp + (id0 & (grp - 1));
        block_compact<NT, R>(kv, res, sc, [&](uint32_t op, int r, uint32_t key) {
            int32_t id = id0 + r;
            if (per_pos) id = s_sel[id >> lg] * grp + (id & (grp - 1));
            if (STAGE) {
                s_out[op] = stage_u32x2{static_cast<uint32_t>(id), key};
            } else {
                put(out, op, id);
                if (osc) put(osc, op, key_to_score(key));
                if (out2) put(out2, op, id);
            }
        });
    }
    if (STAGE) {
        __syncthreads();
        for (int j = tid; j < a.kout; j += NT) {
            const bool kept = j < static_cast<int>(res.keff);
            const stage_u32x2 e = s_out[kept ? j : 0];
            const int32_t id = kept ? static_cast<int32_t>(e[0]) : -1;
            out[j] = id;
            if (osc) osc[j] = kept ? key_to_score(e[1]) : -__builtin_huge_valf();
            if (out2) out2[j] = id;
        }
        return;
    }
    for (int j = static_cast<int>(res.keff) + tid; j < a.kout; j += NT) {
        out[j] = -1;
        if (osc) osc[j] = -__builtin_huge_valf();
        if (out2) out2[j] = -1;
    }
}

// Chunk stage: grid (nchunk, nq).  Input row: keys (and ids, or positions
// mapped by MODE when ids_in is null) of length n_fixed, or the mode's row
// length when n_fixed < 0; output: for each chunk, its top kout (key, id)
// pairs in position order, padded with key 0.
template <int MODE>
__global__ __launch_bounds__(kNT) void select_chunk_kernel(SelectArgs a, const uint32_t *keys_in,
                                                           const int32_t *ids_in, int64_t in_stride,
                                                           int64_t n_fixed, uint32_t *keys_out,
                                                           int32_t *ids_out, int64_t out_stride) {
    __shared__ __attribute__((aligned(16))) SelectScratch sc;
    __shared__ stage_u32x2 s_out[kStageOut];        // (id, key) by output slot
    __shared__ __attribute__((aligned(16))) uint32_t s_h0[kFirstCopies<kNT> * kCopyStride];
    constexpr int R = 32;
    const int tid = threadIdx.x;
    const int qi = blockIdx.y;
    const int64_t n_row = n_fixed >= 0 ? n_fixed : row_length<MODE>(a, qi);
    const int64_t c0 = static_cast<int64_t>(blockIdx.x) * kChunkMax;
    const int64_t n = n_row - c0 < kChunkMax ? n_row - c0 : kChunkMax;   // may be <= 0
    const uint32_t *krow = keys_in + static_cast<int64_t>(qi) * in_stride + c0;
    uint32_t kv[R];
    load_run<R>(krow, static_cast<int64_t>(tid) * R, n > 0 ? n : 0, kv);
    uint32_t *ko = keys_out + static_cast<int64_t>(qi) * out_stride + static_cast<int64_t>(blockIdx.x) * a.kout;
    int32_t *io = ids_out + static_cast<int64_t>(qi) * out_stride + static_cast<int64_t>(blockIdx.x) * a.kout;
    const bool stage = a.kout <= kStageOut;          // staged output, as in select_kernel
    const SelectResult res = block_radix_select<kNT, R, kFirstCopies<kNT>>(kv, static_cast<uint32_t>(a.kout), sc, s_h0);
    if (res.keff > 0) {
        const int32_t *irow = ids_in ? ids_in + static_cast<int64_t>(qi) * in_stride + c0 : nullptr;
        // position ids in the mapped modes: with R <= grp (both powers of
        // two; chunks start on slot bounds) the thread's R positions lie in
        // one slot; with grp < R each position looks up its slot
        const int grp = group_size<MODE>(a);
        const int64_t p0 = c0 + static_cast<int64_t>(tid) * R;
        const int32_t *sb = a.sel_blk + static_cast<int64_t>(qi) * a.m;
        const bool per_pos = !irow && kMapped<MODE> && R > grp;
        int32_t id0 = static_cast<int32_t>(p0);
        if (!irow && kMapped<MODE> && !per_pos && p0 < n_row) {
            const int64_t slot = p0 >> __builtin_ctz(static_cast<unsigned>(grp));   // grp is a power of two
            id0 = static_cast<int32_t>(static_cast<int64_t>(sb[slot]) * grp + (p0 & (grp - 1)));
        }
        block_compact<kNT, R>(kv, res, sc, [&](uint32_t op, int r, uint32_t key) {
            int32_t id;
            if (irow) {
                id = irow[static_cast<int64_t>(tid) * R + r];
            } else if (per_pos) {
                const int64_t pos = p0 + r;
                const int64_t slot = pos >> __builtin_ctz(static_cast<unsigned>(grp));
                id = static_cast<int32_t>(static_cast<int64_t>(sb[slot]) * grp + (pos & (grp - 1)));
            } else {
                id = id0 + r;
            }
            if (stage) {
                s_out[op] = stage_u32x2{static_cast<uint32_t>(id), key};
            } else {
                put(ko, op, key);
                put(io, op, id);
            }
        });
    }
    if (stage) {
        __syncthreads();
        for (int j = tid; j < a.kout; j += kNT) {
            const bool kept = j < static_cast<int>(res.keff);
            const stage_u32x2 e = s_out[kept ? j : 0];
            ko[j] = kept ? e[1] : kNoCandidate;
            io[j] = kept ? static_cast<int32_t>(e[0]) : -1;
        }
        return;
    }
    for (int j = static_cast<int>(res.keff) + tid; j < a.kout; j += kNT) {
        ko[j] = kNoCandidate;
        io[j] = -1;
    }
}

// Final stage over (key, id) pairs: writes the output row.
__global__ __launch_bounds__(kNT) void select_final_kernel(SelectArgs a, const uint32_t *keys_in,
                                                           const int32_t *ids_in, int64_t in_stride,
                                                           int64_t n) {
    __shared__ __attribute__((aligned(16))) SelectScratch sc;
    __shared__ stage_u32x2 s_out[kStageOut];        // (id, key) by output slot
    __shared__ __attribute__((aligned(16))) uint32_t s_h0[kFirstCopies<kNT> * kCopyStride];
    constexpr int R = 32;
    const int tid = threadIdx.x;
    const int qi = blockIdx.x;
    uint32_t kv[R];
    load_run<R>(keys_in + static_cast<int64_t>(qi) * in_stride, static_cast<int64_t>(tid) * R, n, kv);
    int32_t *out = a.out_id + static_cast<int64_t>(qi) * a.kout;
    float *osc = a.out_score ? a.out_score + static_cast<int64_t>(qi) * a.kout : nullptr;
    int32_t *out2 = a.out_id_copy ? a.out_id_copy + static_cast<int64_t>(qi) * a.kout : nullptr;
    const int32_t *irow = ids_in + static_cast<int64_t>(qi) * in_stride;
    const bool stage = a.kout <= kStageOut;          // staged output, as in select_kernel
    const SelectResult res = block_radix_select<kNT, R, kFirstCopies<kNT>>(kv, static_cast<uint32_t>(a.kout), sc, s_h0);
    if (res.keff > 0) {
        block_compact<kNT, R>(kv, res, sc, [&](uint32_t op, int r, uint32_t key) {
            const int32_t id = irow[tid * R + r];
            if (stage) {
                s_out[op] = stage_u32x2{static_cast<uint32_t>(id), key};
            } else {
                put(out, op, id);
                if (osc) put(osc, op, key_to_score(key));
                if (out2) put(out2, op, id);
            }
        });
    }
    if (stage) {
        __syncthreads();
        for (int j = tid; j < a.kout; j += kNT) {
            const bool kept = j < static_cast<int>(res.keff);
            const stage_u32x2 e = s_out[kept ? j : 0];
            const int32_t id = kept ? static_cast<int32_t>(e[0]) : -1;
            out[j] = id;
            if (osc) osc[j] = kept ? key_to_score(e[1]) : -__builtin_huge_valf();
            if (out2) out2[j] = id;
        }
        return;
    }
    for (int j = static_cast<int>(res.keff) + tid; j < a.kout; j += kNT) {
        out[j] = -1;
        if (osc) osc[j] = -__builtin_huge_valf();
        if (out2) out2[j] = -1;
    }
}

template <int MODE>
hipError_t launch_single(KernelKind kind, const SelectArgs &a, int nq, int64_t max_n, hipStream_t st) {
    const dim3 g(nq);
    if (nq >= kManyQueries && max_n <= kNarrowNT * 32) {
        const dim3 b(kNarrowNT);
        const int64_t per = (max_n + kNarrowNT - 1) / kNarrowNT;
        if (a.kout <= kStageOut) {
            if (per <= 4) return launch(kind, select_kernel<MODE, 4, kNarrowNT, true>, g, b, 0, st, static_cast<const uint32_t *>(a.keys), a.keys_stride, a);
            if (per <= 8) return launch(kind, select_kernel<MODE, 8, kNarrowNT, true>, g, b, 0, st, static_cast<const uint32_t *>(a.keys), a.keys_stride, a);
            if (per <= 16) return launch(kind, select_kernel<MODE, 16, kNarrowNT, true>, g, b, 0, st, static_cast<const uint32_t *>(a.keys), a.keys_stride, a);
            return launch(kind, select_kernel<MODE, 32, kNarrowNT, true>, g, b, 0, st, static_cast<const uint32_t *>(a.keys), a.keys_stride, a);
        }
        if (per <= 4) return launch(kind, select_kernel<MODE, 4, kNarrowNT, false>, g, b, 0, st, static_cast<const uint32_t *>(a.keys), a.keys_stride, a);
        if (per <= 8) return launch(kind, select_kernel<MODE, 8, kNarrowNT, false>, g, b, 0, st, static_cast<const uint32_t *>(a.keys), a.keys_stride, a);
        if (per <= 16) return launch(kind, select_kernel<MODE, 16, kNarrowNT, false>, g, b, 0, st, static_cast<const uint32_t *>(a.keys), a.keys_stride, a);
        return launch(kind, select_kernel<MODE, 32, kNarrowNT, false>, g, b, 0, st, static_cast<const uint32_t *>(a.keys), a.keys_stride, a);
    }
    const dim3 b(kNT);
    const int64_t per = (max_n + kNT - 1) / kNT;
    if (a.kout <= kStageOut) {
        if (per <= 1) return launch(kind, select_kernel<MODE, 1, kNT, true>, g, b, 0, st, static_cast<const uint32_t *>(a.keys), a.keys_stride, a);
        if (per <= 2) return launch(kind, select_kernel<MODE, 2, kNT, true>, g, b, 0, st, static_cast<const uint32_t *>(a.keys), a.keys_stride, a);
        if (per <= 4) return launch(kind, select_kernel<MODE, 4, kNT, true>, g, b, 0, st, static_cast<const uint32_t *>(a.keys), a.keys_stride, a);
        if (per <= 8) return launch(kind, select_kernel<MODE, 8, kNT, true>, g, b, 0, st, static_cast<const uint32_t *>(a.keys), a.keys_stride, a);
        if (per <= 16) return launch(kind, select_kernel<MODE, 16, kNT, true>, g, b, 0, st, static_cast<const uint32_t *>(a.keys), a.keys_stride, a);
        return launch(kind, select_kernel<MODE, 32, kNT, true>, g, b, 0, st, static_cast<const uint32_t *>(a.keys), a.keys_stride, a);
    }
    if (per <= 1) return launch(kind, select_kernel<MODE, 1, kNT, false>, g, b, 0, st, static_cast<const uint32_t *>(a.keys), a.keys_stride, a);
    if (per <= 2) return launch(kind, select_kernel<MODE, 2, kNT, false>, g, b, 0, st, static_cast<const uint32_t *>(a.keys), a.keys_stride, a);
    if (per <= 4) return launch(kind, select_kernel<MODE, 4, kNT, false>, g, b, 0, st, static_cast<const uint32_t *>(a.keys), a.keys_stride, a);
    if (per <= 8) return launch(kind, select_kernel<MODE, 8, kNT, false>, g, b, 0, st, static_cast<const uint32_t *>(a.keys), a.keys_stride, a);
    if (per <= 16) return launch(kind, select_kernel<MODE, 16, kNT, false>, g, b, 0, st, static_cast<const uint32_t *>(a.keys), a.keys_stride, a);
    return launch(kind, select_kernel<MODE, 32, kNT, false>, g, b, 0, st, static_cast<const uint32_t *>(a.keys), a.keys_stride, a);
}

template <int MODE>
hipError_t launch_chunked(KernelKind kind, const SelectArgs &a, int nq, int64_t max_n, hipStream_t st) {
    // stage 1 over the raw keys, then chunk stages over (key, id) pairs until
    // one workgroup can finish the row
    uint32_t *bufk[2] = {a.stage_keys[0], a.stage_keys[1]};
    int32_t *bufi[2] = {a.stage_ids[0], a.stage_ids[1]};
    int64_t nchunk = (max_n + kChunkMax - 1) / kChunkMax;
    hipError_t e = launch(kind, select_chunk_kernel<MODE>, dim3(static_cast<uint32_t>(nchunk), nq),
                          dim3(kNT), 0, st, a, static_cast<const uint32_t *>(a.keys),
                          static_cast<const int32_t *>(nullptr), a.keys_stride, int64_t{-1}, bufk[0],
                          bufi[0], a.stage_stride);
    if (e != hipSuccess) return e;
    int cur = 0;
    int64_t n = nchunk * a.kout;
    while (n > kChunkMax) {
        nchunk = (n + kChunkMax - 1) / kChunkMax;
        e = launch(kind, select_chunk_kernel<MODE>, dim3(static_cast<uint32_t>(nchunk), nq), dim3(kNT), 0,
                   st, a, static_cast<const uint32_t *>(bufk[cur]), static_cast<const int32_t *>(bufi[cur]),
                   a.stage_stride, n, bufk[1 - cur], bufi[1 - cur], a.stage_stride);
        if (e != hipSuccess) return e;
        cur = 1 - cur;
        n = nchunk * a.kout;
    }
    return launch(kind, select_final_kernel, dim3(nq), dim3(kNT), 0, st, a,
                  static_cast<const uint32_t *>(bufk[cur]), static_cast<const int32_t *>(bufi[cur]),
                  a.stage_stride, n);
}

}  // namespace

int64_t select_stage_len(int64_t max_n, int kout, int B, bool refine) {
    const bool chunked = max_n > kChunkMax || (refine && max_n / B > kSelMaxM);
    if (!chunked) return 0;
    // the first stage is the longest: one kout-row per chunk of the input
    return (max_n + kChunkMax - 1) / kChunkMax * static_cast<int64_t>(kout);
}

hipError_t launch_select(ScoreMode mode, const SelectArgs &a, int nq, int64_t max_n, hipStream_t st) {
    const KernelKind kind = mode == kScoreBlocks ? kKindSelectBlocks
                          : mode == kScoreRefine ? kKindSelectRefine
                          : mode == kScoreTreeBlocks ? kKindSelectTree : kKindSelectFlat;
    const bool tree = mode == kScoreTreeBlocks;
    if (select_stage_len(max_n, a.kout, tree ? a.G : a.B, mode == kScoreRefine || tree) > 0) {
        if (mode == kScoreBlocks) return launch_chunked<kScoreBlocks>(kind, a, nq, max_n, st);
        if (mode == kScoreRefine) return launch_chunked<kScoreRefine>(kind, a, nq, max_n, st);
        if (tree) return launch_chunked<kScoreTreeBlocks>(kind, a, nq, max_n, st);
        return launch_chunked<kScoreFlat>(kind, a, nq, max_n, st);
    }
    if (mode == kScoreBlocks) return launch_single<kScoreBlocks>(kind, a, nq, max_n, st);
    if (mode == kScoreRefine) return launch_single<kScoreRefine>(kind, a, nq, max_n, st);
    if (tree) return launch_single<kScoreTreeBlocks>(kind, a, nq, max_n, st);
    return launch_single<kScoreFlat>(kind, a, nq, max_n, st);
}

}  // namespace hisa
