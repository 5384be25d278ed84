// The HISA indexing path with the block stage fused into one kernel.
//
// The pages' procedure (gptget.net English summary, "Methodology"; Chinese
// summary, method details): score the mean-pooled block representatives with
// the original indexer, keep the top m blocks, re-score every token of the kept
// blocks with the original indexer, keep the top k tokens.
//
// Block stage (block_stage(), one workgroup, all in LDS):
//    * every wave scores pooled means of the complete blocks b < b_t with the
//      shared MFMA scorer (its first tile loads are issued before anything
//      else, to overlap HBM latency with the staging below);
//    * q is staged in LDS; the rows of the query's own block b_t = t / B
//      (rows b_t*B .. t) are summed by all threads, each over a run of rows
//      of two columns, into the own-block representative
//      bf16(fp32(fp64 sum in row order / count)) -- the same arithmetic and
//      bits as the block pool (OwnRowsPar, block_rep.h), so the pool entry of
//      the own block is never read -- and it is scored like the others;
//    * the top min(m, b_t + 1) blocks (ascending ids) are then selected: by
//      one wave when b_t + 1 <= 2048 (no barriers), by the whole workgroup
//      otherwise.
// Ways to run it, chosen by the host:
//  * decode (few queries), short context: hisa_decode_kernel -- one
//    workgroup per 256 (or, with few queries, 128) candidate positions of a
//    query, 8 waves when the grid has at most one workgroup per compute unit
//    and 4 otherwise (position p = slot*B + r: row r of the
//    slot-th kept block, masked past t).  Each workgroup repeats its query's
//    block stage (the pooled means it reads are shared through L2) and then
//    scores its 128 rows: one launch, no communication between workgroups.
//  * decode, longer context: hisa_dblocks_kernel scores the pooled means once
//    per query (one workgroup per 128 of them), and hisa_dgather_kernel keeps
//    the top m from the block keys and scores its candidate rows.
//  * batch (many queries): hisa_blocks_topm_kernel runs the block stage once
//    per query and writes the kept blocks; hisa_refine_kernel then scores
//    128-row tiles with q staged in LDS.
//  * more than 2048 blocks, query by query (decode past 256K keys at B = 128,
//    and batches): hisa_dblocks_kernel as in decode, the top m as a
//    selection launch, then hisa_refine_kernel.
//  * many queries per sequence (prefill chunks): block stage and refinement
//    both block by block (hisa_prefill.hip).
// Either way the final top k runs as the selection kernel (select.hip).
// Limits (checked by the host): B*d <= 16384, ceil(L/B) <= 8192; decode mode
// also ceil(L/B) <= 2048 and m <= 1024.

#include "block_rep.h"
#include "hisa_internal.h"
#include "scorer.h"
#include "select_core.h"

namespace hisa {
namespace {

constexpr int kK1Threads = 1024;
constexpr int kK1R = kFusedMaxBlocks / kK1Threads;        // block keys per thread, block-wide select
constexpr int kK1WaveMax = 64 * 32;                       // rows the one-wave select takes
constexpr int kK2Threads = 256;
constexpr int kDecodeThreads = 256;
constexpr int kDecodeMaxM = 1024;                         // kept blocks staged in LDS (decode mode)
// Decode mode repeats the block stage in every tile's workgroup, which stops
// paying off with more queries.  Measured per step at 32K keys (one launch
// against the general blocks + refine path): 8 queries 27.4 vs 28.4 us,
// 16 queries 31.8 vs 31.9 us, 24 queries 45.5 vs 37.9 us.
constexpr int kDecodeMaxQueries = 16;
constexpr int kDecodeRowsWide = 256;                      // candidate rows per decode workgroup, big grids
constexpr int kDecodeRowsNarrow = 128;                    // ... and when fewer than kDecodeWideMin would run
constexpr int kDecodeWideMin = 256;
// Grids of at most this many workgroups (one per compute unit) run the decode
// kernel with 8 waves per workgroup instead of 4.  Measured per step at 32K
// keys: 8 queries 25.0 -> 21.8 us; 16 queries (512 workgroups) 29.2 -> 33.8 us,
// so larger grids keep 4 waves.
constexpr int kDecodeEightWaveMaxGrid = 256;
// Up to this many blocks every decode workgroup repeats the block stage (one
// launch); beyond it the block stage runs once per query in its own kernel.
// Measured per step: 256 blocks 28.8 vs 29.7 us, 512 blocks 30.6 vs 28.9,
// 1025 blocks 48.4 vs 40.7 (one launch vs two); with the arguments preloaded
// at dispatch, 512 blocks (4 queries) 21.0 vs 18.9 us.
constexpr int kDecodeOneKernelMaxBlocks = 256;

// LDS slot of block position p: the keys are stored so that the select's
// owner of a contiguous run of positions reads it as conflict-free rows.
__device__ __forceinline__ int k1_slot(int p, int nb) {
    if (nb <= kK1WaveMax) {
        const int rd = (nb + 63) / 64;                        // positions per lane
        return (p % rd) * 64 + p / rd;
    }
    return (p % kK1R) * kK1Threads + p / kK1R;
}

template <int R, typename Emit>
__device__ __forceinline__ uint32_t k1_wave_select(const uint32_t *s_keys, int nb, int m, uint32_t *win, Emit &emit) {
    const int lane = threadIdx.x & 63;
    const int rd = (nb + 63) / 64;
    uint32_t kv[R];
#pragma unroll
    for (int r = 0; r < R; ++r) kv[r] = (r < rd && lane * rd + r < nb) ? s_keys[r * 64 + lane] : kNoCandidate;
    // up to 256 keys the ballot select's 32 short rounds cost less than the
    // histogram's set-up; beyond, its rounds grow with R and the window wins
    const SelectResult res = R <= 4 ? wave_ballot_select<R>(kv, static_cast<uint32_t>(m))
                                    : wave_window_select<R>(kv, static_cast<uint32_t>(m), win);
    if (res.keff > 0)
        wave_compact<R>(kv, res, [&](uint32_t op, int r, uint32_t) { emit(op, lane * rd + r); });
    return res.keff;
}

template <int KS, int NT>
struct BlockStageLds {
    static constexpr int kOwnWords = kFusedOwnElems / 2;
    uint16_t q[64 * QStage<KS>::kStride];
    float w[64];                        // head weights, zero past H
    uint32_t own[kOwnWords];            // own-block rows; after the block stage, the top m's window
    uint16_t mean[128];
};

// Scores every block b <= b_t of one query into s_keys (positions laid out by
// k1_slot) and leaves the query fragments in f.  NT threads; each wave loads
// TB pool tiles at a time (the first batch before anything else, so that HBM
// latency overlaps the staging of q and the loads of the own-block rows, which
// go straight into registers and are summed by all NT threads: at decode
// 32K the block stage took about 800 cycles less than with the rows staged in
// LDS and summed column by column by 128 threads); ends with a barrier.  For the query at the cache's last row (t = L-1) the pool entry of
// its own block is already the mean of rows b_t*B .. t (the pool is current
// through row L-1), so it is scored like the others; any other query's own
// block is recomputed from K.
// With a.pool_out set, every own block is recomputed from K, and when
// writer is true the query at t = L-1 also stores its own block's mean into
// the pool.
template <int MT, int KS, int NT, int TB>
__device__ __forceinline__ void block_stage(const FusedArgs &a, int qi, int s, int64_t t,
                                            BlockStageLds<KS, NT> &L, uint32_t *s_keys,
                                            QFrag<MT, KS> &f, bool writer, bool pool_out_set) {
    constexpr int D = 32 * KS;
    constexpr int NW = NT / 64;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int n = lane & 15, g = lane >> 4;
    const int64_t bt = t / a.B;
    const int nb = static_cast<int>(bt + 1);
    const int64_t r0 = bt * a.B;
    const int own_rows = static_cast<int>(t + 1 - r0);
    const bool own_in_pool = t == a.L - 1 && !pool_out_set;
    const bool write_pool = writer && pool_out_set && t == a.L - 1;
    using Own = OwnRowsPar<D, NT>;
    static_assert(sizeof(typename Own::Scratch) <= sizeof(L.own), "own-block scratch fits the staging words");
    auto &osc = *reinterpret_cast<typename Own::Scratch *>(L.own);
    const uint16_t *own_src = a.K + s * a.k_seq_stride + r0 * D;

    // pool rows 0 .. full-1, 16 per tile, tile i on wave i % NW
    const uint16_t *pool = a.pool + s * a.pool_seq_stride;
    const int full = own_in_pool ? nb : static_cast<int>(bt);
    const int ntiles = (full + 15) / 16;
    bf16x8 kb[TB][KS];
#pragma unroll
    for (int u = 0; u < TB; ++u) {
        const int p = (wave + u * NW) * 16 + n;
        load_row_frag_any<KS>(kb[u], pool + static_cast<int64_t>(p < full ? p : 0) * D, lane);
    }
    Own own;
    if (!own_in_pool) own.load(own_src, own_rows, tid);   // own-block rows: in flight with the pool tiles
    QStager<MT, KS, NT> qst;
    qst.load(a.q + static_cast<int64_t>(qi) * a.H * D, a.H, tid);
    const float wq = a.w[static_cast<int64_t>(qi) * a.H + (lane < a.H ? lane : a.H - 1)];
    pin_loaded(wq);                     // issued with q, not behind the wait for it
    qst.store(L.q, a.H, tid);
    if (tid < 64) L.w[tid] = tid < a.H ? wq : 0.0f;
    if (!own_in_pool) {
        if (a.pool_max)
            own.template partial<true>(own_rows, tid, osc);
        else
            own.template partial<false>(own_rows, tid, osc);
    }
    __syncthreads();
    if (!own_in_pool && tid < D) {
        // own-block representative over rows b_t*B .. t (the block pool's arithmetic)
        uint16_t *dst = write_pool ? a.pool_out + s * a.pool_seq_stride + bt * D : nullptr;
        if (a.pool_max)
            own.template combine<true>(own_src, own_rows, tid, osc, L.mean, dst);
        else
            own.template combine<false>(own_src, own_rows, tid, osc, L.mean, dst);
    }

    load_qfrag_lds_w<MT, KS>(f, L.q, L.w, lane);
    for (int base = wave; base < ntiles; base += TB * NW) {
        if (base != wave) {
#pragma unroll
            for (int u = 0; u < TB; ++u) {
                const int p = (base + u * NW) * 16 + n;
                load_row_frag_any<KS>(kb[u], pool + static_cast<int64_t>(p < full ? p : 0) * D, lane);
            }
        }
#pragma unroll
        for (int u = 0; u < TB; ++u) {
            const int tile = base + u * NW;
            if (tile < ntiles) {
                const int p = tile * 16 + n;
                const float v = score_rows<MT, KS>(f, kb[u]);
                if (g == 0 && p < full) s_keys[k1_slot(p, nb)] = score_to_key(v);
            }
        }
    }

    if (!own_in_pool) {
        __syncthreads();                  // the own-block representative is in L.mean
        if (wave == 0) {
            bf16x8 kbm[KS];
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) kbm[ks] = n == 0 ? load_bf16x8(L.mean + 32 * ks + 8 * g) : zero_bf16x8();
            const float v = score_rows<MT, KS>(f, kbm);
            if (lane == 0) s_keys[k1_slot(nb - 1, nb)] = score_to_key(v);
        }
    }
    __syncthreads();
}

// One wave selects the top m of the nb <= 2048 block keys; emit(slot, block).
// win: kWindowWords words of LDS for the select's histogram.
template <typename Emit>
__device__ __forceinline__ uint32_t block_topm_wave(const uint32_t *s_keys, int nb, int m, uint32_t *win,
                                                    Emit &&emit) {
    const int rd = (nb + 63) / 64;
    uint32_t ke;
    if (rd <= 4) ke = k1_wave_select<4>(s_keys, nb, m, win, emit);
    else if (rd <= 8) ke = k1_wave_select<8>(s_keys, nb, m, win, emit);
    else if (rd <= 16) ke = k1_wave_select<16>(s_keys, nb, m, win, emit);
    else ke = k1_wave_select<32>(s_keys, nb, m, win, emit);
    return ke;
}

template <int MT, int KS>
__global__ __launch_bounds__(kK1Threads) void hisa_blocks_topm_kernel(FusedArgs a) {
    __shared__ __attribute__((aligned(16))) BlockStageLds<KS, kK1Threads> L;
    __shared__ __attribute__((aligned(16))) uint32_t s_keys[kFusedMaxBlocks];   // by k1_slot()
    __shared__ __attribute__((aligned(16))) SelectScratch sc;
    __shared__ uint32_t s_keff;

    const int tid = threadIdx.x, wave = tid >> 6;
    const int qi = blockIdx.x;
    const int s = qi / a.T;
    const int64_t t = query_pos(a.qpos, qi, qi - s * a.T, a.L, a.T);
    int32_t *sel = a.sel_blk + static_cast<int64_t>(qi) * a.m;
    int32_t *ob = a.out_blk ? a.out_blk + static_cast<int64_t>(qi) * a.m : nullptr;
    if (t < 0) {
        for (int j = tid; j < a.m; j += kK1Threads) {
            sel[j] = -1;
            if (ob) ob[j] = -1;
        }
        return;
    }
    const int nb = static_cast<int>(t / a.B + 1);
    QFrag<MT, KS> f;
    block_stage<MT, KS, kK1Threads, 1>(a, qi, s, t, L, s_keys, f, true, a.pool_out != nullptr);

    uint32_t keff;
    if (nb <= kK1WaveMax) {
        // short rows: one wave, no barriers
        if (wave == 0) {
            const uint32_t ke = block_topm_wave(s_keys, nb, a.m, L.own, [&](uint32_t op, int pos) {
                sel[op] = pos;
                if (ob) ob[op] = pos;
            });
            if ((tid & 63) == 0) s_keff = ke;
        }
        __syncthreads();
        keff = s_keff;
    } else {
        uint32_t kv[kK1R];
#pragma unroll
        for (int r = 0; r < kK1R; ++r) kv[r] = tid * kK1R + r < nb ? s_keys[r * kK1Threads + tid] : kNoCandidate;
        const SelectResult res = block_radix_select<kK1Threads, kK1R>(kv, static_cast<uint32_t>(a.m), sc);
        if (res.keff > 0) {
            block_compact<kK1Threads, kK1R>(kv, res, sc, [&](uint32_t op, int r, uint32_t) {
                const int pos = tid * kK1R + r;
                sel[op] = pos;
                if (ob) ob[op] = pos;
            });
        }
        keff = res.keff;
    }
    for (int j = static_cast<int>(keff) + tid; j < a.m; j += kK1Threads) {
        sel[j] = -1;
        if (ob) ob[j] = -1;
    }
}

// Workgroup -> (query qi, tile) in decode mode, tiles = ceil(m*B/ROWS) per
// query.  Workgroups are dealt to the 8 XCDs in turn (linear id i goes to XCD
// i % 8), so the mapping keeps each query's workgroups on as few XCDs as
// possible: all of them share that L2's copy of the query, its pooled means
// and its gathered rows.  qi = -1: nothing to do.
__host__ __device__ inline int decode_grid(int nq, int tiles) {
    if (nq % 8 == 0) return nq * tiles;
    if (8 % nq == 0) {
        const int per = 8 / nq;                      // XCDs per query
        return 8 * ((tiles + per - 1) / per);
    }
    return nq * tiles;
}

__device__ __forceinline__ void decode_tile(int nq, int tiles, int &qi, int &tile) {
    const int i = blockIdx.x, x = i & 7, j = i >> 3;
    if (nq % 8 == 0) {
        qi = x + 8 * (j / tiles);
        tile = j - (j / tiles) * tiles;
    } else if (8 % nq == 0) {
        const int per = 8 / nq;
        qi = x % nq;
        tile = j * per + x / nq;
        if (tile >= tiles) qi = -1;
    } else {
        qi = i / tiles;
        tile = i - qi * tiles;
    }
}

// Decode mode: grid decode_grid(S*T, ceil(m*B/ROWS)), DT threads (256 or 512).  Block stage, top-m
// into LDS, then the workgroup's ROWS candidate rows (ROWS/64 16-row tiles per
// wave).  Wider workgroups repeat the block stage less often; narrow ones keep
// every CU busy when there are few queries.
// Decode kernels take everything a workgroup needs before its first loads
// as leading arguments, which this file's build preloads into scalar
// registers at dispatch: their first loads go out without waiting a memory
// round trip for the argument block (the rest of FusedArgs still comes from
// it).  Packed words: pk = T | H << 8 | log2(B) << 16 | queries << 20,
// pk2 = n2 | m << 12 | (qpos null) << 24 | (pool_out set) << 25, where n2 is
// the kernel's own count (tiles per query, or pooled means).
struct DecodeEarly {
    int nq, n2;
    bool qpos_null, pool_out_set;
};

__device__ __forceinline__ DecodeEarly decode_early(FusedArgs &a, const uint16_t *q, const uint16_t *K,
                                                    const float *w, int32_t k_seq_stride, int32_t Lk, uint32_t pk,
                                                    uint32_t pk2) {
    a.q = q; a.K = K; a.w = w; a.k_seq_stride = k_seq_stride; a.L = Lk;
    a.T = static_cast<int>(pk & 0xffu);
    a.H = static_cast<int>((pk >> 8) & 0xffu);
    a.B = 1 << ((pk >> 16) & 0xfu);
    a.m = static_cast<int>((pk2 >> 12) & 0xfffu);
    return DecodeEarly{static_cast<int>((pk >> 20) & 0xffu), static_cast<int>(pk2 & 0xfffu),
                       ((pk2 >> 24) & 1u) != 0, ((pk2 >> 25) & 1u) != 0};
}

// query_pos() without reading qpos from the argument block when it is null
__device__ __forceinline__ int64_t decode_pos(const FusedArgs &a, const DecodeEarly &e, int qi, int i) {
    if (e.qpos_null) {
        const int64_t t = a.L - a.T + i;
        return t >= 0 && t < a.L ? t : -1;
    }
    return query_pos(a.qpos, qi, i, a.L, a.T);
}

// Early arguments (decode_early): n2 = tiles per query.
template <int MT, int KS, int ROWS, int DT>
__global__ __launch_bounds__(DT) void hisa_decode_kernel(const uint16_t *q, const uint16_t *pool, const uint16_t *K,
                                                         const float *w, int32_t k_seq_stride, int32_t pool_seq_stride,
                                                         int32_t Lk, uint32_t pk, uint32_t pk2, FusedArgs a_in) {
    FusedArgs a = a_in;
    const DecodeEarly e = decode_early(a, q, K, w, k_seq_stride, Lk, pk, pk2);
    a.pool = pool; a.pool_seq_stride = pool_seq_stride;
    const bool pool_out_set = e.pool_out_set;
    constexpr int D = 32 * KS;
    constexpr int NTW = ROWS / (16 * DT / 64);
    __shared__ __attribute__((aligned(16))) BlockStageLds<KS, DT> L;
    __shared__ __attribute__((aligned(16))) uint32_t s_keys[kK1WaveMax];        // by k1_slot()
    __shared__ int32_t s_sel[kDecodeMaxM];
    __shared__ uint32_t s_keff;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int n = lane & 15, g = lane >> 4;
    int qi, tile;
    decode_tile(e.nq, e.n2, qi, tile);
    if (qi < 0) return;
    const int s = qi / a.T;
    const int64_t t = decode_pos(a, e, qi, qi - s * a.T);
    const bool lead = tile == 0;            // also publishes the kept blocks
    if (t < 0) {
        if (lead)
            for (int j = tid; j < a.m; j += DT) {
                a.sel_blk[static_cast<int64_t>(qi) * a.m + j] = -1;
                if (a.out_blk) a.out_blk[static_cast<int64_t>(qi) * a.m + j] = -1;
            }
        return;
    }
    const int64_t bt = t / a.B;
    const int nb = static_cast<int>(bt + 1);
    const int meff = a.m < nb ? a.m : nb;
    const int npos = meff * a.B;
    const int tile0 = tile * ROWS;
    if (tile0 >= npos) return;

    QFrag<MT, KS> f;
    block_stage<MT, KS, DT, DT == 256 ? 4 : 2>(a, qi, s, t, L, s_keys, f, lead, pool_out_set);
    // output rows from the argument block: formed after the block stage, so
    // that no wait for it comes before the stage's first loads
    int32_t *sel = a.sel_blk + static_cast<int64_t>(qi) * a.m;
    int32_t *ob = a.out_blk ? a.out_blk + static_cast<int64_t>(qi) * a.m : nullptr;
    if (wave == 0) {
        const uint32_t ke = block_topm_wave(s_keys, nb, a.m, L.own, [&](uint32_t op, int pos) {
            s_sel[op] = pos;
            if (lead) {
                sel[op] = pos;
                if (ob) ob[op] = pos;
            }
        });
        if (lane == 0) s_keff = ke;
    }
    __syncthreads();
    if (lead)
        for (int j = static_cast<int>(s_keff) + tid; j < a.m; j += DT) {
            sel[j] = -1;
            if (ob) ob[j] = -1;
        }

    // this workgroup's candidate rows: NTW 16-row tiles per wave, every load
    // in flight before any is scored
    bf16x8 kb[NTW][KS];
    bool valid[NTW];
#pragma unroll
    for (int nt = 0; nt < NTW; ++nt) {
        const int p = tile0 + (wave * NTW + nt) * 16 + n;
        const int pc = p < npos ? p : npos - 1;         // npos >= 1: tile0 < npos
        const int slot = pc >> __builtin_ctz(a.B);      // B is a power of two
        const int64_t tok = static_cast<int64_t>(s_sel[slot]) * a.B + (pc & (a.B - 1));
        valid[nt] = p < npos && tok <= t;
        load_row_frag_any<KS>(kb[nt], a.K + s * a.k_seq_stride + (tok <= t ? tok : t) * D, lane);
    }
    // every row load is issued before the first MFMA: left to itself the
    // scheduler issued five of the eight, waited for the first and issued the
    // rest between MFMAs, one more memory round trip for those three
    __builtin_amdgcn_sched_barrier(0);
    float v[NTW];
    score_tiles_frag<MT, KS, NTW>(f, kb, v);
    uint32_t *cand = a.cand_keys + static_cast<int64_t>(qi) * a.cand_stride;
#pragma unroll
    for (int nt = 0; nt < NTW; ++nt) {
        const int p = tile0 + (wave * NTW + nt) * 16 + n;
        if (g == 0 && p < npos) cand[p] = valid[nt] ? score_to_key(v[nt]) : kNoCandidate;
    }
}

// ---------------------------------------------------------------- decode, two kernels
// Long contexts make every decode workgroup's own copy of the block stage
// expensive (1025 pooled means per workgroup at 128K), so the block stage runs
// once per query in hisa_dblocks_kernel -- one workgroup per (query, 128
// pooled means), writing block keys -- and hisa_dgather_kernel reads a
// query's n_b keys, keeps the top m with the one-wave select and scores its
// candidate rows.
constexpr int kDBlkRows = 128;

// Grid decode_grid(S*T, ceil(nblk/128) + 1): per query, one workgroup per 128
// pooled means, plus one (the last) for the own block when it is not taken
// from the pool -- its rows are staged and averaged in a workgroup of their
// own, in parallel with the pool tiles.
// Early arguments (decode_early): n2 = pooled means per sequence (nblk).
// EARLY = false (more blocks or queries than the packed words hold): the
// leading arguments are ignored and everything comes from a_in.
template <int MT, int KS, bool EARLY>
__global__ __launch_bounds__(kDecodeThreads) void hisa_dblocks_kernel(const uint16_t *q, const uint16_t *pool,
                                                                      const uint16_t *K, const float *w,
                                                                      int32_t k_seq_stride, int32_t pool_seq_stride,
                                                                      int32_t Lk, uint32_t pk, uint32_t pk2,
                                                                      FusedArgs a_in) {
    constexpr int D = 32 * KS;
    constexpr int NTW = kDBlkRows / (16 * kDecodeThreads / 64);
    __shared__ __attribute__((aligned(16))) BlockStageLds<KS, kDecodeThreads> L;
    FusedArgs a = a_in;
    DecodeEarly e{a.S * a.T, a.nblk, a.qpos == nullptr, a.pool_out != nullptr};
    if constexpr (EARLY) {
        e = decode_early(a, q, K, w, k_seq_stride, Lk, pk, pk2);
        a.pool = pool; a.pool_seq_stride = pool_seq_stride; a.nblk = e.n2;
    }
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int n = lane & 15, g = lane >> 4;
    const int btiles = (a.nblk + kDBlkRows - 1) / kDBlkRows;
    int qi, j;
    decode_tile(e.nq, btiles + 1, qi, j);
    if (qi < 0) return;
    const int s = qi / a.T;
    const int64_t t = decode_pos(a, e, qi, qi - s * a.T);
    if (t < 0) return;
    const int bt = static_cast<int>(t / a.B);
    // the pool entry of b_t is the own-block mean unless this call writes it
    const bool own_in_pool = t == a.L - 1 && !e.pool_out_set;
    const int full = own_in_pool ? bt + 1 : bt;    // pool rows to score
    const bool own_wg = j == btiles;
    if (own_wg ? own_in_pool : j * kDBlkRows >= full) return;

    if (!own_wg) {
        const int b0 = j * kDBlkRows;
        const uint16_t *pool = a.pool + s * a.pool_seq_stride;
        bf16x8 kb[NTW][KS];
#pragma unroll
        for (int nt = 0; nt < NTW; ++nt) {
            const int p = b0 + (wave * NTW + nt) * 16 + n;
            load_row_frag_any<KS>(kb[nt], pool + static_cast<int64_t>(p < full ? p : 0) * D, lane);
        }
        QStager<MT, KS, kDecodeThreads> qst;
        qst.load(a.q + static_cast<int64_t>(qi) * a.H * D, a.H, tid);
        const float wq = a.w[static_cast<int64_t>(qi) * a.H + (tid < a.H ? tid : a.H - 1)];
        pin_loaded(wq);
        qst.store(L.q, a.H, tid);
        if (tid < 64) L.w[tid] = tid < a.H ? wq : 0.0f;
        __syncthreads();
        QFrag<MT, KS> f;
        load_qfrag_lds_w<MT, KS>(f, L.q, L.w, lane);
        float v[NTW];
        score_tiles_frag<MT, KS, NTW>(f, kb, v);
        uint32_t *keys = a.blk_keys + static_cast<int64_t>(qi) * a.blk_stride;
#pragma unroll
        for (int nt = 0; nt < NTW; ++nt) {
            const int p = b0 + (wave * NTW + nt) * 16 + n;
            if (g == 0 && p < full) keys[p] = score_to_key(v[nt]);
        }
        return;
    }

    // the own block: rows b_t*B .. t summed by all threads (OwnRowsPar), their
    // loads in flight with those of q and w
    const int64_t r0 = static_cast<int64_t>(bt) * a.B;
    const int own_rows = static_cast<int>(t + 1 - r0);
    using Own = OwnRowsPar<D, kDecodeThreads>;
    static_assert(sizeof(typename Own::Scratch) <= sizeof(L.own), "own-block scratch fits the staging words");
    auto &osc = *reinterpret_cast<typename Own::Scratch *>(L.own);
    const uint16_t *own_src = a.K + s * a.k_seq_stride + r0 * D;
    Own own;
    own.load(own_src, own_rows, tid);
    QStager<MT, KS, kDecodeThreads> qst;
    qst.load(a.q + static_cast<int64_t>(qi) * a.H * D, a.H, tid);
    const float wq0 = a.w[static_cast<int64_t>(qi) * a.H + (tid < a.H ? tid : a.H - 1)];   // unconditional load
    const float wq = tid < a.H ? wq0 : 0.0f;
    pin_loaded(wq0);
    qst.store(L.q, a.H, tid);
    if (tid < 64) L.w[tid] = wq;
    if (a.pool_max)
        own.template partial<true>(own_rows, tid, osc);
    else
        own.template partial<false>(own_rows, tid, osc);
    __syncthreads();
    if (tid < D) {
        uint16_t *dst = a.pool_out != nullptr && t == a.L - 1
                            ? a.pool_out + s * a.pool_seq_stride + static_cast<int64_t>(bt) * D
                            : nullptr;
        if (a.pool_max)
            own.template combine<true>(own_src, own_rows, tid, osc, L.mean, dst);
        else
            own.template combine<false>(own_src, own_rows, tid, osc, L.mean, dst);
    }
    __syncthreads();
    if (wave == 0) {
        QFrag<MT, KS> f;
        load_qfrag_lds_w<MT, KS>(f, L.q, L.w, lane);
        bf16x8 kbm[KS];
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) kbm[ks] = n == 0 ? load_bf16x8(L.mean + 32 * ks + 8 * g) : zero_bf16x8();
        const float vo = score_rows<MT, KS>(f, kbm);
        if (lane == 0) a.blk_keys[static_cast<int64_t>(qi) * a.blk_stride + bt] = score_to_key(vo);
    }
}

template <int R, typename Emit>
__device__ __forceinline__ uint32_t dgather_topm(const uint32_t *keys, int nb, int m, int lane, uint32_t *win,
                                                 Emit &&emit) {
    const int rd = (nb + 63) / 64;
    uint32_t kv[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const int p = lane * rd + r;
        kv[r] = (r < rd && p < nb) ? keys[p] : kNoCandidate;
    }
    const SelectResult res = R <= 4 ? wave_ballot_select<R>(kv, static_cast<uint32_t>(m))
                                    : wave_window_select<R>(kv, static_cast<uint32_t>(m), win);
    if (res.keff > 0) wave_compact<R>(kv, res, [&](uint32_t op, int r, uint32_t) { emit(op, lane * rd + r); });
    return res.keff;
}

// Early arguments (decode_early): n2 = tiles per query; the block keys'
// address and row stride take the places of the pool's.
template <int MT, int KS, int ROWS>
__global__ __launch_bounds__(kDecodeThreads) void hisa_dgather_kernel(const uint16_t *q, const uint32_t *blk_keys,
                                                                      const uint16_t *K, const float *w,
                                                                      int32_t k_seq_stride, int32_t blk_stride,
                                                                      int32_t Lk, uint32_t pk, uint32_t pk2,
                                                                      FusedArgs a_in) {
    constexpr int D = 32 * KS;
    constexpr int NTW = ROWS / (16 * kDecodeThreads / 64);
    __shared__ __attribute__((aligned(16))) uint16_t s_q[64 * QStage<KS>::kStride];
    __shared__ float s_w[64];
    __shared__ int32_t s_sel[kDecodeMaxM];
    __shared__ __attribute__((aligned(16))) uint32_t s_win[kWindowWords];
    __shared__ uint32_t s_keff;

    FusedArgs a = a_in;
    const DecodeEarly e = decode_early(a, q, K, w, k_seq_stride, Lk, pk, pk2);
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int n = lane & 15, g = lane >> 4;
    int qi, tile;
    decode_tile(e.nq, e.n2, qi, tile);
    if (qi < 0) return;
    const int s = qi / a.T;
    const int64_t t = decode_pos(a, e, qi, qi - s * a.T);
    const bool lead = tile == 0;            // also publishes the kept blocks
    if (t < 0) {
        if (lead)
            for (int j = tid; j < a.m; j += kDecodeThreads) {
                a.sel_blk[static_cast<int64_t>(qi) * a.m + j] = -1;
                if (a.out_blk) a.out_blk[static_cast<int64_t>(qi) * a.m + j] = -1;
            }
        return;
    }
    const int nb = static_cast<int>(t / a.B + 1);
    const int meff = a.m < nb ? a.m : nb;
    const int npos = meff * a.B;
    const int tile0 = tile * ROWS;
    if (tile0 >= npos) return;

    // q and w are loaded while wave 0 reads the block keys and selects
    QStager<MT, KS, kDecodeThreads> qst;
    qst.load(a.q + static_cast<int64_t>(qi) * a.H * D, a.H, tid);
    const float wq0 = a.w[static_cast<int64_t>(qi) * a.H + (tid < a.H ? tid : a.H - 1)];   // unconditional load
    const float wq = tid < a.H ? wq0 : 0.0f;
    if (wave == 0) {
        const uint32_t *keys = blk_keys + static_cast<int64_t>(qi) * blk_stride;
        auto emit = [&](uint32_t op, int pos) {
            s_sel[op] = pos;
            if (lead) {
                // output rows from the argument block, formed here (after the
                // key loads) so that no wait for it comes before them
                a.sel_blk[static_cast<int64_t>(qi) * a.m + op] = pos;
                if (a.out_blk) a.out_blk[static_cast<int64_t>(qi) * a.m + op] = pos;
            }
        };
        const int rd = (nb + 63) / 64;
        uint32_t ke;
        // the ballot select's work grows with R: above 16 keep R close to rd
        // (1025 blocks, rd = 17: R = 20 took the kernel from 17.3 to 13.9 us;
        // R = 12 for rd = 9 was slower than 16)
        if (rd <= 4) ke = dgather_topm<4>(keys, nb, a.m, lane, s_win, emit);
        else if (rd <= 8) ke = dgather_topm<8>(keys, nb, a.m, lane, s_win, emit);
        else if (rd <= 16) ke = dgather_topm<16>(keys, nb, a.m, lane, s_win, emit);
        else if (rd <= 20) ke = dgather_topm<20>(keys, nb, a.m, lane, s_win, emit);
        else if (rd <= 24) ke = dgather_topm<24>(keys, nb, a.m, lane, s_win, emit);
        else ke = dgather_topm<32>(keys, nb, a.m, lane, s_win, emit);
        if (lane == 0) s_keff = ke;
    }
    pin_loaded(wq0);
    qst.store(s_q, a.H, tid);
    if (tid < 64) s_w[tid] = wq;
    __syncthreads();
    if (lead)
        for (int j = static_cast<int>(s_keff) + tid; j < a.m; j += kDecodeThreads) {
            a.sel_blk[static_cast<int64_t>(qi) * a.m + j] = -1;
            if (a.out_blk) a.out_blk[static_cast<int64_t>(qi) * a.m + j] = -1;
        }

    bf16x8 kb[NTW][KS];
    bool valid[NTW];
#pragma unroll
    for (int nt = 0; nt < NTW; ++nt) {
        const int p = tile0 + (wave * NTW + nt) * 16 + n;
        const int pc = p < npos ? p : npos - 1;         // npos >= 1: tile0 < npos
        const int slot = pc >> __builtin_ctz(a.B);      // B is a power of two
        const int64_t tok = static_cast<int64_t>(s_sel[slot]) * a.B + (pc & (a.B - 1));
        valid[nt] = p < npos && tok <= t;
        load_row_frag_any<KS>(kb[nt], a.K + s * a.k_seq_stride + (tok <= t ? tok : t) * D, lane);
    }
    __builtin_amdgcn_sched_barrier(0);                  // every row load in flight before the MFMAs
    QFrag<MT, KS> f;
    load_qfrag_lds_w<MT, KS>(f, s_q, s_w, lane);
    float v[NTW];
    score_tiles_frag<MT, KS, NTW>(f, kb, v);
    uint32_t *cand = a.cand_keys + static_cast<int64_t>(qi) * a.cand_stride;
#pragma unroll
    for (int nt = 0; nt < NTW; ++nt) {
        const int p = tile0 + (wave * NTW + nt) * 16 + n;
        if (g == 0 && p < npos) cand[p] = valid[nt] ? score_to_key(v[nt]) : kNoCandidate;
    }
}

template <int MT, int KS>
__global__ __launch_bounds__(kK2Threads) void hisa_refine_kernel(FusedArgs a) {
    constexpr int D = 32 * KS;
    __shared__ __attribute__((aligned(16))) uint16_t s_q[64 * QStage<KS>::kStride];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int n = lane & 15, g = lane >> 4;
    const int qi = blockIdx.y;
    const int s = qi / a.T;
    const int64_t t = query_pos(a.qpos, qi, qi - s * a.T, a.L, a.T);
    if (t < 0) return;
    const int64_t bt = t / a.B;
    const int meff = static_cast<int>(a.m < bt + 1 ? a.m : bt + 1);
    const int npos = meff * a.B;
    const int tile0 = blockIdx.x * 128;
    if (tile0 >= npos) return;
    const int32_t *selq = a.sel_blk + static_cast<int64_t>(qi) * a.m;
    uint32_t *cand = a.cand_keys + static_cast<int64_t>(qi) * a.cand_stride;

    // rows first (they come from HBM), then q through LDS
    bf16x8 kb[2][KS];
    bool valid[2];
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
        const int p = tile0 + wave * 32 + nt * 16 + n;
        const int pc = p < npos ? p : npos - 1;         // npos >= 1: tile0 < npos
        const int slot = pc >> __builtin_ctz(a.B);      // B is a power of two
        const int64_t tok = static_cast<int64_t>(selq[slot]) * a.B + (pc & (a.B - 1));
        valid[nt] = p < npos && tok <= t;
        load_row_frag_any<KS>(kb[nt], a.K + s * a.k_seq_stride + (tok <= t ? tok : t) * D, lane);
    }
    stage_query<MT, KS, kK2Threads>(a.q + static_cast<int64_t>(qi) * a.H * D, a.H, s_q, tid);
    __syncthreads();
    QFrag<MT, KS> f;
    load_qfrag_lds<MT, KS>(f, s_q, a.w + static_cast<int64_t>(qi) * a.H, a.H, lane);
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
        const int p = tile0 + wave * 32 + nt * 16 + n;
        const float v = score_rows<MT, KS>(f, kb[nt]);
        if (g == 0 && p < npos) cand[p] = valid[nt] ? score_to_key(v) : kNoCandidate;
    }
}

// More blocks than the one-wave top m takes, query by query: the block scores
// are spread over workgroups (hisa_dblocks_kernel, which also stores the
// fused pool entry), the top m is a selection launch of its own, then the
// refinement.  A single workgroup per query (hisa_blocks_topm_kernel) would
// score thousands of pooled means one tile after another.
template <int MT, int KS>
hipError_t launch_wide_blocks(const FusedArgs &a, dim3 g2, hipStream_t st) {
    const int nq = a.S * a.T;
    const int btiles = (a.nblk + kDBlkRows - 1) / kDBlkRows;
    hipError_t e = launch(kKindScoreBlocks, hisa_dblocks_kernel<MT, KS, false>,
                          dim3(static_cast<uint32_t>(decode_grid(nq, btiles + 1))), dim3(kDecodeThreads), 0, st,
                          static_cast<const uint16_t *>(nullptr), static_cast<const uint16_t *>(nullptr),
                          static_cast<const uint16_t *>(nullptr), static_cast<const float *>(nullptr), 0, 0, 0, 0u, 0u, a);
    if (e != hipSuccess) return e;
    SelectArgs se{};
    se.keys = a.blk_keys; se.keys_stride = a.blk_stride;
    se.qpos = a.qpos; se.L = a.L; se.T = a.T; se.B = a.B; se.m = a.m;
    se.kout = a.m; se.out_id = a.sel_blk; se.out_id_copy = a.out_blk;
    e = launch_select(kScoreBlocks, se, nq, a.nblk, st);
    if (e != hipSuccess) return e;
    return launch(kKindScoreRefine, hisa_refine_kernel<MT, KS>, g2, dim3(kK2Threads), 0, st, a);
}

template <int MT, int KS>
hipError_t launch_fused_ks(const FusedArgs &a, bool decode, hipStream_t st) {
    const int nq = a.S * a.T;
    const dim3 g2(static_cast<uint32_t>((static_cast<int64_t>(a.m) * a.B + 127) / 128), nq);
    if (!a.bucket_off && a.nblk > kK1WaveMax) return launch_wide_blocks<MT, KS>(a, g2, st);
    if (decode) {
        const int64_t mb = static_cast<int64_t>(a.m) * a.B;
        const int wide = static_cast<int>((mb + kDecodeRowsWide - 1) / kDecodeRowsWide);
        const int narrow = static_cast<int>((mb + kDecodeRowsNarrow - 1) / kDecodeRowsNarrow);
        const bool use_wide = static_cast<int64_t>(wide) * nq >= kDecodeWideMin;
        // the decode kernels take the sequence strides as 32-bit preloaded
        // arguments (decode_early); caches laid out wider take the batch path
        // below.  decode_mode() admits only S*T <= 16, H <= 64, m <= 1024, so
        // the packed words hold every count (tiles <= 2048, nblk <= 2048).
        const bool strides32 = a.k_seq_stride < (int64_t{1} << 31) && a.pool_seq_stride < (int64_t{1} << 31) &&
                               a.blk_stride < (int64_t{1} << 31);
        if (strides32) {
            const uint32_t pk = static_cast<uint32_t>(a.T) | static_cast<uint32_t>(a.H) << 8 |
                                static_cast<uint32_t>(__builtin_ctz(static_cast<unsigned>(a.B))) << 16 |
                                static_cast<uint32_t>(nq) << 20;
            const uint32_t flags = (a.qpos == nullptr ? 1u : 0u) << 24 | (a.pool_out != nullptr ? 1u : 0u) << 25 |
                                   static_cast<uint32_t>(a.m) << 12;
            const int32_t kss = static_cast<int32_t>(a.k_seq_stride), pss = static_cast<int32_t>(a.pool_seq_stride);
            const int32_t bstride = static_cast<int32_t>(a.blk_stride), Lk = static_cast<int32_t>(a.L);
            if (a.nblk > kDecodeOneKernelMaxBlocks) {
                // long context: block stage once per query, then the gather
                const int btiles = (a.nblk + kDBlkRows - 1) / kDBlkRows;
                const hipError_t e = launch(kKindScoreBlocks, hisa_dblocks_kernel<MT, KS, true>,
                                            dim3(static_cast<uint32_t>(decode_grid(nq, btiles + 1))),
                                            dim3(kDecodeThreads), 0, st, a.q, a.pool, a.K, a.w, kss, pss, Lk, pk,
                                            flags | static_cast<uint32_t>(a.nblk), a);
                if (e != hipSuccess) return e;
                const int tiles = use_wide ? wide : narrow;
                const dim3 grid(static_cast<uint32_t>(decode_grid(nq, tiles)));
                const uint32_t pk2 = flags | static_cast<uint32_t>(tiles);
                const uint32_t *bk = a.blk_keys;
                if (use_wide)
                    return launch(kKindScoreRefine, hisa_dgather_kernel<MT, KS, kDecodeRowsWide>, grid,
                                  dim3(kDecodeThreads), 0, st, a.q, bk, a.K, a.w, kss, bstride, Lk, pk, pk2, a);
                return launch(kKindScoreRefine, hisa_dgather_kernel<MT, KS, kDecodeRowsNarrow>, grid,
                              dim3(kDecodeThreads), 0, st, a.q, bk, a.K, a.w, kss, bstride, Lk, pk, pk2, a);
            }
            // one workgroup per compute unit or fewer: eight waves per
            // workgroup share its block stage and split its rows more finely
            const int tiles = use_wide ? wide : narrow;
            const bool eight = static_cast<int64_t>(tiles) * nq <= kDecodeEightWaveMaxGrid;
            const dim3 grid(static_cast<uint32_t>(decode_grid(nq, tiles)));
            const uint32_t pk2 = flags | static_cast<uint32_t>(tiles);
            auto go = [&](auto kernel, int threads) {
                return launch(kKindIndexDecode, kernel, grid, dim3(threads), 0, st, a.q, a.pool, a.K, a.w, kss, pss,
                              Lk, pk, pk2, a);
            };
            if (use_wide)
                return eight ? go(hisa_decode_kernel<MT, KS, kDecodeRowsWide, 512>, 512)
                             : go(hisa_decode_kernel<MT, KS, kDecodeRowsWide, 256>, 256);
            return eight ? go(hisa_decode_kernel<MT, KS, kDecodeRowsNarrow, 512>, 512)
                         : go(hisa_decode_kernel<MT, KS, kDecodeRowsNarrow, 256>, 256);
        }
    }
    const hipError_t e = (a.bucket_off && a.nblk <= kBMMaxBlocks)
        ? launch_block_major_blocks(a, st)
        : launch(kKindScoreBlocks, hisa_blocks_topm_kernel<MT, KS>, dim3(nq), dim3(kK1Threads), 0, st, a);
    if (e != hipSuccess) return e;
    if (a.bucket_off) return launch_block_major_refine(a, st);
    return launch(kKindScoreRefine, hisa_refine_kernel<MT, KS>, g2, dim3(kK2Threads), 0, st, a);
}

template <int MT>
hipError_t launch_fused_mt(const FusedArgs &a, bool decode, hipStream_t st) {
    return a.d == 64 ? launch_fused_ks<MT, 2>(a, decode, st) : launch_fused_ks<MT, 4>(a, decode, st);
}

}  // namespace

bool fused_supported(int d, int64_t L, int B, int m) {
    (void)m;
    return static_cast<int64_t>(B) * d <= kFusedOwnElems && (L + B - 1) / B <= kFusedMaxBlocks;
}

bool decode_mode(int S, int T, int64_t L, int B, int m) {
    return static_cast<int64_t>(S) * T <= kDecodeMaxQueries && (L + B - 1) / B <= kK1WaveMax &&
           m <= kDecodeMaxM;
}

bool pool_update_fusable(int S, int T, int d, int64_t L, int B, int m) {
    return fused_supported(d, L, B, m) && !block_major_mode(S, T, d, L, B, m);
}

hipError_t launch_fused_blocks_refine(const FusedArgs &a, hipStream_t st) {
    const bool decode = decode_mode(a.S, a.T, a.L, a.B, a.m);
    if (a.H <= 16) return launch_fused_mt<1>(a, decode, st);
    if (a.H <= 32) return launch_fused_mt<2>(a, decode, st);
    return launch_fused_mt<4>(a, decode, st);
}

}  // namespace hisa
