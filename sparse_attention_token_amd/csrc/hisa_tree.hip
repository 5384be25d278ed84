// The upper two levels of the three-level tree in one kernel.
//
// Page "Hierarchical Indexing Makes Sparse Attention Actually Fast", section
// "HISA's Approach: Hierarchical Summarization of the KV Cache", searches a
// tree of key-cache summaries from the top, keeping a beam of W nodes per level.
// With three levels -- super-blocks of G blocks, blocks of B keys, keys -- a
// query at t (b_t = t / B, u_t = b_t / G) does:
//   1. score every super-block u <= u_t with the indexer score: the super pool
//      entry for u < u_t, and for u_t the pooling of the pool entries
//      u_t*G .. b_t-1 followed by the own-block representative (rows b_t*B..t),
//      each weighted by its key count (the mean over the super-block's tokens);
//   2. keep the top W super-blocks;
//   3. score the blocks b <= b_t inside them (pool entries, own block for b_t);
//   4. keep the top m blocks.
// The token level (gather, score, top k) then runs as in the two-level path.
//
// tree_top_kernel does steps 1-3 with several 512-thread workgroups per
// query: each stages q and w in LDS and holds them as MFMA fragments (the
// shared scorer of scorer.h, so every score has the bits of the general
// path's kernels), scores the super-blocks with its 8 waves (16-row tiles,
// four in flight per wave) and keeps the top W with the one-wave ballot select
// over keys kept in LDS -- the same in every workgroup of the query -- and then
// scores its own slice of 128 of the kept super-blocks' blocks (one tile per
// wave) into the workspace.  tree_topm_kernel then keeps the top m of those
// keys for each query in one wave (step 4).  Done by one workgroup per query,
// the block level's 1024 rows took four rounds of one workgroup, and a decode
// batch of a few sequences kept a few compute units busy.  For the query at
// the cache's last row the pools already hold its own block and own
// super-block (the caller keeps them current through row L-1), so both are
// read like the other rows; any other query's own block is staged and pooled
// here (the pool's arithmetic), and its own super-block pooled from the pool
// entries and that.
// Limits (checked by the host, tree_top_supported): at most 2048 super-blocks
// visible, W*G <= 2048, B*d <= 16384.

#include <type_traits>

#include "block_rep.h"
#include "hisa_internal.h"
#include "scorer.h"
#include "select_core.h"

namespace hisa {
namespace {

constexpr int kTopThreads = 512;
constexpr int kTopWaves = kTopThreads / 64;
constexpr int kTopMaxRows = 2048;      // rows one ballot select takes (64 lanes x 32)
constexpr int kTopTB = 4;              // tiles in flight per wave
constexpr int kSliceRows = 16 * kTopWaves;   // fewest blocks per workgroup at the block level: a tile per wave
constexpr int kTopGroups = 512;        // workgroups sought per launch: slices repeat the super-block stage
constexpr int kTopmWaves = 4;          // queries per tree_topm_kernel workgroup, one wave each

template <int KS>
struct TreeTopLds {
    uint16_t q[64 * QStage<KS>::kStride];
    float w[64];
    uint32_t own[kFusedOwnElems / 2];  // own-block rows
    uint16_t rep[128];                 // own-block representative
    uint16_t srep[128];                // own super-block representative
    uint32_t keys[kTopMaxRows];        // keys by select slot
    int32_t sb[kTopMaxRows];           // kept super-blocks, ascending
    uint32_t keff;
};

// Select slot of position p among n <= 2048: lane p / rd holds it in register
// p % rd, and the layout makes a register's 64 reads one conflict-free row.
__device__ __forceinline__ int top_slot(int p, int n) {
    const int rd = (n + 63) / 64;
    return (p % rd) * 64 + p / rd;
}

// One wave: top kout of the n keys in s_keys; emit(op, position) for each kept
// one in increasing position order.  Returns the number kept.  win: 2112 words
// of LDS for the select's histogram.
template <typename Emit>
__device__ __forceinline__ uint32_t top_select(const uint32_t *s_keys, int n, int kout, uint32_t *win, Emit &&emit) {
    const int lane = threadIdx.x & 63;
    const int rd = (n + 63) / 64;
    auto run = [&](auto tag) -> uint32_t {
        constexpr int R = decltype(tag)::value;
        uint32_t kv[R];
#pragma unroll
        for (int r = 0; r < R; ++r) kv[r] = (r < rd && lane * rd + r < n) ? s_keys[r * 64 + lane] : kNoCandidate;
        const SelectResult res = R <= 4 ? wave_ballot_select<R>(kv, static_cast<uint32_t>(kout))
                                        : wave_window_select<R>(kv, static_cast<uint32_t>(kout), win);
        if (res.keff > 0) wave_compact<R>(kv, res, [&](uint32_t op, int r, uint32_t) { emit(op, lane * rd + r); });
        return res.keff;
    };
    if (rd <= 4) return run(std::integral_constant<int, 4>{});
    if (rd <= 8) return run(std::integral_constant<int, 8>{});
    if (rd <= 16) return run(std::integral_constant<int, 16>{});
    return run(std::integral_constant<int, 32>{});
}

// Scores n rows, row(p) giving row p's address (null: no candidate), and
// hands each key to store(p, key).  Waves take 16-row tiles round-robin,
// kTopTB at a time with their loads issued first.
template <int MT, int KS, typename RowOf, typename Store>
__device__ __forceinline__ void score_into(const QFrag<MT, KS> &f, int n, RowOf &&row_of, Store &&store) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int r = lane & 15, g = lane >> 4;
    const int ntiles = (n + 15) / 16;
    for (int base = wave; base < ntiles; base += kTopTB * kTopWaves) {
        bf16x8 kb[kTopTB][KS];
        bool valid[kTopTB];
#pragma unroll
        for (int u = 0; u < kTopTB; ++u) {
            const int p = (base + u * kTopWaves) * 16 + r;
            const uint16_t *row = p < n ? row_of(p) : nullptr;
            valid[u] = row != nullptr;
            load_row_frag<KS>(kb[u], row, lane);
        }
#pragma unroll
        for (int u = 0; u < kTopTB; ++u) {
            const int tile = base + u * kTopWaves;
            if (tile < ntiles) {
                const int p = tile * 16 + r;
                const float v = score_rows<MT, KS>(f, kb[u]);
                if (g == 0 && p < n) store(p, valid[u] ? score_to_key(v) : kNoCandidate);
            }
        }
    }
}

// Own super-block representative: per column, the pool entries b0 .. bt-1 in
// order (B keys each) and then the own-block representative (own_cnt keys):
// the count-weighted mean over the super-block's tokens, bf16(fp32(fp64
// sum_b cnt_b * r_b in block order / sum_b cnt_b)), or the first largest value.
template <bool MAX>
__device__ __forceinline__ uint16_t super_column(const uint16_t *pool_col, int d, int64_t b0, int64_t bt, int B,
                                                 uint16_t own, int own_cnt) {
    double sum = 0.0;
    float bestf = -__builtin_huge_valf();
    uint16_t best = 0;
    auto take = [&](uint16_t h, int cnt) {
        const float v = bf16_to_f32(h);
        if (MAX) {
            if (v > bestf) {
                bestf = v;
                best = h;
            }
        } else {
            sum += static_cast<double>(v) * static_cast<double>(cnt);   // exact product
        }
    };
    int64_t b = b0;
    for (; b + 8 <= bt; b += 8) {               // 8 loads in flight, added in block order
        uint16_t x[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) x[j] = pool_col[(b + j) * d];
#pragma unroll
        for (int j = 0; j < 8; ++j) take(x[j], B);
    }
    for (; b < bt; ++b) take(pool_col[b * d], B);
    take(own, own_cnt);
    return MAX ? best
               : f32_to_bf16_rne(static_cast<float>(sum / static_cast<double>((bt - b0) * B + own_cnt)));
}

// Grid S*T*nslice: workgroup (query qi, slice) scores blocks
// slice*rows .. slice*rows+rows-1 of the kept super-blocks' blocks (in kept
// order) into tblk_keys[qi]; slice 0 also publishes the kept super-blocks.
//
// The leading arguments are what a workgroup needs before its first loads (q,
// w and the own block's rows); this file is built with kernarg preloading,
// so they arrive in scalar registers at dispatch instead of after a memory
// round trip for the argument block.  pk = H | log2(B) << 8 | log2(G) << 12 |
// (qpos null) << 16.  EARLY = false (a key stride past 2^31 elements): they
// are ignored and everything comes from a_in.
template <int MT, int KS, bool MAX, bool EARLY>
__global__ __launch_bounds__(kTopThreads) void tree_top_kernel(const uint16_t *q, const float *w, const uint16_t *K,
                                                               int32_t k_seq_stride, int32_t Lk, int32_t T,
                                                               uint32_t pk, int nslice, int rows, TreeTopArgs a_in) {
    constexpr int D = 32 * KS;
    __shared__ __attribute__((aligned(16))) TreeTopLds<KS> L;
    TreeTopArgs a = a_in;
    bool qpos_null = a.qpos == nullptr;
    if constexpr (EARLY) {
        a.q = q; a.w = w; a.K = K; a.k_seq_stride = k_seq_stride; a.L = Lk; a.T = T;
        a.H = static_cast<int>(pk & 0xffu);
        a.B = 1 << ((pk >> 8) & 0xfu);
        a.G = 1 << ((pk >> 12) & 0xfu);
        qpos_null = ((pk >> 16) & 1u) != 0;
    }
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int qi = blockIdx.x / nslice;
    const int slice = blockIdx.x - qi * nslice;
    const bool lead = slice == 0;
    const int s = qi / a.T;
    int64_t t;
    if (qpos_null) {
        t = a.L - a.T + (qi - s * a.T);
        t = t >= 0 && t < a.L ? t : -1;
    } else {
        t = query_pos(a.qpos, qi, qi - s * a.T, a.L, a.T);
    }
    if (t < 0) {                                 // no candidate at all (tree_topm_kernel pads the blocks)
        if (lead)
            for (int j = tid; j < a.W; j += kTopThreads) {
                a.sel_sb[static_cast<int64_t>(qi) * a.W + j] = -1;
                if (a.out_sblk) a.out_sblk[static_cast<int64_t>(qi) * a.W + j] = -1;
            }
        return;
    }
    const int64_t bt = t / a.B;
    const int64_t st = bt / a.G;
    const int ns = static_cast<int>(st + 1);
    const bool own_from_pool = t == a.L - 1;

    // ---- stage q, w and (when the pools do not hold them) the own block's rows
    const int64_t r0 = bt * a.B;
    const int own_rows = static_cast<int>(t + 1 - r0);
    uint16_t *s_own = reinterpret_cast<uint16_t *>(L.own);
    QStager<MT, KS, kTopThreads> qst;           // q and w loads in flight with the rows'
    qst.load(a.q + static_cast<int64_t>(qi) * a.H * D, a.H, tid);
    const float wq0 = a.w[static_cast<int64_t>(qi) * a.H + (tid < a.H ? tid : a.H - 1)];   // unconditional load
    const float wq = tid < a.H ? wq0 : 0.0f;
    if (!own_from_pool) {
        constexpr int kPer = (kFusedOwnElems / 8 + kTopThreads - 1) / kTopThreads;
        const int chunks = own_rows * D / 8;
        const u32x4 *src = reinterpret_cast<const u32x4 *>(a.K + s * a.k_seq_stride + r0 * D);
        u32x4 *dst = reinterpret_cast<u32x4 *>(s_own);
        u32x4 v[kPer];
#pragma unroll
        for (int i = 0; i < kPer; ++i)
            if (tid + i * kTopThreads < chunks) v[i] = src[tid + i * kTopThreads];
#pragma unroll
        for (int i = 0; i < kPer; ++i)
            if (tid + i * kTopThreads < chunks) dst[tid + i * kTopThreads] = v[i];
    }
    pin_loaded(wq0);
    qst.store(L.q, a.H, tid);
    if (tid < 64) L.w[tid] = wq;
    __syncthreads();
    // the pools and output rows from the argument block, formed after the
    // first loads so that no wait for it comes before them
    const uint16_t *pool = a.pool + s * a.pool_seq_stride;
    const uint16_t *spool = a.spool + s * a.spool_seq_stride;
    int32_t *ssb = a.sel_sb + static_cast<int64_t>(qi) * a.W;
    int32_t *osb = a.out_sblk ? a.out_sblk + static_cast<int64_t>(qi) * a.W : nullptr;
    if (!own_from_pool) {
        own_rows_rep<D, 64, MAX>(s_own, own_rows, L.rep, nullptr);     // ends with a barrier
        if (tid < D) L.srep[tid] = super_column<MAX>(pool + tid, D, st * a.G, bt, a.B, L.rep[tid], own_rows);
        __syncthreads();
    }
    const uint16_t *own_rep = own_from_pool ? pool + bt * D : L.rep;
    const uint16_t *own_srep = own_from_pool ? spool + st * D : L.srep;
    QFrag<MT, KS> f;
    load_qfrag_lds_w<MT, KS>(f, L.q, L.w, lane);

    // ---- levels 1-2: super-block scores, top W (the same in every slice)
    score_into<MT, KS>(
        f, ns,
        [&](int u) -> const uint16_t * { return u < st ? spool + static_cast<int64_t>(u) * D : own_srep; },
        [&](int u, uint32_t key) { L.keys[top_slot(u, ns)] = key; });
    __syncthreads();
    if (wave == 0) {
        const uint32_t ke = top_select(L.keys, ns, a.W, L.own, [&](uint32_t op, int u) {
            L.sb[op] = u;
            if (lead) {
                ssb[op] = u;
                if (osb) osb[op] = u;
            }
        });
        if (lane == 0) L.keff = ke;
    }
    __syncthreads();
    const int weff = static_cast<int>(L.keff);
    if (lead)
        for (int j = weff + tid; j < a.W; j += kTopThreads) {
            ssb[j] = -1;
            if (osb) osb[j] = -1;
        }

    // ---- level 2: this workgroup's slice of the kept super-blocks' blocks
    const int nt = weff * a.G;
    const int p0 = slice * rows;
    if (p0 >= nt) return;
    uint32_t *keys = a.tblk_keys + static_cast<int64_t>(qi) * a.tblk_stride + p0;
    score_into<MT, KS>(
        f, nt - p0 < rows ? nt - p0 : rows,
        [&](int i) -> const uint16_t * {
            const int p = p0 + i;
            const int slot = p / a.G;
            const int64_t b = static_cast<int64_t>(L.sb[slot]) * a.G + (p - slot * a.G);
            return b < bt ? pool + b * D : (b == bt ? own_rep : nullptr);
        },
        [&](int i, uint32_t key) { keys[i] = key; });
}

// Level 3 of the search for query qi (t >= 0), by one wave: the top m of the
// W*G block keys tree_top_kernel wrote (kept super-block order); emit(op, b)
// gets the kept block ids in ascending order.  Returns the number kept.
// Lane l holds positions l*rd .. l*rd + rd - 1 with rd = ceil(ntb / 64) for
// the launch's bound ntb on weff*G, so the keys are loaded together with the
// kept super-blocks rather than after them; positions past the query's
// weff*G are dropped once weff is known.  R >= rd.  s_sb: W ints of LDS,
// win: kWindowWords words, both this wave's alone.
template <int R, typename Emit>
__device__ __forceinline__ uint32_t tree_topm_wave(const TreeTopArgs &a, int qi, int ntb, int32_t *s_sb,
                                                   uint32_t *win, Emit &&emit) {
    const int lane = threadIdx.x & 63;
    const int rd = (ntb + 63) / 64;
    const uint32_t *keys = a.tblk_keys + static_cast<int64_t>(qi) * a.tblk_stride;
    uint32_t kv[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {                      // every load issued before any is used
        const int p = lane * rd + r;
        kv[r] = keys[(r < rd && p < ntb) ? p : 0];
    }
    // the kept super-blocks (ascending, then -1) into LDS for the block ids
    const int32_t *ssb = a.sel_sb + static_cast<int64_t>(qi) * a.W;
    int weff = 0;
    for (int j0 = 0; j0 < a.W; j0 += 64) {
        const int j = j0 + lane;
        const int32_t u = ssb[j < a.W ? j : a.W - 1];
        if (j < a.W) s_sb[j] = u;
        weff += static_cast<int>(__popcll(__ballot(j < a.W && u >= 0)));
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    const int nt = weff * a.G;                         // <= ntb
#pragma unroll
    for (int r = 0; r < R; ++r)
        if (!(r < rd && lane * rd + r < nt)) kv[r] = kNoCandidate;
    const SelectResult res = R <= 4 ? wave_ballot_select<R>(kv, static_cast<uint32_t>(a.m))
                                    : wave_window_select<R>(kv, static_cast<uint32_t>(a.m), win);
    if (res.keff > 0)
        wave_compact<R>(kv, res, [&](uint32_t op, int r, uint32_t) {
            const int p = lane * rd + r;
            const int slot = p / a.G;
            emit(op, s_sb[slot] * a.G + (p - slot * a.G));
        });
    return res.keff;
}

// Level 3 alone, one wave per query (many queries: the refinement then runs
// as score_kernel).
template <int R>
__global__ __launch_bounds__(64 * kTopmWaves) void tree_topm_kernel(TreeTopArgs a, int ntb) {
    __shared__ int32_t s_sb[kTopmWaves][kTopMaxRows];
    __shared__ __attribute__((aligned(16))) uint32_t s_win[kTopmWaves][kWindowWords];
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int qi = blockIdx.x * kTopmWaves + wv;
    if (qi >= a.S * a.T) return;                       // whole wave
    const int s = qi / a.T;
    const int64_t t = query_pos(a.qpos, qi, qi - s * a.T, a.L, a.T);
    int32_t *sel = a.sel_blk + static_cast<int64_t>(qi) * a.m;
    int32_t *ob = a.out_blk ? a.out_blk + static_cast<int64_t>(qi) * a.m : nullptr;
    uint32_t keff = 0;
    if (t >= 0)
        keff = tree_topm_wave<R>(a, qi, ntb, s_sb[wv], s_win[wv], [&](uint32_t op, int32_t b) {
            sel[op] = b;
            if (ob) ob[op] = b;
        });
    for (int j = static_cast<int>(keff) + lane; j < a.m; j += 64) {
        sel[j] = -1;
        if (ob) ob[j] = -1;
    }
}

// Level 3 and the token level's scores for few queries, grid S*T*tiles: every
// workgroup of a query repeats its top m in wave 0 while the others stage q
// and w (a launch of its own cost more than the repeated select), then scores
// its kTreeGatherRows candidate rows (tile) into cand_keys, as score_kernel's
// refine mode does: row p is token p % B of kept slot p / B; slots past the
// kept count, and tokens past t, give no candidate.
constexpr int kTreeGatherThreads = 256;
constexpr int kTreeGatherRows = 128;          // 2 tiles of 16 rows per wave
constexpr int kTreeGatherMaxQueries = 16;
constexpr int kTreeGatherMaxM = 1024;

// Leading arguments preloaded at dispatch (as tree_top_kernel's): q, w, the
// block keys and kept super-blocks with the keys' row stride, L, pk = T | H
// << 8 | log2(B) << 16 | (qpos null) << 24 and pk2 = m | W << 16 (the launch
// holds at most 16 queries and m <= 1024, W <= 2048).
template <int MT, int KS, int R>
__global__ __launch_bounds__(kTreeGatherThreads) void tree_gather_kernel(const uint16_t *q, const float *w,
                                                                         const uint32_t *tblk_keys,
                                                                         const int32_t *sel_sb, int32_t tblk_stride,
                                                                         int32_t Lk, uint32_t pk, uint32_t pk2,
                                                                         int ntb, int tiles, TreeTopArgs a_in) {
    constexpr int D = 32 * KS;
    constexpr int NTW = kTreeGatherRows / (16 * kTreeGatherThreads / 64);
    __shared__ __attribute__((aligned(16))) uint16_t s_q[64 * QStage<KS>::kStride];
    __shared__ float s_w[64];
    __shared__ int32_t s_sb[kTopMaxRows];
    __shared__ int32_t s_sel[kTreeGatherMaxM];
    __shared__ __attribute__((aligned(16))) uint32_t s_win[kWindowWords];
    __shared__ uint32_t s_keff;

    TreeTopArgs a = a_in;
    a.q = q; a.w = w; a.tblk_keys = const_cast<uint32_t *>(tblk_keys); a.sel_sb = const_cast<int32_t *>(sel_sb);
    a.tblk_stride = tblk_stride; a.L = Lk;
    a.T = static_cast<int>(pk & 0xffu);
    a.H = static_cast<int>((pk >> 8) & 0xffu);
    a.B = 1 << ((pk >> 16) & 0xfu);
    const bool qpos_null = ((pk >> 24) & 1u) != 0;
    a.m = static_cast<int>(pk2 & 0xffffu);
    a.W = static_cast<int>(pk2 >> 16);
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int n = lane & 15, g = lane >> 4;
    const int qi = blockIdx.x / tiles;
    const int tile = blockIdx.x - qi * tiles;
    const bool lead = tile == 0;                       // also publishes the kept blocks
    const int s = qi / a.T;
    int64_t t;
    if (qpos_null) {
        t = a.L - a.T + (qi - s * a.T);
        t = t >= 0 && t < a.L ? t : -1;
    } else {
        t = query_pos(a.qpos, qi, qi - s * a.T, a.L, a.T);
    }
    if (t < 0) {                                       // the select reads no candidate row
        if (lead)
            for (int j = tid; j < a.m; j += kTreeGatherThreads) {
                a.sel_blk[static_cast<int64_t>(qi) * a.m + j] = -1;
                if (a.out_blk) a.out_blk[static_cast<int64_t>(qi) * a.m + j] = -1;
            }
        return;
    }
    const int64_t bt = t / a.B;
    // the refine-mode row length the select reads: min(m, b_t + 1) slots of B
    const int npos = static_cast<int>((a.m < bt + 1 ? a.m : bt + 1) * a.B);
    const int tile0 = tile * kTreeGatherRows;
    if (tile0 >= npos) return;

    QStager<MT, KS, kTreeGatherThreads> qst;
    qst.load(a.q + static_cast<int64_t>(qi) * a.H * D, a.H, tid);
    const float wq0 = a.w[static_cast<int64_t>(qi) * a.H + (tid < a.H ? tid : a.H - 1)];   // unconditional load
    const float wq = tid < a.H ? wq0 : 0.0f;
    if (wave == 0) {
        const uint32_t ke = tree_topm_wave<R>(a, qi, ntb, s_sb, s_win, [&](uint32_t op, int32_t b) {
            s_sel[op] = b;
            if (lead) {
                // output rows from the argument block, formed here, after the
                // first loads
                a.sel_blk[static_cast<int64_t>(qi) * a.m + op] = b;
                if (a.out_blk) a.out_blk[static_cast<int64_t>(qi) * a.m + op] = b;
            }
        });
        if (lane == 0) s_keff = ke;
    }
    pin_loaded(wq0);
    qst.store(s_q, a.H, tid);
    if (tid < 64) s_w[tid] = wq;
    __syncthreads();
    const int keff = static_cast<int>(s_keff);
    if (lead)
        for (int j = keff + tid; j < a.m; j += kTreeGatherThreads) {
            a.sel_blk[static_cast<int64_t>(qi) * a.m + j] = -1;
            if (a.out_blk) a.out_blk[static_cast<int64_t>(qi) * a.m + j] = -1;
        }

    // rows past the kept slots, or past t, load row t (a valid row) and are
    // stored as no candidate
    bf16x8 kb[NTW][KS];
    bool valid[NTW];
#pragma unroll
    for (int nt = 0; nt < NTW; ++nt) {
        const int p = tile0 + (wave * NTW + nt) * 16 + n;
        const int slot = p / a.B;
        const int64_t tok = slot < keff ? static_cast<int64_t>(s_sel[slot]) * a.B + (p - slot * a.B) : t;
        valid[nt] = p < npos && slot < keff && tok <= t;
        load_row_frag_any<KS>(kb[nt], a.K + s * a.k_seq_stride + (tok <= t ? tok : t) * D, lane);
    }
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
hipError_t launch_top_ks(const TreeTopArgs &a, hipStream_t st, bool *scored) {
    const int nq = a.S * a.T;
    const int64_t ns = ((a.L + a.B - 1) / a.B + a.G - 1) / a.G;
    const int64_t ntb = (a.W < ns ? a.W : ns) * a.G;   // at most 2048 (tree_top_supported)
    // slices of at least 128 blocks, as many as keep about kTopGroups
    // workgroups busy (one for large batches: no repeated super-block stage)
    const int most = static_cast<int>((ntb + kSliceRows - 1) / kSliceRows);
    const int want = (kTopGroups + nq - 1) / nq;
    const int nslice = want < most ? want : most;
    const int rows = static_cast<int>((ntb + nslice - 1) / nslice + 15) / 16 * 16;
    const dim3 grid(static_cast<uint32_t>(nq * nslice)), block(kTopThreads);
    // preloaded words (tree_top_kernel); a key stride past 2^31 elements takes
    // the variant reading the struct
    const bool early = a.k_seq_stride < (int64_t{1} << 31);
    const uint32_t pk = static_cast<uint32_t>(a.H) | static_cast<uint32_t>(__builtin_ctz(static_cast<unsigned>(a.B))) << 8 |
                        static_cast<uint32_t>(__builtin_ctz(static_cast<unsigned>(a.G))) << 12 |
                        (a.qpos == nullptr ? 1u : 0u) << 16;
    const int32_t kss = early ? static_cast<int32_t>(a.k_seq_stride) : 0, Lk = static_cast<int32_t>(a.L);
    auto top = [&](auto kernel) {
        return launch(kKindTreeTop, kernel, grid, block, 0, st, a.q, a.w, a.K, kss, Lk, a.T, pk, nslice, rows, a);
    };
    hipError_t e = a.pool_max ? (early ? top(tree_top_kernel<MT, KS, true, true>) : top(tree_top_kernel<MT, KS, true, false>))
                              : (early ? top(tree_top_kernel<MT, KS, false, true>) : top(tree_top_kernel<MT, KS, false, false>));
    if (e != hipSuccess) return e;
    const int nt = static_cast<int>(ntb);
    const int rd = (nt + 63) / 64;
    *scored = nq <= kTreeGatherMaxQueries && a.m <= kTreeGatherMaxM;
    if (*scored) {
        const int tiles = static_cast<int>((static_cast<int64_t>(a.m) * a.B + kTreeGatherRows - 1) / kTreeGatherRows);
        const dim3 g3(static_cast<uint32_t>(nq * tiles)), b3(kTreeGatherThreads);
        // nq <= 16 (so T <= 16), m <= 1024, W <= 2048 and the key rows' stride
        // below 2^31: every field fits its packed place
        const uint32_t gk = static_cast<uint32_t>(a.T) | static_cast<uint32_t>(a.H) << 8 |
                            static_cast<uint32_t>(__builtin_ctz(static_cast<unsigned>(a.B))) << 16 |
                            (a.qpos == nullptr ? 1u : 0u) << 24;
        const uint32_t gk2 = static_cast<uint32_t>(a.m) | static_cast<uint32_t>(a.W) << 16;
        const int32_t ts = static_cast<int32_t>(a.tblk_stride);
        auto gather = [&](auto kernel) {
            return launch(kKindScoreRefine, kernel, g3, b3, 0, st, a.q, a.w, static_cast<const uint32_t *>(a.tblk_keys),
                          static_cast<const int32_t *>(a.sel_sb), ts, Lk, gk, gk2, nt, tiles, a);
        };
        if (rd <= 4) return gather(tree_gather_kernel<MT, KS, 4>);
        if (rd <= 8) return gather(tree_gather_kernel<MT, KS, 8>);
        if (rd <= 16) return gather(tree_gather_kernel<MT, KS, 16>);
        return gather(tree_gather_kernel<MT, KS, 32>);
    }
    const dim3 g2(static_cast<uint32_t>((nq + kTopmWaves - 1) / kTopmWaves)), b2(64 * kTopmWaves);
    if (rd <= 4) return launch(kKindSelectTree, tree_topm_kernel<4>, g2, b2, 0, st, a, nt);
    if (rd <= 8) return launch(kKindSelectTree, tree_topm_kernel<8>, g2, b2, 0, st, a, nt);
    if (rd <= 16) return launch(kKindSelectTree, tree_topm_kernel<16>, g2, b2, 0, st, a, nt);
    return launch(kKindSelectTree, tree_topm_kernel<32>, g2, b2, 0, st, a, nt);
}

template <int MT>
hipError_t launch_top_mt(const TreeTopArgs &a, hipStream_t st, bool *scored) {
    return a.d == 64 ? launch_top_ks<MT, 2>(a, st, scored) : launch_top_ks<MT, 4>(a, st, scored);
}

}  // namespace

bool tree_top_supported(int d, int64_t L, int B, int G, int W) {
    const int64_t ns = ((L + B - 1) / B + G - 1) / G;
    return static_cast<int64_t>(B) * d <= kFusedOwnElems && ns <= kTopMaxRows &&
           static_cast<int64_t>(W) * G <= kTopMaxRows;
}

hipError_t launch_tree_top(const TreeTopArgs &a, hipStream_t st, bool *scored) {
    if (a.H <= 16) return launch_top_mt<1>(a, st, scored);
    if (a.H <= 32) return launch_top_mt<2>(a, st, scored);
    return launch_top_mt<4>(a, st, scored);
}

}  // namespace hisa
