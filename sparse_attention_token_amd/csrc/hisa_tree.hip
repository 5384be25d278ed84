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
// tree_top_kernel does steps 1-4 for one query per 512-thread workgroup:
// q and w are staged in LDS and held as MFMA fragments (the shared scorer of
// scorer.h, so every score has the bits of the general path's kernels); the
// 8 waves score 16-row tiles, four tiles in flight per wave; each top-W / top-m
// is the one-wave ballot select over keys kept in LDS.  For the query at the
// cache's last row the pools already hold its own block and own super-block
// (the caller keeps them current through row L-1), so both are read like the
// other rows; any other query's own block is staged and pooled here (the pool's
// arithmetic), and its own super-block pooled from the pool entries and that.
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

// Scores n rows, row(p) giving row p's address (null: no candidate), into
// keys[top_slot(p, n)].  Waves take 16-row tiles round-robin, kTopTB at a time
// with their loads issued first.  Ends with a barrier.
template <int MT, int KS, typename RowOf>
__device__ __forceinline__ void score_into(const QFrag<MT, KS> &f, int n, uint32_t *keys, RowOf &&row_of) {
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
                if (g == 0 && p < n) keys[top_slot(p, n)] = valid[u] ? score_to_key(v) : kNoCandidate;
            }
        }
    }
    __syncthreads();
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

template <int MT, int KS, bool MAX>
__global__ __launch_bounds__(kTopThreads) void tree_top_kernel(TreeTopArgs a) {
    constexpr int D = 32 * KS;
    __shared__ __attribute__((aligned(16))) TreeTopLds<KS> L;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int qi = blockIdx.x;
    const int s = qi / a.T;
    const int64_t t = query_pos(a.qpos, qi, qi - s * a.T, a.L, a.T);
    int32_t *sel = a.sel_blk + static_cast<int64_t>(qi) * a.m;
    int32_t *ob = a.out_blk ? a.out_blk + static_cast<int64_t>(qi) * a.m : nullptr;
    int32_t *osb = a.out_sblk ? a.out_sblk + static_cast<int64_t>(qi) * a.W : nullptr;
    if (t < 0) {                                 // no candidate at all
        for (int j = tid; j < a.m; j += kTopThreads) {
            sel[j] = -1;
            if (ob) ob[j] = -1;
        }
        if (osb)
            for (int j = tid; j < a.W; j += kTopThreads) osb[j] = -1;
        return;
    }
    const int64_t bt = t / a.B;
    const int64_t st = bt / a.G;
    const int ns = static_cast<int>(st + 1);
    const bool own_from_pool = t == a.L - 1;
    const uint16_t *pool = a.pool + s * a.pool_seq_stride;
    const uint16_t *spool = a.spool + s * a.spool_seq_stride;

    // ---- stage q, w and (when the pools do not hold them) the own block's rows
    const int64_t r0 = bt * a.B;
    const int own_rows = static_cast<int>(t + 1 - r0);
    uint16_t *s_own = reinterpret_cast<uint16_t *>(L.own);
    QStager<MT, KS, kTopThreads> qst;           // q and w loads in flight with the rows'
    qst.load(a.q + static_cast<int64_t>(qi) * a.H * D, a.H, tid);
    const float wq = tid < a.H ? a.w[static_cast<int64_t>(qi) * a.H + tid] : 0.0f;
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
    qst.store(L.q, a.H, tid);
    if (tid < 64) L.w[tid] = wq;
    __syncthreads();
    if (!own_from_pool) {
        own_rows_rep<D, 64, MAX>(s_own, own_rows, L.rep, nullptr);     // ends with a barrier
        if (tid < D) L.srep[tid] = super_column<MAX>(pool + tid, D, st * a.G, bt, a.B, L.rep[tid], own_rows);
        __syncthreads();
    }
    const uint16_t *own_rep = own_from_pool ? pool + bt * D : L.rep;
    const uint16_t *own_srep = own_from_pool ? spool + st * D : L.srep;
    QFrag<MT, KS> f;
    load_qfrag_lds_w<MT, KS>(f, L.q, L.w, lane);

    // ---- levels 1-2: super-block scores, top W
    score_into<MT, KS>(f, ns, L.keys, [&](int u) -> const uint16_t * {
        return u < st ? spool + static_cast<int64_t>(u) * D : own_srep;
    });
    if (wave == 0) {
        const uint32_t ke = top_select(L.keys, ns, a.W, L.own, [&](uint32_t op, int u) {
            L.sb[op] = u;
            if (osb) osb[op] = u;
        });
        if (lane == 0) L.keff = ke;
    }
    __syncthreads();
    const int weff = static_cast<int>(L.keff);
    if (osb)
        for (int j = weff + tid; j < a.W; j += kTopThreads) osb[j] = -1;

    // ---- levels 2-3: the blocks of the kept super-blocks, top m
    const int nt = weff * a.G;
    score_into<MT, KS>(f, nt, L.keys, [&](int p) -> const uint16_t * {
        const int slot = p / a.G;
        const int64_t b = static_cast<int64_t>(L.sb[slot]) * a.G + (p - slot * a.G);
        return b < bt ? pool + b * D : (b == bt ? own_rep : nullptr);
    });
    if (wave == 0) {
        const uint32_t ke = top_select(L.keys, nt, a.m, L.own, [&](uint32_t op, int p) {
            const int slot = p / a.G;
            const int32_t b = L.sb[slot] * a.G + (p - slot * a.G);
            sel[op] = b;
            if (ob) ob[op] = b;
        });
        if (lane == 0) L.keff = ke;
    }
    __syncthreads();
    for (int j = static_cast<int>(L.keff) + tid; j < a.m; j += kTopThreads) {
        sel[j] = -1;
        if (ob) ob[j] = -1;
    }
}

template <int MT, int KS>
hipError_t launch_top_ks(const TreeTopArgs &a, hipStream_t st) {
    const dim3 grid(static_cast<uint32_t>(a.S * a.T)), block(kTopThreads);
    if (a.pool_max) return launch(kKindTreeTop, tree_top_kernel<MT, KS, true>, grid, block, 0, st, a);
    return launch(kKindTreeTop, tree_top_kernel<MT, KS, false>, grid, block, 0, st, a);
}

template <int MT>
hipError_t launch_top_mt(const TreeTopArgs &a, hipStream_t st) {
    return a.d == 64 ? launch_top_ks<MT, 2>(a, st) : launch_top_ks<MT, 4>(a, st);
}

}  // namespace

bool tree_top_supported(int d, int64_t L, int B, int G, int W) {
    const int64_t ns = ((L + B - 1) / B + G - 1) / G;
    return static_cast<int64_t>(B) * d <= kFusedOwnElems && ns <= kTopMaxRows &&
           static_cast<int64_t>(W) * G <= kTopMaxRows;
}

hipError_t launch_tree_top(const TreeTopArgs &a, hipStream_t st) {
    if (a.H <= 16) return launch_top_mt<1>(a, st);
    if (a.H <= 32) return launch_top_mt<2>(a, st);
    return launch_top_mt<4>(a, st);
}

}  // namespace hisa
