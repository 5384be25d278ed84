// C-ABI entry points of libhisa: argument checks, workspace layout, launches.
// Every check runs on the host before anything is enqueued.

#include <algorithm>
#include <cstring>
#include <mutex>
#include <vector>

#include "../../include/hisa.h"
#include "hisa_internal.h"

namespace hisa {
namespace {

constexpr size_t kAlign = 256;

inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }
inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

inline bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

inline bool block_size_ok(int B) {
    return B == 16 || B == 32 || B == 64 || B == 128 || B == 256;
}

int check_query_shape(int S, int T, int H, int d, int64_t L, int k) {
    if (S < 1 || T < 1 || H < 1 || d < 1 || L < 1 || k < 1) return HISA_ERR_ARG;
    if (d != 64 && d != 128) return HISA_ERR_UNSUPPORTED;
    if (H > 64) return HISA_ERR_UNSUPPORTED;
    if (L >= (int64_t{1} << 31)) return HISA_ERR_UNSUPPORTED;
    if (k > 16384) return HISA_ERR_UNSUPPORTED;
    if (static_cast<int64_t>(S) * T > 65535) return HISA_ERR_UNSUPPORTED;
    return HISA_OK;
}

int check_hisa_params(int B, int m) {
    if (B < 1 || m < 1) return HISA_ERR_ARG;
    if (!block_size_ok(B)) return HISA_ERR_UNSUPPORTED;
    if (m > 4096 || static_cast<int64_t>(m) * B > (int64_t{1} << 20)) return HISA_ERR_UNSUPPORTED;
    return HISA_OK;
}

int check_cache(const uint16_t *K, int64_t k_seq_stride, int S, int d, int64_t L) {
    if (!K || !aligned16(K)) return HISA_ERR_ARG;
    if (k_seq_stride < 0 || (k_seq_stride & 7) != 0) return HISA_ERR_ARG;
    if (S > 1 && k_seq_stride < L * d) return HISA_ERR_ARG;
    return HISA_OK;
}

int check_pool(const uint16_t *pool, int64_t pool_seq_stride, int S, int d, int64_t L, int B) {
    if (!pool || !aligned16(pool)) return HISA_ERR_ARG;
    if (pool_seq_stride < 0 || (pool_seq_stride & 7) != 0) return HISA_ERR_ARG;
    if (S > 1 && pool_seq_stride < ceil_div(L, B) * d) return HISA_ERR_ARG;
    return HISA_OK;
}

int check_append(const uint16_t *K, int64_t k_seq_stride, int S, int d, int B, int64_t L_old, int64_t L_new,
                 const uint16_t *pool_mean, int64_t pool_seq_stride) {
    if (S < 1 || d < 1 || B < 1 || L_old < 0 || L_new < L_old) return HISA_ERR_ARG;
    if (d != 64 && d != 128) return HISA_ERR_UNSUPPORTED;
    if (!block_size_ok(B)) return HISA_ERR_UNSUPPORTED;
    if (L_new >= (int64_t{1} << 31) || S > 65535) return HISA_ERR_UNSUPPORTED;
    const int st = check_cache(K, k_seq_stride, S, d, L_new);
    if (st != HISA_OK) return st;
    return check_pool(pool_mean, pool_seq_stride, S, d, L_new, B);
}

// ---------------------------------------------------------------- workspace layouts
struct StageBufs {
    size_t keys[2], ids[2];
    int64_t stride;
};

// carve the two ping-pong (key, id) buffers of the chunked selection
size_t carve_stage(size_t off, int64_t nq, int64_t len, StageBufs &sb) {
    sb.stride = static_cast<int64_t>(align_up(static_cast<size_t>(len), 64));
    const size_t bytes = static_cast<size_t>(nq) * sb.stride * 4;
    for (int i = 0; i < 2; ++i) {
        sb.keys[i] = off; off = align_up(off + bytes, kAlign);
        sb.ids[i] = off;  off = align_up(off + bytes, kAlign);
    }
    return off;
}

struct HisaLayout {
    size_t own_rep, blk_keys, sel_blk, cand_keys, bucket_off, bucket_ent, total;
    int64_t blk_stride, cand_stride;
    StageBufs stage;
};

HisaLayout hisa_layout(int S, int T, int d, int64_t L, int B, int m, int k) {
    HisaLayout l{};
    const int64_t nq = static_cast<int64_t>(S) * T;
    const int64_t nblk = ceil_div(L, B);
    l.blk_stride = static_cast<int64_t>(align_up(static_cast<size_t>(nblk), 64));
    l.cand_stride = static_cast<int64_t>(align_up(static_cast<size_t>(m) * B, 64));
    size_t off = 0;
    l.own_rep = off;   off = align_up(off + static_cast<size_t>(nq) * d * sizeof(uint16_t), kAlign);
    l.blk_keys = off;  off = align_up(off + static_cast<size_t>(nq) * l.blk_stride * sizeof(uint32_t), kAlign);
    l.sel_blk = off;   off = align_up(off + static_cast<size_t>(nq) * m * sizeof(int32_t), kAlign);
    l.cand_keys = off; off = align_up(off + static_cast<size_t>(nq) * l.cand_stride * sizeof(uint32_t), kAlign);
    if (block_major_mode(S, T, d, L, B, m)) {
        const size_t nchunk = static_cast<size_t>(bucket_chunks(S, T));
        l.bucket_off = off; off = align_up(off + nchunk * (nblk + 1) * sizeof(int32_t), kAlign);
        l.bucket_ent = off; off = align_up(off + nchunk * kChunkQueries * m * sizeof(uint32_t), kAlign);
    }
    const int64_t len = std::max(select_stage_len(nblk, m, B, false),
                                 select_stage_len(static_cast<int64_t>(m) * B, k, B, true));
    off = carve_stage(off, nq, len, l.stage);
    l.total = off + kAlign;   // slack to align the caller's base pointer
    return l;
}

// three-level tree (hisa_tree_index)
struct TreeLayout {
    size_t own_rep, own_srep, sblk_keys, sel_sb, tblk_keys, sel_blk, cand_keys, total;
    int64_t sblk_stride, tblk_stride, cand_stride;
    StageBufs stage;
};

TreeLayout tree_layout(int S, int T, int d, int64_t L, int B, int G, int W, int m, int k) {
    TreeLayout l{};
    const int64_t nq = static_cast<int64_t>(S) * T;
    const int64_t ns = ceil_div(ceil_div(L, B), G);
    const int64_t ntb = std::min<int64_t>(W, ns) * G;          // blocks of the kept super-blocks
    l.sblk_stride = static_cast<int64_t>(align_up(static_cast<size_t>(ns), 64));
    l.tblk_stride = static_cast<int64_t>(align_up(static_cast<size_t>(ntb), 64));
    l.cand_stride = static_cast<int64_t>(align_up(static_cast<size_t>(m) * B, 64));
    const size_t rep = static_cast<size_t>(nq) * d * sizeof(uint16_t);
    size_t off = 0;
    l.own_rep = off;   off = align_up(off + rep, kAlign);
    l.own_srep = off;  off = align_up(off + rep, kAlign);
    l.sblk_keys = off; off = align_up(off + static_cast<size_t>(nq) * l.sblk_stride * sizeof(uint32_t), kAlign);
    l.sel_sb = off;    off = align_up(off + static_cast<size_t>(nq) * W * sizeof(int32_t), kAlign);
    l.tblk_keys = off; off = align_up(off + static_cast<size_t>(nq) * l.tblk_stride * sizeof(uint32_t), kAlign);
    l.sel_blk = off;   off = align_up(off + static_cast<size_t>(nq) * m * sizeof(int32_t), kAlign);
    l.cand_keys = off; off = align_up(off + static_cast<size_t>(nq) * l.cand_stride * sizeof(uint32_t), kAlign);
    const int64_t len = std::max({select_stage_len(ns, W, B * G, false),
                                  select_stage_len(ntb, m, G, true),
                                  select_stage_len(static_cast<int64_t>(m) * B, k, B, true)});
    off = carve_stage(off, nq, len, l.stage);
    l.total = off + kAlign;
    return l;
}

inline bool fanout_ok(int G) { return G >= 1 && G <= 256 && (G & (G - 1)) == 0; }

int check_tree_params(int B, int G, int W, int m) {
    const int st = check_hisa_params(B, m);
    if (st != HISA_OK) return st;
    if (G < 1 || W < 1) return HISA_ERR_ARG;
    if (!fanout_ok(G)) return HISA_ERR_UNSUPPORTED;
    if (W > kSelMaxM || static_cast<int64_t>(W) * G > (int64_t{1} << 20)) return HISA_ERR_UNSUPPORTED;
    return HISA_OK;
}

struct FlatLayout {
    size_t keys, bucket_off, bucket_ent, total;
    int64_t stride;
    bool block_major;         // prefill chunks: flat_block_major_mode
    StageBufs stage;
};

FlatLayout flat_layout(int S, int T, int d, int64_t L, int k) {
    FlatLayout l{};
    const int64_t nq = static_cast<int64_t>(S) * T;
    l.block_major = flat_block_major_mode(S, T, d, L);
    const int64_t nblk = ceil_div(L, kFlatBlock);
    // block by block, every block's rows are written whole (positions past t
    // as "no candidate"), so a row holds nblk * kFlatBlock keys
    const int64_t row = l.block_major ? nblk * kFlatBlock : L;
    l.stride = static_cast<int64_t>(align_up(static_cast<size_t>(row), 64));
    l.keys = 0;
    size_t off = align_up(static_cast<size_t>(nq) * l.stride * sizeof(uint32_t), kAlign);
    if (l.block_major) {
        const size_t nchunk = static_cast<size_t>(bucket_chunks(S, T));
        l.bucket_off = off; off = align_up(off + nchunk * (nblk + 1) * sizeof(int32_t), kAlign);
        l.bucket_ent = off; off = align_up(off + nchunk * kChunkQueries * nblk * sizeof(uint32_t), kAlign);
    }
    off = carve_stage(off, nq, select_stage_len(L, k, 1, false), l.stage);
    l.total = off + kAlign;
    return l;
}

void set_stage(SelectArgs &se, char *base, const StageBufs &sb) {
    for (int i = 0; i < 2; ++i) {
        se.stage_keys[i] = reinterpret_cast<uint32_t *>(base + sb.keys[i]);
        se.stage_ids[i] = reinterpret_cast<int32_t *>(base + sb.ids[i]);
    }
    se.stage_stride = sb.stride;
}

inline char *align_ptr(void *p) {
    return reinterpret_cast<char *>(align_up(reinterpret_cast<uintptr_t>(p), kAlign));
}

inline int hip_status(hipError_t e) { return e == hipSuccess ? HISA_OK : HISA_ERR_HIP; }

// ---------------------------------------------------------------- profiler state
struct Profiler {
    bool on = false;
    int cap = 0;
    int used = 0;
    std::vector<hipEvent_t> ev;
    std::vector<int> kind;
};
Profiler g_prof;

void prof_release() {
    for (hipEvent_t e : g_prof.ev) (void)hipEventDestroy(e);
    g_prof.ev.clear();
    g_prof.kind.clear();
    g_prof.on = false;
    g_prof.cap = g_prof.used = 0;
}

const char *const kKindNames[kKindCount] = {
    "pool_append", "own_mean", "score_blocks", "select_blocks",
    "score_refine", "select_refine", "score_flat", "select_flat",
    "index_decode", "bucket", "own_super", "score_tree", "select_tree", "tree_top",
    "sparse_attention", "attention_combine", "bucket_flat",
};

}  // namespace

bool prof_events(KernelKind kind, hipEvent_t *start, hipEvent_t *stop) {
    if (!g_prof.on || g_prof.used >= g_prof.cap) return false;
    *start = g_prof.ev[2 * g_prof.used];
    *stop = g_prof.ev[2 * g_prof.used + 1];
    g_prof.kind[g_prof.used] = kind;
    ++g_prof.used;
    return true;
}

}  // namespace hisa

using namespace hisa;

extern "C" {

int hisa_abi_version(void) { return HISA_ABI_VERSION; }

const char *hisa_status_string(int status) {
    switch (status) {
        case HISA_OK: return "ok";
        case HISA_ERR_ARG: return "invalid argument (null pointer, negative size, bad stride or length)";
        case HISA_ERR_UNSUPPORTED: return "unsupported shape";
        case HISA_ERR_WORKSPACE: return "workspace too small";
        case HISA_ERR_HIP: return "HIP runtime error while enqueuing";
        case HISA_ERR_SCRATCH: return "the call needs more workspace than the library's static scratch (16 MiB)";
        default: return "unknown status";
    }
}

int hisa_pool_append_mode(const uint16_t *K, int64_t k_seq_stride, int S, int d, int B,
                          int64_t L_old, int64_t L_new, uint16_t *pool_rep, int64_t pool_seq_stride,
                          int pool_kind, void *stream) {
    if (pool_kind != HISA_POOL_MEAN && pool_kind != HISA_POOL_MAX) return HISA_ERR_ARG;
    const int st = check_append(K, k_seq_stride, S, d, B, L_old, L_new, pool_rep, pool_seq_stride);
    if (st != HISA_OK) return st;
    if (L_old == L_new) return HISA_OK;
    const int64_t blk0 = L_old / B;
    const int64_t blk1 = (L_new - 1) / B;
    return hip_status(launch_pool_append(K, k_seq_stride, S, d, B, blk0, blk1 - blk0 + 1, L_new,
                                         pool_kind == HISA_POOL_MAX, pool_rep, pool_seq_stride,
                                         static_cast<hipStream_t>(stream)));
}

int hisa_pool_append(const uint16_t *K, int64_t k_seq_stride, int S, int d, int B,
                     int64_t L_old, int64_t L_new, uint16_t *pool_mean, int64_t pool_seq_stride,
                     void *stream) {
    return hisa_pool_append_mode(K, k_seq_stride, S, d, B, L_old, L_new, pool_mean, pool_seq_stride,
                                 HISA_POOL_MEAN, stream);
}

size_t hisa_index_workspace(int S, int T, int H, int d, int64_t L, int B, int m, int k) {
    if (check_query_shape(S, T, H, d, L, k) != HISA_OK) return 0;
    if (check_hisa_params(B, m) != HISA_OK) return 0;
    return hisa_layout(S, T, d, L, B, m, k).total;
}

}  // extern "C"

namespace {

int check_index(const uint16_t *q, const float *w, const int32_t *qpos, const uint16_t *K,
                int64_t k_seq_stride, int64_t L, const uint16_t *pool_mean, int64_t pool_seq_stride,
                int S, int T, int H, int d, int B, int m, int k, const int32_t *out_idx, const void *ws,
                size_t ws_bytes) {
    int st = check_query_shape(S, T, H, d, L, k);
    if (st != HISA_OK) return st;
    st = check_hisa_params(B, m);
    if (st != HISA_OK) return st;
    if (!q || !w || !out_idx || !aligned16(q)) return HISA_ERR_ARG;
    if (!qpos && T > L) return HISA_ERR_ARG;
    st = check_cache(K, k_seq_stride, S, d, L);
    if (st != HISA_OK) return st;
    st = check_pool(pool_mean, pool_seq_stride, S, d, L, B);
    if (st != HISA_OK) return st;
    if (!ws) return HISA_ERR_ARG;
    if (ws_bytes < hisa_layout(S, T, d, L, B, m, k).total) return HISA_ERR_WORKSPACE;
    return HISA_OK;
}

// hisa_index once its arguments are checked.  pool_out (the pool itself, or
// null): the fused block stage also stores the own-block mean of the query at
// t = L-1 (only on paths where pool_update_fusable() holds).
int run_index(const uint16_t *q, const float *w, const int32_t *qpos, const uint16_t *K,
              int64_t k_seq_stride, int64_t L, const uint16_t *pool_mean, uint16_t *pool_out,
              int64_t pool_seq_stride, int S, int T, int H, int d, int B, int m, int k,
              int32_t *out_idx, float *out_score, int32_t *out_blk, void *ws, bool pool_max, hipStream_t hs) {
    int st = HISA_OK;
    const HisaLayout lay = hisa_layout(S, T, d, L, B, m, k);

    char *base = align_ptr(ws);
    uint16_t *own_rep = reinterpret_cast<uint16_t *>(base + lay.own_rep);
    uint32_t *blk_keys = reinterpret_cast<uint32_t *>(base + lay.blk_keys);
    int32_t *sel_blk = reinterpret_cast<int32_t *>(base + lay.sel_blk);
    uint32_t *cand_keys = reinterpret_cast<uint32_t *>(base + lay.cand_keys);
    const int nq = S * T;

    SelectArgs se{};
    se.qpos = qpos; se.L = L; se.T = T; se.B = B; se.m = m;
    set_stage(se, base, lay.stage);

    if (fused_supported(d, L, B, m)) {
        FusedArgs fa{};
        fa.q = q; fa.w = w; fa.qpos = qpos;
        fa.K = K; fa.k_seq_stride = k_seq_stride; fa.L = L;
        fa.pool = pool_mean; fa.pool_seq_stride = pool_seq_stride;
        fa.S = S; fa.T = T; fa.H = H; fa.d = d; fa.B = B; fa.m = m; fa.k = k;
        fa.sel_blk = sel_blk; fa.out_blk = out_blk;
        fa.cand_keys = cand_keys; fa.cand_stride = lay.cand_stride;
        fa.out_idx = out_idx; fa.out_score = out_score;
        fa.nblk = static_cast<int>(ceil_div(L, B));
        fa.blk_keys = blk_keys;
        fa.blk_stride = lay.blk_stride;
        fa.pool_out = pool_out;
        fa.pool_max = pool_max ? 1 : 0;
        if (block_major_mode(S, T, d, L, B, m)) {
            fa.bucket_off = reinterpret_cast<int32_t *>(base + lay.bucket_off);
            fa.bucket_ent = reinterpret_cast<uint32_t *>(base + lay.bucket_ent);
            fa.own_rep = own_rep;
            fa.blk_keys = blk_keys;
            fa.blk_stride = lay.blk_stride;
        }
        st = hip_status(launch_fused_blocks_refine(fa, hs));
        if (st != HISA_OK) return st;
        se.keys = cand_keys; se.keys_stride = lay.cand_stride;
        se.kout = k; se.sel_blk = sel_blk;
        se.out_id = out_idx; se.out_score = out_score; se.out_id_copy = nullptr;
        return hip_status(launch_select(kScoreRefine, se, nq, static_cast<int64_t>(m) * B, hs));
    }

    // general path (any supported shape): own-block means, then score and
    // select twice
    st = hip_status(launch_own_mean(K, k_seq_stride, qpos, L, S, T, d, B, pool_max, own_rep, hs));
    if (st != HISA_OK) return st;

    ScoreArgs sa{};
    sa.q = q; sa.w = w; sa.qpos = qpos;
    sa.K = K; sa.k_seq_stride = k_seq_stride; sa.L = L;
    sa.pool = pool_mean; sa.pool_seq_stride = pool_seq_stride;
    sa.own_rep = own_rep; sa.sel_blk = sel_blk;
    sa.S = S; sa.T = T; sa.H = H; sa.d = d; sa.B = B; sa.m = m;

    // stage 1: block scores and the top-m blocks
    sa.keys = blk_keys; sa.keys_stride = lay.blk_stride;
    st = hip_status(launch_score(kScoreBlocks, sa, ceil_div(L, B), hs));
    if (st != HISA_OK) return st;
    se.keys = blk_keys; se.keys_stride = lay.blk_stride;
    se.kout = m; se.sel_blk = nullptr;
    se.out_id = sel_blk; se.out_score = nullptr; se.out_id_copy = out_blk;
    st = hip_status(launch_select(kScoreBlocks, se, nq, ceil_div(L, B), hs));
    if (st != HISA_OK) return st;

    // stage 2: token refinement inside the kept blocks and the final top-k
    sa.keys = cand_keys; sa.keys_stride = lay.cand_stride;
    st = hip_status(launch_score(kScoreRefine, sa, static_cast<int64_t>(m) * B, hs));
    if (st != HISA_OK) return st;
    se.keys = cand_keys; se.keys_stride = lay.cand_stride;
    se.kout = k; se.sel_blk = sel_blk;
    se.out_id = out_idx; se.out_score = out_score; se.out_id_copy = nullptr;
    return hip_status(launch_select(kScoreRefine, se, nq, static_cast<int64_t>(m) * B, hs));
}
}  // namespace

extern "C" {

int hisa_index_mode(const uint16_t *q, const float *w, const int32_t *qpos, const uint16_t *K,
                    int64_t k_seq_stride, int64_t L, const uint16_t *pool_rep,
                    int64_t pool_seq_stride, int S, int T, int H, int d, int B, int m, int k,
                    int32_t *out_idx, float *out_score, int32_t *out_blk, void *ws, size_t ws_bytes,
                    int pool_kind, void *stream) {
    if (pool_kind != HISA_POOL_MEAN && pool_kind != HISA_POOL_MAX) return HISA_ERR_ARG;
    const int st = check_index(q, w, qpos, K, k_seq_stride, L, pool_rep, pool_seq_stride, S, T, H, d, B, m, k,
                               out_idx, ws, ws_bytes);
    if (st != HISA_OK) return st;
    return run_index(q, w, qpos, K, k_seq_stride, L, pool_rep, nullptr, pool_seq_stride, S, T, H, d, B, m, k,
                     out_idx, out_score, out_blk, ws, pool_kind == HISA_POOL_MAX, static_cast<hipStream_t>(stream));
}

int hisa_index(const uint16_t *q, const float *w, const int32_t *qpos, const uint16_t *K,
               int64_t k_seq_stride, int64_t L, const uint16_t *pool_mean,
               int64_t pool_seq_stride, int S, int T, int H, int d, int B, int m, int k,
               int32_t *out_idx, float *out_score, int32_t *out_blk, void *ws, size_t ws_bytes,
               void *stream) {
    return hisa_index_mode(q, w, qpos, K, k_seq_stride, L, pool_mean, pool_seq_stride, S, T, H, d, B, m, k,
                           out_idx, out_score, out_blk, ws, ws_bytes, HISA_POOL_MEAN, stream);
}

int hisa_append_index_mode(const uint16_t *K, int64_t k_seq_stride, int64_t L_old, int64_t L_new,
                           uint16_t *pool_rep, int64_t pool_seq_stride, const uint16_t *q, const float *w,
                           const int32_t *qpos, int S, int T, int H, int d, int B, int m, int k, int32_t *out_idx,
                           float *out_score, int32_t *out_blk, void *ws, size_t ws_bytes, int pool_kind,
                           void *stream) {
    if (pool_kind != HISA_POOL_MEAN && pool_kind != HISA_POOL_MAX) return HISA_ERR_ARG;
    int st = check_append(K, k_seq_stride, S, d, B, L_old, L_new, pool_rep, pool_seq_stride);
    if (st != HISA_OK) return st;
    st = check_index(q, w, qpos, K, k_seq_stride, L_new, pool_rep, pool_seq_stride, S, T, H, d, B, m, k, out_idx,
                     ws, ws_bytes);
    if (st != HISA_OK) return st;
    hipStream_t hs = static_cast<hipStream_t>(stream);
    const bool pmax = pool_kind == HISA_POOL_MAX;
    // The fused form needs the query at t = L_new-1 in every sequence (no
    // explicit positions) and the appended rows all in its own block.
    const bool fuse = qpos == nullptr && L_old < L_new && L_old / B == (L_new - 1) / B &&
                      pool_update_fusable(S, T, d, L_new, B, m);
    if (!fuse) {
        if (L_old < L_new) {
            const int64_t blk0 = L_old / B;
            st = hip_status(launch_pool_append(K, k_seq_stride, S, d, B, blk0, (L_new - 1) / B - blk0 + 1, L_new,
                                               pmax, pool_rep, pool_seq_stride, hs));
            if (st != HISA_OK) return st;
        }
        return run_index(q, w, qpos, K, k_seq_stride, L_new, pool_rep, nullptr, pool_seq_stride, S, T, H, d, B, m,
                         k, out_idx, out_score, out_blk, ws, pmax, hs);
    }
    return run_index(q, w, qpos, K, k_seq_stride, L_new, pool_rep, pool_rep, pool_seq_stride, S, T, H, d, B, m, k,
                     out_idx, out_score, out_blk, ws, pmax, hs);
}

int hisa_append_index(const uint16_t *K, int64_t k_seq_stride, int64_t L_old, int64_t L_new,
                      uint16_t *pool_mean, int64_t pool_seq_stride, const uint16_t *q, const float *w,
                      const int32_t *qpos, int S, int T, int H, int d, int B, int m, int k, int32_t *out_idx,
                      float *out_score, int32_t *out_blk, void *ws, size_t ws_bytes, void *stream) {
    return hisa_append_index_mode(K, k_seq_stride, L_old, L_new, pool_mean, pool_seq_stride, q, w, qpos, S, T, H, d,
                                  B, m, k, out_idx, out_score, out_blk, ws, ws_bytes, HISA_POOL_MEAN, stream);
}

}  // extern "C"

// ---------------------------------------------------------------- static scratch
// The workspace of hisa_append_index_static: a device array in the library,
// one copy per GPU.  In host code `scratch` names a host-side stand-in for the
// symbol, not a device address; the device address of each GPU's copy comes
// from hipGetSymbolAddress with that GPU current, looked up once per device,
// and only that address is ever handed to a kernel.
static __device__ __attribute__((aligned(256))) unsigned char scratch[HISA_STATIC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices] = {};

// Device address of `scratch` on the GPU that runs `stream`.
int static_scratch(hipStream_t stream, void **out) {
    int dev = -1;
    if (hipStreamGetDevice(stream, &dev) != hipSuccess) return HISA_ERR_HIP;
    if (dev < 0 || dev >= kMaxDevices) return HISA_ERR_UNSUPPORTED;
    std::lock_guard<std::mutex> guard(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        int cur = -1;
        if (hipGetDevice(&cur) != hipSuccess) return HISA_ERR_HIP;
        if (cur != dev && hipSetDevice(dev) != hipSuccess) return HISA_ERR_HIP;
        void *p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (cur != dev) (void)hipSetDevice(cur);
        if (e != hipSuccess || p == nullptr) return HISA_ERR_HIP;
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return HISA_OK;
}

}  // namespace

extern "C" {

int hisa_append_index_static(const uint16_t *K, int64_t k_seq_stride, int64_t L_old, int64_t L_new,
                             uint16_t *pool_mean, int64_t pool_seq_stride, const uint16_t *q, const float *w,
                             const int32_t *qpos, int S, int T, int H, int d, int B, int m, int k,
                             int32_t *out_idx, float *out_score, int32_t *out_blk, void *stream) {
    // the plain call's checks, with the scratch array standing in for the
    // workspace (its address is not needed to size it); all of them run
    // before the device is touched
    int st = check_append(K, k_seq_stride, S, d, B, L_old, L_new, pool_mean, pool_seq_stride);
    if (st != HISA_OK) return st;
    static const char kSized = 0;
    st = check_index(q, w, qpos, K, k_seq_stride, L_new, pool_mean, pool_seq_stride, S, T, H, d, B, m, k, out_idx,
                     &kSized, HISA_STATIC_SCRATCH_BYTES);
    if (st == HISA_ERR_WORKSPACE) return HISA_ERR_SCRATCH;
    if (st != HISA_OK) return st;
    void *ws = nullptr;
    st = static_scratch(static_cast<hipStream_t>(stream), &ws);
    if (st != HISA_OK) return st;
    return hisa_append_index_mode(K, k_seq_stride, L_old, L_new, pool_mean, pool_seq_stride, q, w, qpos, S, T, H, d,
                                  B, m, k, out_idx, out_score, out_blk, ws, HISA_STATIC_SCRATCH_BYTES, HISA_POOL_MEAN,
                                  stream);
}

}  // extern "C"

namespace {

// Levels 1-2 of hisa_tree_index as separate launches (any supported shape):
// own-block and own super-block representatives, super-block scores, top W,
// the blocks inside them, top m into the workspace's kept-block table.
int tree_upper_levels(const uint16_t *q, const float *w, const int32_t *qpos, const uint16_t *K,
                      int64_t k_seq_stride, int64_t L, const uint16_t *pool_rep, int64_t pool_seq_stride,
                      const uint16_t *spool_rep, int64_t spool_seq_stride, int S, int T, int H, int d, int B, int G,
                      int W, int m, int32_t *out_blk, int32_t *out_sblk, const TreeLayout &lay, char *base, bool pmax,
                      hipStream_t hs) {
    int st = HISA_OK;
    uint16_t *own_rep = reinterpret_cast<uint16_t *>(base + lay.own_rep);
    uint16_t *own_srep = reinterpret_cast<uint16_t *>(base + lay.own_srep);
    uint32_t *sblk_keys = reinterpret_cast<uint32_t *>(base + lay.sblk_keys);
    int32_t *sel_sb = reinterpret_cast<int32_t *>(base + lay.sel_sb);
    uint32_t *tblk_keys = reinterpret_cast<uint32_t *>(base + lay.tblk_keys);
    int32_t *sel_blk = reinterpret_cast<int32_t *>(base + lay.sel_blk);
    const int nq = S * T;
    const int64_t ns = ceil_div(ceil_div(L, B), G);
    const int64_t ntb = std::min<int64_t>(W, ns) * G;

    // own block and own super-block representatives of every query
    st = hip_status(launch_own_mean(K, k_seq_stride, qpos, L, S, T, d, B, pmax, own_rep, hs));
    if (st != HISA_OK) return st;
    st = hip_status(launch_own_super(pool_rep, pool_seq_stride, own_rep, qpos, L, S, T, d, B, G, pmax, own_srep, hs));
    if (st != HISA_OK) return st;

    ScoreArgs sa{};
    sa.q = q; sa.w = w; sa.qpos = qpos;
    sa.K = K; sa.k_seq_stride = k_seq_stride; sa.L = L;
    sa.S = S; sa.T = T; sa.H = H; sa.d = d;
    SelectArgs se{};
    se.qpos = qpos; se.L = L; se.T = T;
    set_stage(se, base, lay.stage);

    // level 1: super-blocks are blocks of B*G keys with the super pool as
    // their representatives; keep the top W
    sa.pool = spool_rep; sa.pool_seq_stride = spool_seq_stride; sa.own_rep = own_srep;
    sa.B = B * G; sa.m = 1;
    sa.keys = sblk_keys; sa.keys_stride = lay.sblk_stride;
    st = hip_status(launch_score(kScoreBlocks, sa, ns, hs));
    if (st != HISA_OK) return st;
    se.B = B * G; se.m = 1; se.kout = W;
    se.keys = sblk_keys; se.keys_stride = lay.sblk_stride; se.sel_blk = nullptr;
    se.out_id = sel_sb; se.out_score = nullptr; se.out_id_copy = out_sblk;
    st = hip_status(launch_select(kScoreBlocks, se, nq, ns, hs));
    if (st != HISA_OK) return st;

    // level 2: the blocks of the kept super-blocks; keep the top m
    sa.pool = pool_rep; sa.pool_seq_stride = pool_seq_stride; sa.own_rep = own_rep;
    sa.B = B; sa.G = G; sa.W = W; sa.sel_sb = sel_sb;
    sa.keys = tblk_keys; sa.keys_stride = lay.tblk_stride;
    st = hip_status(launch_score(kScoreTreeBlocks, sa, ntb, hs));
    if (st != HISA_OK) return st;
    se.B = B; se.G = G; se.m = W; se.kout = m;
    se.keys = tblk_keys; se.keys_stride = lay.tblk_stride; se.sel_blk = sel_sb;
    se.out_id = sel_blk; se.out_score = nullptr; se.out_id_copy = out_blk;
    return hip_status(launch_select(kScoreTreeBlocks, se, nq, ntb, hs));
}

}  // namespace

extern "C" {

int hisa_tree_append(const uint16_t *K, int64_t k_seq_stride, int S, int d, int B, int G, int64_t L_old,
                     int64_t L_new, uint16_t *pool_rep, int64_t pool_seq_stride, uint16_t *spool_rep,
                     int64_t spool_seq_stride, int pool_kind, void *stream) {
    if (pool_kind != HISA_POOL_MEAN && pool_kind != HISA_POOL_MAX) return HISA_ERR_ARG;
    if (G < 1) return HISA_ERR_ARG;
    if (!fanout_ok(G)) return HISA_ERR_UNSUPPORTED;
    int st = check_append(K, k_seq_stride, S, d, B, L_old, L_new, pool_rep, pool_seq_stride);
    if (st != HISA_OK) return st;
    const int64_t nblk = ceil_div(L_new, B);
    st = check_pool(spool_rep, spool_seq_stride, S, d, nblk, G);
    if (st != HISA_OK) return st;
    if (L_old == L_new) return HISA_OK;
    hipStream_t hs = static_cast<hipStream_t>(stream);
    const bool pmax = pool_kind == HISA_POOL_MAX;
    // leaf level: the blocks holding the new rows
    const int64_t blk0 = L_old / B;
    if (blk0 == nblk - 1 && tree_append_one_supported(B))     // one block (decode): both levels in one launch
        return hip_status(launch_tree_append_one(K, k_seq_stride, S, d, B, G, blk0, L_new, pmax, pool_rep,
                                                 pool_seq_stride, spool_rep, spool_seq_stride, hs));
    st = hip_status(launch_pool_append(K, k_seq_stride, S, d, B, blk0, nblk - blk0, L_new, pmax, pool_rep,
                                       pool_seq_stride, hs));
    if (st != HISA_OK) return st;
    // next level up: the super-blocks holding those blocks, from their block
    // representatives weighted by key counts
    const int64_t sb0 = blk0 / G;
    return hip_status(launch_super_append(pool_rep, pool_seq_stride, S, d, B, G, sb0, ceil_div(nblk, G) - sb0, L_new,
                                          pmax, spool_rep, spool_seq_stride, hs));
}

size_t hisa_tree_index_workspace(int S, int T, int H, int d, int64_t L, int B, int G, int W, int m, int k) {
    if (check_query_shape(S, T, H, d, L, k) != HISA_OK) return 0;
    if (check_tree_params(B, G, W, m) != HISA_OK) return 0;
    return tree_layout(S, T, d, L, B, G, W, m, k).total;
}

int hisa_tree_index(const uint16_t *q, const float *w, const int32_t *qpos, const uint16_t *K,
                    int64_t k_seq_stride, int64_t L, const uint16_t *pool_rep, int64_t pool_seq_stride,
                    const uint16_t *spool_rep, int64_t spool_seq_stride, int S, int T, int H, int d, int B, int G,
                    int W, int m, int k, int32_t *out_idx, float *out_score, int32_t *out_blk, int32_t *out_sblk,
                    void *ws, size_t ws_bytes, int pool_kind, void *stream) {
    if (pool_kind != HISA_POOL_MEAN && pool_kind != HISA_POOL_MAX) return HISA_ERR_ARG;
    int st = check_query_shape(S, T, H, d, L, k);
    if (st != HISA_OK) return st;
    st = check_tree_params(B, G, W, m);
    if (st != HISA_OK) return st;
    if (!q || !w || !out_idx || !aligned16(q)) return HISA_ERR_ARG;
    if (!qpos && T > L) return HISA_ERR_ARG;
    st = check_cache(K, k_seq_stride, S, d, L);
    if (st != HISA_OK) return st;
    st = check_pool(pool_rep, pool_seq_stride, S, d, L, B);
    if (st != HISA_OK) return st;
    st = check_pool(spool_rep, spool_seq_stride, S, d, ceil_div(L, B), G);
    if (st != HISA_OK) return st;
    if (!ws) return HISA_ERR_ARG;
    const TreeLayout lay = tree_layout(S, T, d, L, B, G, W, m, k);
    if (ws_bytes < lay.total) return HISA_ERR_WORKSPACE;

    hipStream_t hs = static_cast<hipStream_t>(stream);
    const bool pmax = pool_kind == HISA_POOL_MAX;
    char *base = align_ptr(ws);
    int32_t *sel_blk = reinterpret_cast<int32_t *>(base + lay.sel_blk);
    uint32_t *cand_keys = reinterpret_cast<uint32_t *>(base + lay.cand_keys);
    const int nq = S * T;
    bool scored = false;     // the token level's scores already in cand_keys

    if (tree_top_supported(d, L, B, G, W)) {
        // levels 1-2 in two launches (tree_top_kernel, then tree_gather_kernel
        // with the token scores for few queries, else tree_topm_kernel)
        TreeTopArgs ta{};
        ta.q = q; ta.w = w; ta.qpos = qpos;
        ta.K = K; ta.k_seq_stride = k_seq_stride; ta.L = L;
        ta.pool = pool_rep; ta.pool_seq_stride = pool_seq_stride;
        ta.spool = spool_rep; ta.spool_seq_stride = spool_seq_stride;
        ta.S = S; ta.T = T; ta.H = H; ta.d = d; ta.B = B; ta.G = G; ta.W = W; ta.m = m;
        ta.pool_max = pmax ? 1 : 0;
        ta.sel_blk = sel_blk; ta.out_blk = out_blk; ta.out_sblk = out_sblk;
        ta.sel_sb = reinterpret_cast<int32_t *>(base + lay.sel_sb);
        ta.tblk_keys = reinterpret_cast<uint32_t *>(base + lay.tblk_keys);
        ta.tblk_stride = lay.tblk_stride;
        ta.cand_keys = cand_keys; ta.cand_stride = lay.cand_stride;
        st = hip_status(launch_tree_top(ta, hs, &scored));
        if (st != HISA_OK) return st;
    } else {
        st = tree_upper_levels(q, w, qpos, K, k_seq_stride, L, pool_rep, pool_seq_stride, spool_rep,
                               spool_seq_stride, S, T, H, d, B, G, W, m, out_blk, out_sblk, lay, base, pmax, hs);
        if (st != HISA_OK) return st;
    }

    // level 3: the tokens of the kept blocks (slots past the kept count hold
    // -1 and give no candidate); keep the top k
    if (!scored) {
        ScoreArgs sa{};
        sa.q = q; sa.w = w; sa.qpos = qpos;
        sa.K = K; sa.k_seq_stride = k_seq_stride; sa.L = L;
        sa.S = S; sa.T = T; sa.H = H; sa.d = d; sa.B = B; sa.m = m; sa.sel_blk = sel_blk;
        sa.keys = cand_keys; sa.keys_stride = lay.cand_stride;
        st = hip_status(launch_score(kScoreRefine, sa, static_cast<int64_t>(m) * B, hs));
        if (st != HISA_OK) return st;
    }
    SelectArgs se{};
    se.qpos = qpos; se.L = L; se.T = T;
    set_stage(se, base, lay.stage);
    se.B = B; se.m = m; se.kout = k;
    se.keys = cand_keys; se.keys_stride = lay.cand_stride; se.sel_blk = sel_blk;
    se.out_id = out_idx; se.out_score = out_score; se.out_id_copy = nullptr;
    return hip_status(launch_select(kScoreRefine, se, nq, static_cast<int64_t>(m) * B, hs));
}



}  // extern "C"

namespace {

int check_attention_shape(int S, int T, int Ha, int Dk, int Dv, int k) {
    if (S < 1 || T < 1 || Ha < 1 || Dk < 1 || Dv < 1 || k < 1) return HISA_ERR_ARG;
    if (!attention_shape_supported(Dk, Dv)) return HISA_ERR_UNSUPPORTED;
    if (Ha % 16 != 0 || Ha > 128) return HISA_ERR_UNSUPPORTED;
    if (k > (1 << 20) || static_cast<int64_t>(S) * T > 65535) return HISA_ERR_UNSUPPORTED;
    return HISA_OK;
}

struct AttnLayout {
    int nsplit, tps;
    size_t part_o, part_m, part_l, total;
};

AttnLayout attention_layout(int S, int T, int Ha, int Dk, int Dv, int k) {
    AttnLayout l{};
    attention_split(S * T, Ha, Dk, Dv, k, l.nsplit, l.tps);
    size_t off = 0;
    if (l.nsplit > 1) {
        const size_t rows = static_cast<size_t>(S) * T * l.nsplit * Ha;
        l.part_o = off; off = align_up(off + rows * Dv * sizeof(float), kAlign);
        l.part_m = off; off = align_up(off + rows * sizeof(float), kAlign);
        l.part_l = off; off = align_up(off + rows * sizeof(float), kAlign);
    }
    l.total = off + kAlign;
    return l;
}

}  // namespace

extern "C" {

size_t hisa_sparse_attention_workspace(int S, int T, int Ha, int Dk, int Dv, int k) {
    if (check_attention_shape(S, T, Ha, Dk, Dv, k) != HISA_OK) return 0;
    return attention_layout(S, T, Ha, Dk, Dv, k).total;
}

int hisa_sparse_attention(const uint16_t *q, const uint16_t *kv, int64_t kv_seq_stride, int64_t kv_row_stride,
                          int64_t L, const int32_t *idx, int S, int T, int Ha, int Dk, int Dv, int k, float scale,
                          float *out, float *lse, void *ws, size_t ws_bytes, void *stream) {
    int st = check_attention_shape(S, T, Ha, Dk, Dv, k);
    if (st != HISA_OK) return st;
    if (L < 1) return HISA_ERR_ARG;
    if (L >= (int64_t{1} << 31)) return HISA_ERR_UNSUPPORTED;
    if (!q || !kv || !idx || !out || !aligned16(q) || !aligned16(kv) || !aligned16(out)) return HISA_ERR_ARG;
    if (kv_row_stride < Dk || (kv_row_stride & 7) != 0) return HISA_ERR_ARG;
    if (kv_seq_stride < 0 || (kv_seq_stride & 7) != 0 || (S > 1 && kv_seq_stride < L * kv_row_stride))
        return HISA_ERR_ARG;
    if (!(scale == scale) || scale > 3.0e38f || scale < -3.0e38f) return HISA_ERR_ARG;
    if (!ws) return HISA_ERR_ARG;
    const AttnLayout lay = attention_layout(S, T, Ha, Dk, Dv, k);
    if (ws_bytes < lay.total) return HISA_ERR_WORKSPACE;
    char *base = align_ptr(ws);
    AttnArgs a{};
    a.q = q; a.kv = kv; a.kv_seq_stride = kv_seq_stride; a.kv_row_stride = kv_row_stride; a.L = L;
    a.idx = idx; a.S = S; a.T = T; a.Ha = Ha; a.Dk = Dk; a.Dv = Dv; a.k = k;
    a.scale_log2 = static_cast<float>(static_cast<double>(scale) * 1.4426950408889634);
    a.nsplit = lay.nsplit; a.tps = lay.tps; a.npair = S * T * lay.nsplit;
    a.out = out; a.lse = lse;
    if (lay.nsplit > 1) {
        a.part_o = reinterpret_cast<float *>(base + lay.part_o);
        a.part_m = reinterpret_cast<float *>(base + lay.part_m);
        a.part_l = reinterpret_cast<float *>(base + lay.part_l);
    }
    return hip_status(launch_attention(a, static_cast<hipStream_t>(stream)));
}

size_t dsa_flat_workspace(int S, int T, int H, int d, int64_t L, int k) {
    if (check_query_shape(S, T, H, d, L, k) != HISA_OK) return 0;
    return flat_layout(S, T, d, L, k).total;
}

int dsa_flat_index(const uint16_t *q, const float *w, const int32_t *qpos, const uint16_t *K,
                   int64_t k_seq_stride, int64_t L, int S, int T, int H, int d, int k,
                   int32_t *out_idx, float *out_score, void *ws, size_t ws_bytes, void *stream) {
    int st = check_query_shape(S, T, H, d, L, k);
    if (st != HISA_OK) return st;
    if (!q || !w || !out_idx || !aligned16(q)) return HISA_ERR_ARG;
    if (!qpos && T > L) return HISA_ERR_ARG;
    st = check_cache(K, k_seq_stride, S, d, L);
    if (st != HISA_OK) return st;
    const FlatLayout lay = flat_layout(S, T, d, L, k);
    if (!ws) return HISA_ERR_ARG;
    if (ws_bytes < lay.total) return HISA_ERR_WORKSPACE;

    hipStream_t hs = static_cast<hipStream_t>(stream);
    char *base = align_ptr(ws);
    uint32_t *keys = reinterpret_cast<uint32_t *>(base + lay.keys);
    if (lay.block_major) {
        // many queries per sequence: the block-major refinement with every
        // block b <= b_t kept, in slot b, so key position p is token p
        FusedArgs fa{};
        fa.q = q; fa.w = w; fa.qpos = qpos;
        fa.K = K; fa.k_seq_stride = k_seq_stride; fa.L = L;
        fa.S = S; fa.T = T; fa.H = H; fa.d = d; fa.B = kFlatBlock;
        fa.nblk = static_cast<int>(ceil_div(L, kFlatBlock));
        fa.m = fa.nblk;
        fa.cand_keys = keys; fa.cand_stride = lay.stride;
        fa.bucket_off = reinterpret_cast<int32_t *>(base + lay.bucket_off);
        fa.bucket_ent = reinterpret_cast<uint32_t *>(base + lay.bucket_ent);
        st = hip_status(launch_flat_block_major(fa, hs));
    } else {
        ScoreArgs sa{};
        sa.q = q; sa.w = w; sa.qpos = qpos;
        sa.K = K; sa.k_seq_stride = k_seq_stride; sa.L = L;
        sa.keys = keys; sa.keys_stride = lay.stride;
        sa.S = S; sa.T = T; sa.H = H; sa.d = d; sa.B = 1; sa.m = 1;
        st = hip_status(launch_score(kScoreFlat, sa, L, hs));
    }
    if (st != HISA_OK) return st;
    SelectArgs se{};
    set_stage(se, align_ptr(ws), lay.stage);
    se.keys = keys; se.keys_stride = lay.stride;
    se.qpos = qpos; se.L = L; se.T = T; se.B = 1; se.m = 1;
    se.kout = k; se.out_id = out_idx; se.out_score = out_score;
    return hip_status(launch_select(kScoreFlat, se, S * T, L, hs));
}

int hisa_profile_enable(int max_launches) {
    if (max_launches < 0) return HISA_ERR_ARG;
    prof_release();
    if (max_launches == 0) return HISA_OK;
    g_prof.ev.resize(2 * static_cast<size_t>(max_launches));
    for (auto &e : g_prof.ev) {
        if (hipEventCreate(&e) != hipSuccess) {
            e = nullptr;
            prof_release();
            return HISA_ERR_HIP;
        }
    }
    g_prof.kind.assign(static_cast<size_t>(max_launches), -1);
    g_prof.cap = max_launches;
    g_prof.on = true;
    return HISA_OK;
}

int hisa_profile_read(int kind, double *total_ms, int *launches) {
    if (kind < 0 || kind >= kKindCount || !total_ms || !launches) return HISA_ERR_ARG;
    *total_ms = 0.0;
    *launches = 0;
    if (!g_prof.on || g_prof.used == 0) return HISA_OK;
    if (hipEventSynchronize(g_prof.ev[2 * g_prof.used - 1]) != hipSuccess) return HISA_ERR_HIP;
    for (int i = 0; i < g_prof.used; ++i) {
        if (g_prof.kind[i] != kind) continue;
        float ms = 0.0f;
        if (hipEventElapsedTime(&ms, g_prof.ev[2 * i], g_prof.ev[2 * i + 1]) != hipSuccess)
            return HISA_ERR_HIP;
        *total_ms += ms;
        ++*launches;
    }
    return HISA_OK;
}

int hisa_kernel_kinds(void) { return kKindCount; }

const char *hisa_kernel_name(int kind) {
    return (kind >= 0 && kind < kKindCount) ? kKindNames[kind] : "unknown";
}

}  // extern "C"
