// Internal declarations of libhisa (not part of the C ABI).
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace hisa {

// ---------------------------------------------------------------- types
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------- bf16 <-> fp32
__device__ __forceinline__ float bf16_to_f32(uint16_t h) {
    return __uint_as_float(static_cast<uint32_t>(h) << 16);
}

// fp32 -> bf16, round to nearest, ties to even (finite inputs).
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
    uint32_t u = __float_as_uint(f);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return static_cast<uint16_t>(u >> 16);
}

// ---------------------------------------------------------------- sortable keys
// Scores are ranked through an order-preserving map float -> uint32 (larger
// score -> larger key; -0 is first folded onto +0 so the two tie).  Key 0 is
// reserved for "no candidate": no finite score maps to it.
__device__ __forceinline__ uint32_t score_to_key(float f) {
    uint32_t u = __float_as_uint(f == 0.0f ? 0.0f : f);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float key_to_score(uint32_t k) {
    uint32_t u = (k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k;
    return __uint_as_float(u);
}

constexpr uint32_t kNoCandidate = 0u;

// Query position of flat query id qi = s*T + i (qpos == nullptr: t = L - T + i).
// Returns -1 for positions outside [0, L).
__device__ __forceinline__ int64_t query_pos(const int32_t *qpos, int qi, int i, int64_t L, int T) {
    int64_t t = qpos ? static_cast<int64_t>(qpos[qi]) : (L - T + i);
    return (t >= 0 && t < L) ? t : -1;
}

// ---------------------------------------------------------------- launchers
// kScoreTreeBlocks: the blocks inside a query's kept super-blocks (three-level tree)
enum ScoreMode { kScoreBlocks = 0, kScoreRefine = 1, kScoreFlat = 2, kScoreTreeBlocks = 3 };

struct ScoreArgs {
    const uint16_t *q;        // [S*T][H][d]
    const float *w;           // [S*T][H]
    const int32_t *qpos;      // [S*T] or null
    const uint16_t *K;        // key cache
    int64_t k_seq_stride;
    int64_t L;
    const uint16_t *pool;     // block means
    int64_t pool_seq_stride;
    const uint16_t *own_rep;  // [S*T][d] own-block partial means (blocks mode)
    const int32_t *sel_blk;   // [S*T][m] kept blocks, ascending, -1 padded (refine mode)
    const int32_t *sel_sb;    // [S*T][W] kept super-blocks, ascending (tree-blocks mode)
    uint32_t *keys;           // out: [S*T][keys_stride]
    int64_t keys_stride;
    int S, T, H, d, B, m;
    int G, W;                 // tree-blocks mode: blocks per super-block, kept super-blocks
};

struct SelectArgs {
    const uint32_t *keys;     // [S*T][keys_stride]
    int64_t keys_stride;
    const int32_t *qpos;
    int64_t L;
    int T, B, m;
    int G;                    // tree-blocks mode: blocks per super-block
    int kout;                 // entries per output row
    // refine mode: [S*T][m] kept blocks; tree-blocks mode: [S*T][m] kept
    // super-blocks (m is then the super-block count W)
    const int32_t *sel_blk;
    int32_t *out_id;          // [S*T][kout]
    float *out_score;         // [S*T][kout] or null
    int32_t *out_id_copy;     // [S*T][kout] or null (second copy of out_id)
    // chunked selection of long rows: two ping-pong (key, id) buffers of
    // [S*T][stage_stride] (see select_stage_len)
    uint32_t *stage_keys[2];
    int32_t *stage_ids[2];
    int64_t stage_stride;
};

constexpr int kSelMaxM = 4096;          // kept blocks the refine-mode select stages in LDS

// Length of one query's row in the chunked-selection buffers (0: not needed).
int64_t select_stage_len(int64_t max_n, int kout, int B, bool refine);

// ---------------------------------------------------------------- fused HISA path
constexpr int kFusedOwnElems = 16384;   // B*d of the staged own block
constexpr int kFusedMaxBlocks = 8192;   // ceil(L/B)

struct FusedArgs {
    const uint16_t *q;        // [S*T][H][d]
    const float *w;           // [S*T][H]
    const int32_t *qpos;      // [S*T] or null
    const uint16_t *K;
    int64_t k_seq_stride;
    int64_t L;
    const uint16_t *pool;
    int64_t pool_seq_stride;
    int S, T, H, d, B, m, k;
    int32_t *sel_blk;         // ws [S*T][m]: kept blocks, ascending, -1 padded
    int32_t *out_blk;         // [S*T][m] or null
    uint32_t *cand_keys;      // ws [S*T][cand_stride]
    int64_t cand_stride;
    int32_t *out_idx;         // [S*T][k]
    float *out_score;         // [S*T][k] or null
    // block-major refinement (see block_major_mode): for each chunk of up to
    // kChunkQueries consecutive queries of one sequence, the (query, slot)
    // pairs of its kept blocks grouped by block id
    int nblk;                 // ceil(L/B)
    int32_t *bucket_off;      // ws [nchunk][nblk + 1]
    uint32_t *bucket_ent;     // ws [nchunk][kChunkQueries * m]: (query in chunk) << 16 | slot
    // block-major block stage (block_major_mode with nblk <= kBMMaxBlocks)
    uint16_t *own_rep;        // ws [S*T][d]: own-block representative of every query
    uint32_t *blk_keys;       // ws [S*T][blk_stride]: block keys by block id
    int64_t blk_stride;
    int pool_max;             // representatives by max pooling (else mean)
    // pool entry update fused into the block stage (pool_update_fusable):
    // non-null, every own block is computed from K, and the query at t = L-1
    // writes its own block's mean into pool_out[s][b_t] (the same buffer as
    // pool; no other workgroup reads that entry)
    uint16_t *pool_out;
};

constexpr int kBMMaxBlocks = 2048;       // block-major block stage: one wave selects the top m

constexpr int kChunkQueries = 256;

bool fused_supported(int d, int64_t L, int B, int m);
// Many queries per sequence: refine block by block (each key block is read
// once per chunk of queries) instead of query by query.
bool block_major_mode(int S, int T, int d, int64_t L, int B, int m);
inline int64_t bucket_chunks(int S, int T) {
    return static_cast<int64_t>(S) * ((T + kChunkQueries - 1) / kChunkQueries);
}
hipError_t launch_fused_blocks_refine(const FusedArgs &a, hipStream_t st);
// Whether launch_fused_blocks_refine takes a path that honours pool_out (every
// path but the block-major one).
bool pool_update_fusable(int S, int T, int d, int64_t L, int B, int m);
hipError_t launch_block_major_refine(const FusedArgs &a, hipStream_t st);
hipError_t launch_block_major_blocks(const FusedArgs &a, hipStream_t st);

// The flat indexer block by block for many queries per sequence: every query
// scores every block b <= b_t of kFlatBlock keys through the block-major
// refinement (a.m = a.nblk slots, slot b = block b, so candidate position p
// is token p).  Workspace: bucket_off / bucket_ent as for block_major_mode,
// cand_keys rows of at least nblk * kFlatBlock keys.
constexpr int kFlatBlock = 128;
bool flat_block_major_mode(int S, int T, int d, int64_t L);
hipError_t launch_flat_block_major(const FusedArgs &a, hipStream_t st);

// pool_max: max-pooled representatives instead of means (everywhere below)
hipError_t launch_pool_append(const uint16_t *K, int64_t k_seq_stride, int S, int d, int B,
                              int64_t blk0, int64_t nblk, int64_t L_new, bool pool_max, uint16_t *pool,
                              int64_t pool_seq_stride, hipStream_t st);

// Super-blocks [sb0, sb0 + nsb) of the three-level tree from the block pool of
// a cache holding L_new rows (children weighted by their key counts).
hipError_t launch_super_append(const uint16_t *pool, int64_t pool_seq_stride, int S, int d, int B, int G,
                               int64_t sb0, int64_t nsb, int64_t L_new, bool pool_max, uint16_t *spool,
                               int64_t spool_seq_stride, hipStream_t st);

// Both tree levels in one launch when the new rows all lie in block blk (the
// last one) and B <= 128: block blk from K, then its super-block from the pool.
bool tree_append_one_supported(int B);
hipError_t launch_tree_append_one(const uint16_t *K, int64_t k_seq_stride, int S, int d, int B, int G, int64_t blk,
                                  int64_t L_new, bool pool_max, uint16_t *pool, int64_t pool_seq_stride,
                                  uint16_t *spool, int64_t spool_seq_stride, hipStream_t st);

// Own-block representatives of queries at the consecutive positions
// t = L - T + i (requires T <= L): one pass per block.
hipError_t launch_own_prefix_mean(const uint16_t *K, int64_t k_seq_stride, int64_t L, int S, int T, int d, int B,
                                  bool pool_max, uint16_t *own_rep, hipStream_t st);

hipError_t launch_own_mean(const uint16_t *K, int64_t k_seq_stride, const int32_t *qpos,
                           int64_t L, int S, int T, int d, int B, bool pool_max, uint16_t *own_rep,
                           hipStream_t st);

// Own super-block representative of every query (three-level tree): pools the
// block representatives pool[s][b] for st*G <= b < b_t (B keys each), then
// own_rep[qi] (t + 1 - b_t*B keys), weighted by those counts.
hipError_t launch_own_super(const uint16_t *pool, int64_t pool_seq_stride, const uint16_t *own_rep,
                            const int32_t *qpos, int64_t L, int S, int T, int d, int B, int G, bool pool_max,
                            uint16_t *own_srep, hipStream_t st);

// ---------------------------------------------------------------- three-level tree
// Upper two levels of hisa_tree_index in one kernel (hisa_tree.hip): for every
// query the top W super-blocks, then the top m blocks inside them.
struct TreeTopArgs {
    const uint16_t *q;        // [S*T][H][d]
    const float *w;           // [S*T][H]
    const int32_t *qpos;      // [S*T] or null
    const uint16_t *K;
    int64_t k_seq_stride;
    int64_t L;
    const uint16_t *pool;     // block representatives, current through row L-1
    int64_t pool_seq_stride;
    const uint16_t *spool;    // super-block representatives, current through row L-1
    int64_t spool_seq_stride;
    int S, T, H, d, B, G, W, m;
    int pool_max;
    int32_t *sel_blk;         // [S*T][m]: kept blocks, ascending, -1 padded
    int32_t *out_blk;         // [S*T][m] or null
    int32_t *out_sblk;        // [S*T][W] or null
    int32_t *sel_sb;          // [S*T][W]: kept super-blocks, ascending, -1 padded (workspace)
    uint32_t *tblk_keys;      // [S*T][tblk_stride]: keys of the kept super-blocks' blocks (workspace)
    int64_t tblk_stride;
    uint32_t *cand_keys;      // [S*T][cand_stride]: token keys, refine-mode layout (workspace)
    int64_t cand_stride;
};

bool tree_top_supported(int d, int64_t L, int B, int G, int W);
// Levels 1-2 and the top m; for few queries also the token level's scores
// (cand_keys), which *scored reports -- otherwise the caller scores them.
hipError_t launch_tree_top(const TreeTopArgs &a, hipStream_t st, bool *scored);

// ---------------------------------------------------------------- sparse attention (attention.hip)
struct AttnArgs {
    const uint16_t *q;        // [S*T][Ha][Dk]
    const uint16_t *kv;       // latent rows: key = first Dk entries, value = first Dv
    int64_t kv_seq_stride;
    int64_t kv_row_stride;
    int64_t L;
    const int32_t *idx;       // [S*T][k], entries outside [0, L) skipped
    int S, T, Ha, Dk, Dv, k;
    float scale_log2;         // scale * log2(e)
    int nsplit;               // workgroups per (query, head group) along the set
    int tps;                  // set entries per split (a multiple of 64)
    int npair;                // S*T*nsplit
    float *out;               // [S*T][Ha][Dv]
    float *lse;               // [S*T][Ha] or null
    float *part_o;            // ws [S*T*nsplit][Ha][Dv] (nsplit > 1)
    float *part_m;            // ws [S*T*nsplit][Ha]
    float *part_l;            // ws [S*T*nsplit][Ha]
};

bool attention_shape_supported(int Dk, int Dv);
void attention_split(int nq, int Ha, int Dk, int Dv, int k, int &nsplit, int &tps);
hipError_t launch_attention(const AttnArgs &a, hipStream_t st);

hipError_t launch_score(ScoreMode mode, const ScoreArgs &a, int64_t max_pos, hipStream_t st);

// max_n: an upper bound on the candidate count of every query (sizes the per-thread chunk)
hipError_t launch_select(ScoreMode mode, const SelectArgs &a, int nq, int64_t max_n, hipStream_t st);

// profiler hooks (hisa_abi.hip)
enum KernelKind {
    kKindPoolAppend = 0,
    kKindOwnMean,
    kKindScoreBlocks,
    kKindSelectBlocks,
    kKindScoreRefine,
    kKindSelectRefine,
    kKindScoreFlat,
    kKindSelectFlat,
    kKindIndexDecode,      // block stage + top-m + refinement in one launch
    kKindBucket,           // (query, slot) pairs grouped by kept block
    kKindOwnSuper,         // own super-block representatives (tree)
    kKindScoreTree,        // blocks inside the kept super-blocks (tree)
    kKindSelectTree,
    kKindTreeTop,          // super-blocks -> top W -> blocks -> top m in one launch (tree)
    kKindAttention,        // sparse attention over the selected set
    kKindAttnCombine,      // merge of the attention's split partials
    kKindBucketFlat,       // the flat indexer's (query, block) pairs grouped by block (prefill chunks)
    kKindCount
};

// When the optional profiler is recording, hands out the event pair for the
// next launch of `kind` and returns true.
bool prof_events(KernelKind kind, hipEvent_t *start, hipEvent_t *stop);

// Launch `kernel` on `st`.  While profiling, the start/stop events ride on the
// dispatch itself (hipExtLaunchKernelGGL), so they time the kernel's execution
// rather than the gap between separately enqueued markers.
template <typename F, typename... Args>
hipError_t launch(KernelKind kind, F kernel, dim3 grid, dim3 block, uint32_t shmem, hipStream_t st,
                  Args... args) {
    hipEvent_t e0, e1;
    if (prof_events(kind, &e0, &e1))
        hipExtLaunchKernelGGL(kernel, grid, block, shmem, st, e0, e1, 0, args...);
    else
        kernel<<<grid, block, shmem, st>>>(args...);
    return hipGetLastError();
}

}  // namespace hisa
