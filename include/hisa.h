/*
 * libhisa -- HISA hierarchical indexer and flat DSA indexer for token-level
 * sparse attention, hand-written HIP for AMD Instinct MI355X (gfx950).
 *
 * What is computed (pages about "HISA: Efficient Hierarchical Indexing for
 * Fine-Grained Sparse Attention", arXiv 2603.28458):
 *
 *   DSA indexer score of key x for a query with H indexer heads
 *       s(q, w, x) = sum_h w_h * ReLU(q_h . x)
 *   (the pages describe the original indexer as a lightweight dot-product
 *   scorer over the key cache; the per-head weighted ReLU form is the DSA one.)
 *
 *   dsa_flat_index   -- the flat indexer: score every key j <= t of the
 *                       prefix for each query and keep the k best; it reads
 *                       the whole prefix per query, the cost HISA removes
 *                       (arXiv abstract).
 *   hisa_pool_append -- block representatives: mean pooling of contiguous
 *                       blocks of B keys (gptget.net English summary,
 *                       "Methodology"; Chinese summary, method details),
 *                       maintained as keys are appended to the cache.
 *   hisa_index       -- the two-stage replacement of the flat indexer:
 *                       (1) score the block representatives with the original
 *                       indexer and keep the top m blocks; (2) re-score every
 *                       token of the kept blocks with the original indexer and
 *                       keep the top k tokens (same pages and sections).
 *
 * Conventions shared by every entry point
 *   - bf16 tensors are passed as uint16_t bit patterns; fp32 as float.
 *   - All tensor pointers are DEVICE pointers (hipMalloc / torch CUDA tensors)
 *     unless stated otherwise.  The caller owns every buffer.  The library
 *     makes no device allocation and keeps no state between calls (the
 *     optional profiler below is the one exception).
 *   - Work is enqueued asynchronously on `stream` (a hipStream_t, NULL = the
 *     legacy default stream).  Outputs are valid once the stream has reached
 *     the end of the call.  Calls on distinct buffers are thread-safe.
 *   - Query positions are 0-based.  A query at position t sees keys j <= t.
 *   - Ranking everywhere is (score descending, index ascending); -0 == +0.
 *   - Every argument is checked on the host before anything is enqueued; on
 *     error nothing is enqueued and a negative HISA_ERR_* code is returned.
 *     Device-side values (query positions) outside [0, L) are not errors: such
 *     a query selects nothing (its output row is all -1).
 *   - Supported shapes: d in {64, 128}; 1 <= H <= 64; B in {16,32,64,128,256};
 *     1 <= m <= 4096, m*B <= 2^20; 1 <= k <= 16384; 1 <= L < 2^31;
 *     S*T <= 65535.  Other values return HISA_ERR_UNSUPPORTED.
 *   - Strides are in elements and must be multiples of 8 (16-byte rows).
 */
#ifndef HISA_H
#define HISA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define HISA_ABI_VERSION 6   /* 2: adds hisa_append_index; 3: adds the *_mode calls (max pooling);
                                4: adds the three-level tree calls hisa_tree_*;
                                5: adds hisa_sparse_attention;
                                6: adds hisa_append_index_static and HISA_ERR_SCRATCH */

#if defined(__GNUC__)
#define HISA_API __attribute__((visibility("default")))
#else
#define HISA_API
#endif

enum hisa_status {
    HISA_OK = 0,
    HISA_ERR_ARG = -1,          /* null pointer, negative size, inconsistent stride or length */
    HISA_ERR_UNSUPPORTED = -2,  /* shape outside the supported set above */
    HISA_ERR_WORKSPACE = -3,    /* ws_bytes smaller than the *_workspace() size */
    HISA_ERR_HIP = -4,          /* a HIP runtime error while enqueuing the kernels */
    HISA_ERR_SCRATCH = -5       /* hisa_append_index_static: the call needs more than
                                   HISA_STATIC_SCRATCH_BYTES of workspace */
};

/* How block representatives are pooled (the *_mode calls; the others use mean). */
enum hisa_pool_kind {
    HISA_POOL_MEAN = 0,         /* mean of the block's keys (see hisa_pool_append) */
    HISA_POOL_MAX = 1           /* per-dimension maximum of the block's keys (see hisa_pool_append_mode) */
};

/* HISA_ABI_VERSION of the loaded library. */
HISA_API int hisa_abi_version(void);

/* Static, human-readable name of a status code (never NULL). */
HISA_API const char *hisa_status_string(int status);

/*
 * hisa_pool_append -- fold key rows [L_old, L_new) into their blocks' means.
 * (Mean-pooled block representatives: gptget.net English summary,
 * "Methodology"; maintenance as the cache grows: its "Limitations" and
 * "Future Work" sections name the storage and upkeep of the representatives.)
 *
 *   K         bf16 [S][*][d]: row j of sequence s at K + s*k_seq_stride + j*d.
 *             Rows [0, L_new) must already hold the keys.
 *   pool_mean bf16 [S][*][d]: entry b of sequence s at
 *             pool_mean + s*pool_seq_stride + b*d.  Block b covers rows
 *             [b*B, min(b*B + B, L_new)).
 *   Every block that holds at least one row of [L_old, L_new) is recomputed
 *   from K:   mean_b = bf16_RNE( fp32_RNE( (sum_j K_j in fp64, increasing j) / cnt_b ) ).
 *   The result is a pure function of K and L_new: re-running a call, or
 *   splitting [L_old, L_new) into several calls, gives the same bits as one
 *   bulk call with L_old = 0.  Cost: at most B rows read per touched block.
 *   Blocks entirely before L_old are not touched.  L_old == L_new is a no-op.
 *   Requires 0 <= L_old <= L_new; for S > 1, k_seq_stride >= L_new*d and
 *   pool_seq_stride >= ceil(L_new/B)*d.
 */
HISA_API int hisa_pool_append(const uint16_t *K, int64_t k_seq_stride, int S, int d, int B,
                              int64_t L_old, int64_t L_new,
                              uint16_t *pool_mean, int64_t pool_seq_stride, void *stream);

/* Bytes of device workspace hisa_index needs for these sizes (0 on bad sizes). */
HISA_API size_t hisa_index_workspace(int S, int T, int H, int d, int64_t L, int B, int m, int k);

/*
 * hisa_index -- the two-stage HISA indexer (drop-in for the flat indexer).
 *
 *   q        bf16 [S][T][H][d]  indexer queries (row-major, contiguous)
 *   w        fp32 [S][T][H]     per-head weights
 *   qpos     int32 [S][T] or NULL; NULL means t = L - T + i for query i.
 *   K        key cache, layout as in hisa_pool_append; rows [0, L) are read.
 *   pool_mean block means as left by hisa_pool_append(): the pool must be
 *            current through row L-1 (hisa_pool_append() with L_new = L has
 *            completed, e.g. earlier on the same stream).  The representative
 *            of a query's own block floor(t/B) is the mean of rows
 *            [floor(t/B)*B, t]: for t = L-1 that is exactly the pool entry;
 *            for any other t it is recomputed from K with the same arithmetic.
 *   Steps per query (t = its position, b_t = floor(t/B)):
 *     1. sigma_b = s(q, w, mean_b) for b = 0..b_t                      (fp32)
 *     2. M = top min(m, b_t+1) blocks by (sigma desc, b asc)
 *     3. C = { j : floor(j/B) in M, j <= t }
 *     4. s_j = s(q, w, K_j) for j in C                                 (fp32)
 *     5. top min(k, |C|) of C by (s desc, j asc)
 *   Arithmetic: bf16 x bf16 products accumulated in fp32 on the matrix cores,
 *   fp32 ReLU, weighting and head sum.
 *   out_idx   int32 [S][T][k]  selected token ids, ascending, then -1 padding.
 *   out_score fp32 [S][T][k] or NULL: s_j of out_idx (-inf for padding).
 *   out_blk   int32 [S][T][m] or NULL: M ascending, then -1 padding.
 *   ws        device workspace of at least hisa_index_workspace(...) bytes
 *             (any alignment: the size includes slack for internal
 *             alignment); contents on entry are ignored and are clobbered.
 */
HISA_API int hisa_index(const uint16_t *q, const float *w, const int32_t *qpos,
                        const uint16_t *K, int64_t k_seq_stride, int64_t L,
                        const uint16_t *pool_mean, int64_t pool_seq_stride,
                        int S, int T, int H, int d, int B, int m, int k,
                        int32_t *out_idx, float *out_score, int32_t *out_blk,
                        void *ws, size_t ws_bytes, void *stream);

/*
 * hisa_append_index -- one decode step in one call: exactly
 *     hisa_pool_append(K, k_seq_stride, S, d, B, L_old, L_new, pool_mean, pool_seq_stride, stream);
 *     hisa_index(q, w, qpos, K, k_seq_stride, L_new, pool_mean, pool_seq_stride,
 *                S, T, H, d, B, m, k, out_idx, out_score, out_blk, ws, ws_bytes, stream);
 * with the same outputs and the pool left with the same bits.  (The pages keep
 * the block summaries up to date as keys are appended: page "Hierarchical
 * Indexing Makes Sparse Attention Actually Fast", section "HISA's Approach:
 * Hierarchical Summarization of the KV Cache".)
 * When qpos is NULL, every appended row lies in the last block
 * (floor(L_old/B) == floor((L_new-1)/B) and L_old < L_new) and the batch does
 * not take the block-by-block prefill path (it does when T >= 128), the last
 * block's mean is computed once, by the block stage of the query at
 * t = L_new-1, and stored to the pool from there instead of in a launch of
 * its own.  Otherwise the two calls run as written above.
 *   The pool must be current through row L_old-1 on entry (as for a
 *   hisa_pool_append() / hisa_index() pair).  Workspace: hisa_index_workspace()
 *   with L = L_new.  Argument checks and errors are those of the two calls;
 *   nothing is enqueued when either would reject its arguments.
 */
HISA_API int hisa_append_index(const uint16_t *K, int64_t k_seq_stride, int64_t L_old, int64_t L_new,
                               uint16_t *pool_mean, int64_t pool_seq_stride,
                               const uint16_t *q, const float *w, const int32_t *qpos,
                               int S, int T, int H, int d, int B, int m, int k,
                               int32_t *out_idx, float *out_score, int32_t *out_blk,
                               void *ws, size_t ws_bytes, void *stream);

/*
 * Max pooling (the *_mode calls with pool_kind = HISA_POOL_MAX).  Page
 * "Hierarchical Indexing Makes Sparse Attention Actually Fast", section "HISA's
 * Approach: Hierarchical Summarization of the KV Cache", names max pooling
 * beside mean pooling for the coarse summaries of a group of keys.  Here a
 * block's representative is then, per dimension, the largest of its keys'
 * values (compared as real numbers; among equal values, which only +0 and -0
 * can be with different bits, the one of the lowest row), with no rounding;
 * a query's own block is represented over its rows up to t, as for the mean.
 * Each *_mode call is its plain counterpart with that representative; with
 * pool_kind = HISA_POOL_MEAN it is exactly the plain call.  A pool built with
 * one kind must be used with the same kind.  pool_kind outside the enum
 * returns HISA_ERR_ARG.
 */
HISA_API int hisa_pool_append_mode(const uint16_t *K, int64_t k_seq_stride, int S, int d, int B,
                                   int64_t L_old, int64_t L_new,
                                   uint16_t *pool_rep, int64_t pool_seq_stride, int pool_kind, void *stream);
HISA_API int hisa_index_mode(const uint16_t *q, const float *w, const int32_t *qpos,
                             const uint16_t *K, int64_t k_seq_stride, int64_t L,
                             const uint16_t *pool_rep, int64_t pool_seq_stride,
                             int S, int T, int H, int d, int B, int m, int k,
                             int32_t *out_idx, float *out_score, int32_t *out_blk,
                             void *ws, size_t ws_bytes, int pool_kind, void *stream);
HISA_API int hisa_append_index_mode(const uint16_t *K, int64_t k_seq_stride, int64_t L_old, int64_t L_new,
                                    uint16_t *pool_rep, int64_t pool_seq_stride,
                                    const uint16_t *q, const float *w, const int32_t *qpos,
                                    int S, int T, int H, int d, int B, int m, int k,
                                    int32_t *out_idx, float *out_score, int32_t *out_blk,
                                    void *ws, size_t ws_bytes, int pool_kind, void *stream);

/*
 * hisa_append_index_static -- hisa_append_index (mean pooling) for callers
 * that cannot allocate device memory: code under HIP graph capture, tight
 * serving loops, and harnesses that forbid hipMalloc.  The arguments, results
 * and errors are those of hisa_append_index without ws / ws_bytes: the
 * workspace is instead a device array inside the library of
 * HISA_STATIC_SCRATCH_BYTES (16 MiB), one copy per GPU, held until the
 * process ends.  The call itself allocates nothing (no hipMalloc, no library
 * routine that allocates); on its first use on a device it looks up that
 * device's copy of the array (the device that owns `stream`, or the current
 * device for the NULL stream).
 *   - A call whose workspace, hisa_index_workspace(S, T, H, d, L_new, B, m, k),
 *     exceeds HISA_STATIC_SCRATCH_BYTES returns HISA_ERR_SCRATCH and enqueues
 *     nothing.  16 MiB holds, for example, a decode batch of 64 queries with
 *     m*B = 16384 candidates each over 2^20 keys (6.1 MiB); a 4096-query
 *     prefill chunk over 2^17 keys (147 MiB) does not fit.
 *   - Every call on one GPU shares that GPU's array, which keeps the last
 *     call's contents (nothing in it needs to start at zero).  Calls that can
 *     overlap on one GPU -- on different streams, or from different threads
 *     without ordering -- race on it and must not be issued; calls ordered on
 *     one stream are fine.
 */
#define HISA_STATIC_SCRATCH_BYTES ((size_t)16 << 20)
HISA_API int hisa_append_index_static(const uint16_t *K, int64_t k_seq_stride, int64_t L_old, int64_t L_new,
                                      uint16_t *pool_mean, int64_t pool_seq_stride,
                                      const uint16_t *q, const float *w, const int32_t *qpos,
                                      int S, int T, int H, int d, int B, int m, int k,
                                      int32_t *out_idx, float *out_score, int32_t *out_blk, void *stream);

/*
 * Three-level tree: super-blocks -> blocks -> tokens.  Page "Hierarchical
 * Indexing Makes Sparse Attention Actually Fast", section "HISA's Approach:
 * Hierarchical Summarization of the KV Cache", organises the summaries of the
 * key cache as a tree searched top-down with a beam of W nodes per level, the
 * tree kept current by refreshing only the nodes on the path from a new key up
 * to the root.  Here the tree has three levels: blocks of B keys (the pool of
 * hisa_pool_append) grouped into super-blocks of G consecutive blocks.
 *
 *   Super-block representative: the pooling of pool_kind (mean or max, as for
 *   blocks) over its blocks' representatives, in block order, taken as rows:
 *       mean_u = bf16_RNE( fp32_RNE( (sum_b pool_b in fp64, increasing b) / cnt_u ) )
 *   over the blocks b in [u*G, min(u*G + G, ceil(L/B))).  For max pooling it
 *   equals the max over the super-block's keys.
 *
 * hisa_tree_append -- hisa_pool_append_mode of rows [L_old, L_new) into the
 *   block pool, then the same recomputation one level up: every super-block
 *   holding a recomputed block is recomputed from the block pool.
 *   spool_rep bf16 [S][*][d]: entry u of sequence s at spool_rep +
 *             s*spool_seq_stride + u*d.  For S > 1, spool_seq_stride >=
 *             ceil(ceil(L_new/B)/G)*d.
 *   G in {1, 2, 4, ..., 256}.  Other arguments and checks as for
 *   hisa_pool_append_mode.  Both pools are pure functions of K and L_new.
 *
 * hisa_tree_index -- per query (t, b_t = floor(t/B), u_t = floor(b_t/G)):
 *     1. score every super-block u <= u_t; super-blocks u < u_t use the spool
 *        entry, u_t uses the pooling of blocks u_t*G .. b_t-1 from the pool
 *        followed by the query's own-block representative (rows b_t*B .. t);
 *        keep the top min(W, u_t+1) by (score desc, u asc);
 *     2. score the blocks b <= b_t of the kept super-blocks (pool entries,
 *        and the own-block representative for b_t); keep the top m;
 *     3. score the tokens j <= t of the kept blocks; keep the top k.
 *   Scores, ranking and tie-break as in hisa_index.  With W >= u_t+1 the
 *   result is hisa_index's; with G = 1 (a super-block is a block) it is
 *   hisa_index's with m replaced by min(m, W).
 *   pool_rep, spool_rep: current through row L-1 (hisa_tree_append with
 *            L_new = L has completed).
 *   out_idx, out_score, out_blk: as in hisa_index (out_blk lists the kept
 *            blocks, at most min(m, number of blocks in step 2)).
 *   out_sblk int32 [S][T][W] or NULL: kept super-blocks, ascending, -1 padded.
 *   Supported: B, m, k, H, d, S*T as for hisa_index; G as above;
 *   1 <= W <= 4096, W*G <= 2^20.
 *   ws: at least hisa_tree_index_workspace(...) bytes, as for hisa_index.
 */
HISA_API int hisa_tree_append(const uint16_t *K, int64_t k_seq_stride, int S, int d, int B, int G,
                              int64_t L_old, int64_t L_new,
                              uint16_t *pool_rep, int64_t pool_seq_stride,
                              uint16_t *spool_rep, int64_t spool_seq_stride, int pool_kind, void *stream);
HISA_API size_t hisa_tree_index_workspace(int S, int T, int H, int d, int64_t L, int B, int G, int W, int m, int k);
HISA_API int hisa_tree_index(const uint16_t *q, const float *w, const int32_t *qpos,
                             const uint16_t *K, int64_t k_seq_stride, int64_t L,
                             const uint16_t *pool_rep, int64_t pool_seq_stride,
                             const uint16_t *spool_rep, int64_t spool_seq_stride,
                             int S, int T, int H, int d, int B, int G, int W, int m, int k,
                             int32_t *out_idx, float *out_score, int32_t *out_blk, int32_t *out_sblk,
                             void *ws, size_t ws_bytes, int pool_kind, void *stream);

/*
 * hisa_sparse_attention -- the step after the indexer: attention computed
 * only over each query's selected tokens (arXiv abstract, mlsanity.com page:
 * the downstream sparse attention attends over the selected subset, the
 * token-level top-k set the Sparse MLA operator consumes).  The pages give no
 * formula for that operator; here it is softmax attention restricted to the
 * set, in the decode form of multi-head latent attention: every token stores
 * one latent row shared by all heads, whose first Dk entries are its key and
 * whose first Dv entries (Dv <= Dk) are its value.  For head h of query
 * (s, i) and the listed tokens j = idx[s][i][0..k) with 0 <= j < L (other
 * entries, such as the -1 padding of the indexers' outputs, are skipped; a
 * token listed twice counts twice):
 *     s_j   = scale * (q_h . kv_j[0..Dk))          (bf16 x bf16, fp32 accumulation)
 *     out_h = sum_j softmax(s)_j kv_j[0..Dv)
 *     lse_h = ln sum_j exp(s_j)
 * An empty set gives out = 0 and lse = -inf.
 *   Precision: each softmax weight is rounded to bf16 for the value product
 *   (fp32 accumulation) and the output is normalised by the sum of the
 *   rounded weights, so it is a convex combination of the values with
 *   weights within 2^-8 (relative) of the exact softmax.
 *   q      bf16 [S][T][Ha][Dk], contiguous.
 *   kv     bf16 latent cache: row j of sequence s at kv + s*kv_seq_stride +
 *          j*kv_row_stride (kv_row_stride >= Dk, a multiple of 8; for S > 1
 *          kv_seq_stride >= L*kv_row_stride).
 *   idx    int32 [S][T][k] (e.g. out_idx of hisa_index).
 *   out    fp32 [S][T][Ha][Dv]; lse fp32 [S][T][Ha] or NULL.
 *   ws     at least hisa_sparse_attention_workspace(...) bytes (partial
 *          results when a query's set is split over several workgroups).
 *   Supported: (Dk, Dv) in {(64,64), (128,128), (192,128), (576,512)};
 *   Ha a multiple of 16 up to 128; 1 <= k <= 2^20; S*T <= 65535;
 *   1 <= L < 2^31; scale finite.
 */
HISA_API size_t hisa_sparse_attention_workspace(int S, int T, int Ha, int Dk, int Dv, int k);
HISA_API int hisa_sparse_attention(const uint16_t *q, const uint16_t *kv, int64_t kv_seq_stride,
                                   int64_t kv_row_stride, int64_t L, const int32_t *idx,
                                   int S, int T, int Ha, int Dk, int Dv, int k, float scale,
                                   float *out, float *lse, void *ws, size_t ws_bytes, void *stream);

/* Bytes of device workspace dsa_flat_index needs for these sizes (0 on bad sizes). */
HISA_API size_t dsa_flat_workspace(int S, int T, int H, int d, int64_t L, int k);

/*
 * dsa_flat_index -- the flat DSA indexer (the baseline HISA replaces): for each
 * query, s_j = s(q, w, K_j) for every j <= t, keep the top min(k, t+1) by
 * (s desc, j asc).  Same argument conventions and output layout as hisa_index.
 * Uses the same scoring arithmetic as hisa_index, so for a given (query, key)
 * both return the same fp32 bits.
 */
HISA_API int dsa_flat_index(const uint16_t *q, const float *w, const int32_t *qpos,
                            const uint16_t *K, int64_t k_seq_stride, int64_t L,
                            int S, int T, int H, int d, int k,
                            int32_t *out_idx, float *out_score,
                            void *ws, size_t ws_bytes, void *stream);

/*
 * Optional kernel profiler (for benchmarks; not thread-safe).
 * hisa_profile_enable(n > 0) starts recording a HIP event pair around every
 * kernel the library enqueues, for up to n kernel launches; n == 0 stops and
 * releases the events.  hisa_profile_read() synchronises the recorded events
 * and returns, for kernel kind `kind`, the summed duration in milliseconds and
 * the number of launches recorded since enable; it returns HISA_ERR_ARG for an
 * unknown kind.  hisa_kernel_name(kind) names kind 0..hisa_kernel_kinds()-1.
 */
HISA_API int hisa_profile_enable(int max_launches);
HISA_API int hisa_profile_read(int kind, double *total_ms, int *launches);
HISA_API int hisa_kernel_kinds(void);
HISA_API const char *hisa_kernel_name(int kind);

#ifdef __cplusplus
}
#endif

#endif /* HISA_H */
