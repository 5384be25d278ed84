/*
 * HISA hierarchical indexer and flat DSA indexer -- CPU ORACLE.
 *
 * TEST INFRASTRUCTURE ONLY.  Plain, slow, obviously correct reference of what
 * the indexing path computes.  Only the test-suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library; the product path never
 * does.  It shares no code, header, table or helper with the HIP library.
 *
 * Sources (the pages about "HISA: Efficient Hierarchical Indexing for
 * Fine-Grained Sparse Attention", arXiv 2603.28458):
 *   [P2-Method]  gptget.net English summary, "Methodology": two stages, block
 *                representatives by mean pooling, top-m blocks, then the
 *                original indexer on the tokens of the kept blocks.
 *   [P5-Detail]  gptget.net Chinese summary, method details (方法详解): split
 *                the length-L prefix into contiguous blocks of size B, mean-pool
 *                each block, score every block representative with the
 *                original indexer, keep the top m blocks, take all their
 *                tokens, re-score them with the original indexer, keep k.
 *   [Abstract]   arXiv abstract (mlsanity.com page): the indexer scores every
 *                historical key of the prefix for each query (flat DSA); HISA
 *                keeps the token-level top-k set the sparse attention consumes.
 *   [P1-Summary] "Hierarchical Indexing Makes Sparse Attention Actually Fast",
 *                section "HISA's Approach: Hierarchical Summarization of the KV
 *                Cache": the coarse summaries pool the keys of a group by mean
 *                pooling or max pooling.
 *
 * Readings where the pages are silent (each also listed in the design notes):
 *   - indexer score s(q,w,x) = sum_h w_h * max(0, q_h . x), no extra scale;
 *   - a query at position t sees keys j <= t (inclusive causal prefix);
 *   - blocks are aligned at token 0; the query's own block b_t = floor(t/B) is
 *     represented by the mean of its keys j in [b_t*B, t] only;
 *   - representative = bf16_RNE(fp32_RNE(sum_j K_j / cnt)), the sum taken in
 *     fp64 in increasing j (bf16 representatives feed a bf16 scorer);
 *   - ranking is by (score descending, index ascending); -0 equals +0;
 *   - fewer than k candidates: the rest of the row is -1 (score -inf).
 *
 * Arithmetic: every dot product and the head sum are accumulated in fp64
 * from the exact bf16/fp32 inputs; ranks are taken on the fp64 values; the
 * reported scores are those values rounded to fp32.
 *
 * Build: gcc -O2 -fopenmp -ffp-contract=off -shared -fPIC (no fast-math).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* ---------- bf16 <-> binary64/binary32 (data decoding, not method) ---------- */

static double bf16_val(uint16_t h)
{
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* float32 -> bf16, round to nearest, ties to even (finite inputs). */
static uint16_t bf16_round(float f)
{
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

/* ---------- the indexer score (DSA form) ---------- */

/* s(q, w, x) = sum over heads h of w_h * ReLU(q_h . x)
 * q: H x d bf16 (row h = head h), w: H fp32, x: d bf16. */
double oracle_score(const uint16_t *q, const float *w, const uint16_t *x, int H, int d)
{
    double s = 0.0;
    for (int h = 0; h < H; ++h) {
        double dot = 0.0;
        for (int i = 0; i < d; ++i)
            dot += bf16_val(q[(size_t)h * d + i]) * bf16_val(x[i]);
        double relu = dot > 0.0 ? dot : 0.0;
        s += (double)w[h] * relu;
    }
    return s;
}

/* ---------- mean pooling of a run of key rows ---------- */

/* out = bf16(fp32(mean of rows [row0, row1) of K)), K rows of d bf16. */
void oracle_mean_rows(const uint16_t *K, int64_t row0, int64_t row1, int d, uint16_t *out)
{
    double cnt = (double)(row1 - row0);
    for (int i = 0; i < d; ++i) {
        double sum = 0.0;
        for (int64_t j = row0; j < row1; ++j)
            sum += bf16_val(K[(size_t)j * d + i]);
        out[i] = bf16_round((float)(sum / cnt));
    }
}

/* ---------- max pooling of a run of key rows [P1-Summary] ---------- */

/* out[i] = the largest of K[j][i] over rows j in [row0, row1), compared as
 * real values; among equal values (only +0 and -0 can be equal with
 * different bits) the one of the lowest row is kept.  Exact: no rounding. */
void oracle_max_rows(const uint16_t *K, int64_t row0, int64_t row1, int d, uint16_t *out)
{
    for (int i = 0; i < d; ++i) {
        uint16_t best = K[(size_t)row0 * d + i];
        for (int64_t j = row0 + 1; j < row1; ++j) {
            uint16_t h = K[(size_t)j * d + i];
            if (bf16_val(h) > bf16_val(best)) best = h;
        }
        out[i] = best;
    }
}

/* Block representative of rows [row0, row1): mode 0 = mean, 1 = max. */
static void rep_rows(const uint16_t *K, int64_t row0, int64_t row1, int d, int mode, uint16_t *out)
{
    if (mode == 1)
        oracle_max_rows(K, row0, row1, d, out);
    else
        oracle_mean_rows(K, row0, row1, d, out);
}

/* Block pool of a key cache holding L rows: block b covers rows
 * [b*B, min(b*B + B, L)).  reps: [S, ceil(L/B), d]; mode as rep_rows. */
void oracle_pool_mode(const uint16_t *K, int64_t k_seq_stride, int S, int64_t L, int d, int B,
                      int mode, uint16_t *reps)
{
    int64_t nblk = (L + B - 1) / B;
    for (int s = 0; s < S; ++s) {
        const uint16_t *Ks = K + (size_t)s * k_seq_stride;
#pragma omp parallel for schedule(static)
        for (int64_t b = 0; b < nblk; ++b) {
            int64_t r1 = (b + 1) * B < L ? (b + 1) * B : L;
            rep_rows(Ks, b * B, r1, d, mode, reps + ((size_t)s * nblk + b) * d);
        }
    }
}

void oracle_pool(const uint16_t *K, int64_t k_seq_stride, int S, int64_t L, int d, int B,
                 uint16_t *means)
{
    oracle_pool_mode(K, k_seq_stride, S, L, d, B, 0, means);
}

/* ---------- ranking: (score desc, index asc) ---------- */

typedef struct {
    double s;
    int64_t i;
} cand_t;

static int by_score_then_index(const void *pa, const void *pb)
{
    const cand_t *a = (const cand_t *)pa, *b = (const cand_t *)pb;
    if (a->s > b->s) return -1;
    if (a->s < b->s) return 1;
    return (a->i < b->i) ? -1 : (a->i > b->i);
}

static int by_index(const void *pa, const void *pb)
{
    int32_t a = *(const int32_t *)pa, b = *(const int32_t *)pb;
    return (a > b) - (a < b);
}

/* Keep the first min(k, n) entries of the ranked list; pad with -1 / -inf. */
static int emit_top(cand_t *c, int64_t n, int k, int32_t *out_idx, float *out_score)
{
    qsort(c, (size_t)n, sizeof *c, by_score_then_index);
    int keff = n < k ? (int)n : k;
    for (int i = 0; i < keff; ++i) {
        out_idx[i] = (int32_t)c[i].i;
        if (out_score) out_score[i] = (float)c[i].s;
    }
    for (int i = keff; i < k; ++i) {
        out_idx[i] = -1;
        if (out_score) out_score[i] = -INFINITY;
    }
    return keff;
}

/* ---------- flat DSA indexer: every key of the prefix ---------- */

/* Top-k over j in [0, t] of s(q, w, K_j).  Returns k_eff = min(k, t+1).
 * Output is ranked (score desc, index asc).  all_scores (nullable, t+1). */
int oracle_flat_query(const uint16_t *q, const float *w, const uint16_t *K, int H, int d,
                      int64_t t, int k, int32_t *out_idx, float *out_score, double *all_scores)
{
    int64_t n = t + 1;
    cand_t *c = (cand_t *)malloc((size_t)n * sizeof *c);
    if (!c) return -1;
    for (int64_t j = 0; j < n; ++j) {
        c[j].s = oracle_score(q, w, K + (size_t)j * d, H, d);
        c[j].i = j;
        if (all_scores) all_scores[j] = c[j].s;
    }
    int keff = emit_top(c, n, k, out_idx, out_score);
    free(c);
    return keff;
}

/* ---------- HISA: token refinement inside a given block set ---------- */

/* Candidates C = { j : floor(j/B) in blocks, j <= t }; top-k of s(q,w,K_j) over C.
 * blocks: nsel distinct block ids (any order).  Returns k_eff = min(k, |C|).
 * cand_count (nullable) receives |C|. */
int oracle_refine_query(const uint16_t *q, const float *w, const uint16_t *K, int H, int d,
                        int64_t t, int B, const int32_t *blocks, int nsel, int k,
                        int32_t *out_idx, float *out_score, int64_t *cand_count)
{
    int64_t n = 0;
    cand_t *c = (cand_t *)malloc(((size_t)nsel * B + 1) * sizeof *c);
    if (!c) return -1;
    for (int b = 0; b < nsel; ++b) {
        int64_t j0 = (int64_t)blocks[b] * B;
        for (int64_t j = j0; j < j0 + B && j <= t; ++j) {
            c[n].s = oracle_score(q, w, K + (size_t)j * d, H, d);
            c[n].i = j;
            ++n;
        }
    }
    if (cand_count) *cand_count = n;
    int keff = emit_top(c, n, k, out_idx, out_score);
    free(c);
    return keff;
}

/* ---------- HISA: full two-stage query ---------- */

/* One query at position t against the key cache K (rows 0..t are read).
 *  full_means (nullable): precomputed bf16 means of complete blocks
 *      ([b][d] for b < floor(t/B)); when null they are computed here.
 *  out_blk [m]: kept block ids, ascending, -1 padded.
 *  blk_score (nullable) [floor(t/B)+1]: fp64 block scores.
 *  Returns k_eff. */
int oracle_hisa_query_mode(const uint16_t *q, const float *w, const uint16_t *K,
                           const uint16_t *full_means, int H, int d, int64_t t, int B, int m, int k,
                           int mode, int32_t *out_idx, float *out_score, int32_t *out_blk,
                           double *blk_score)
{
    int64_t bt = t / B;          /* the query's own block */
    int64_t nb = bt + 1;         /* blocks visible to the query */
    uint16_t *rep = (uint16_t *)malloc((size_t)d * sizeof *rep);
    cand_t *bc = (cand_t *)malloc((size_t)nb * sizeof *bc);
    int32_t *sel = (int32_t *)malloc((size_t)(m > 0 ? m : 1) * sizeof *sel);
    if (!rep || !bc || !sel) {
        free(rep); free(bc); free(sel);
        return -1;
    }
    /* stage 1: score every block representative with the original indexer */
    for (int64_t b = 0; b < nb; ++b) {
        const uint16_t *r;
        if (b < bt && full_means) {
            r = full_means + (size_t)b * d;
        } else {
            int64_t r1 = (b < bt) ? (b + 1) * B : t + 1;
            rep_rows(K, b * B, r1, d, mode, rep);
            r = rep;
        }
        bc[b].s = oracle_score(q, w, r, H, d);
        bc[b].i = b;
        if (blk_score) blk_score[b] = bc[b].s;
    }
    /* keep the top m blocks */
    qsort(bc, (size_t)nb, sizeof *bc, by_score_then_index);
    int meff = nb < m ? (int)nb : m;
    for (int i = 0; i < meff; ++i) sel[i] = (int32_t)bc[i].i;
    qsort(sel, (size_t)meff, sizeof *sel, by_index);
    for (int i = 0; i < m; ++i) out_blk[i] = i < meff ? sel[i] : -1;
    /* stage 2: original indexer on every token of the kept blocks */
    int keff = oracle_refine_query(q, w, K, H, d, t, B, sel, meff, k, out_idx, out_score, NULL);
    free(rep); free(bc); free(sel);
    return keff;
}

/* Mean-pooled representatives (the pages' main reading). */
int oracle_hisa_query(const uint16_t *q, const float *w, const uint16_t *K,
                      const uint16_t *full_means, int H, int d, int64_t t, int B, int m, int k,
                      int32_t *out_idx, float *out_score, int32_t *out_blk, double *blk_score)
{
    return oracle_hisa_query_mode(q, w, K, full_means, H, d, t, B, m, k, 0, out_idx, out_score,
                                  out_blk, blk_score);
}

/* ---------- three-level hierarchy: super-blocks -> blocks -> tokens [P1-Summary] ---------- */

/* The summary page's tree read as three levels over the key cache: blocks of
 * B keys grouped into super-blocks of G blocks.  Every node summarises a
 * group of tokens by mean (or max) pooling over those tokens; the page keeps
 * the tree current by updating only the path from a new key's leaf to the
 * root, so a node's summary is formed from its children's:
 *   - a block pools its keys (rep_rows);
 *   - a super-block's mean is the mean over its tokens written through its
 *     children: each child block's representative weighted by the number of
 *     keys it covers, bf16(fp32(sum_b cnt_b * r_b / sum_b cnt_b)), the sum in
 *     fp64 in block order (cnt_b * r_b is exact);
 *   - a super-block's max is the max of its children's maxima, which is the
 *     max over its tokens.
 * A node that holds the query position t covers its tokens up to t: the own
 * block pools its keys j <= t, and the own super-block its complete blocks
 * (B keys each) and then the own block (t + 1 - floor(t/B)*B keys).
 * The query keeps the W best super-blocks, then the m best of the blocks
 * inside them (blocks b <= floor(t/B)), then the k best tokens j <= t of
 * those blocks; every ranking is (score desc, id asc).
 *  out_sblk [W]: kept super-blocks, ascending, -1 padded (nullable).
 *  out_blk [m]: kept blocks, ascending, -1 padded.
 *  out_sscore [floor(t/(B*G)) + 1]: score of every super-block (nullable).
 * Returns k_eff, or -1 on allocation failure. */

/* representative of block b as the query at t sees it (own block: keys <= t) */
static void block_rep_at(const uint16_t *K, int64_t b, int64_t t, int B, int d, int mode, uint16_t *out)
{
    int64_t bt = t / B;
    rep_rows(K, b * B, b < bt ? (b + 1) * B : t + 1, d, mode, out);
}

/* Summary of a super-block from its n children in order: kids [n][d] (their
 * representatives) covering cnt[c] keys each.  mode 0: the count-weighted
 * mean; mode 1: the max of the children (the earliest among equal values). */
static void super_rep(const uint16_t *kids, const int64_t *cnt, int64_t n, int d, int mode, uint16_t *out)
{
    if (mode == 1) {
        oracle_max_rows(kids, 0, n, d, out);
        return;
    }
    double total = 0.0;
    for (int64_t c = 0; c < n; ++c) total += (double)cnt[c];
    for (int i = 0; i < d; ++i) {
        double sum = 0.0;
        for (int64_t c = 0; c < n; ++c)
            sum += (double)cnt[c] * bf16_val(kids[(size_t)c * d + i]);
        out[i] = bf16_round((float)(sum / total));
    }
}

/* Super-block pool of a key cache holding L rows: super-block u covers blocks
 * [u*G, min(u*G + G, ceil(L/B))), the last block holding L - (ceil(L/B)-1)*B
 * keys.  reps: [S, ceil(ceil(L/B)/G), d]; mode as rep_rows. */
int oracle_super_pool(const uint16_t *K, int64_t k_seq_stride, int S, int64_t L, int d, int B, int G,
                      int mode, uint16_t *reps)
{
    int64_t nblk = (L + B - 1) / B, nsb = (nblk + G - 1) / G;
    uint16_t *kids = (uint16_t *)malloc((size_t)G * d * sizeof *kids);
    int64_t *cnt = (int64_t *)malloc((size_t)G * sizeof *cnt);
    if (!kids || !cnt) {
        free(kids); free(cnt);
        return -1;
    }
    for (int s = 0; s < S; ++s) {
        const uint16_t *Ks = K + (size_t)s * k_seq_stride;
        for (int64_t u = 0; u < nsb; ++u) {
            int64_t b1 = (u + 1) * G < nblk ? (u + 1) * G : nblk;
            for (int64_t b = u * G; b < b1; ++b) {
                int64_t r1 = (b + 1) * B < L ? (b + 1) * B : L;
                rep_rows(Ks, b * B, r1, d, mode, kids + (size_t)(b - u * G) * d);
                cnt[b - u * G] = r1 - b * B;
            }
            super_rep(kids, cnt, b1 - u * G, d, mode, reps + ((size_t)s * nsb + u) * d);
        }
    }
    free(kids); free(cnt);
    return 0;
}

int oracle_tree_query(const uint16_t *q, const float *w, const uint16_t *K, int H, int d, int64_t t,
                      int B, int G, int W, int m, int k, int mode, int32_t *out_idx, float *out_score,
                      int32_t *out_blk, int32_t *out_sblk, double *out_sscore)
{
    int64_t bt = t / B, st = bt / G;
    int64_t ns = st + 1;             /* super-blocks visible to the query */
    uint16_t *rep = (uint16_t *)malloc((size_t)d * sizeof *rep);
    uint16_t *kids = (uint16_t *)malloc((size_t)G * d * sizeof *kids);
    int64_t *cnt = (int64_t *)malloc((size_t)G * sizeof *cnt);
    cand_t *sc = (cand_t *)malloc((size_t)ns * sizeof *sc);
    int32_t *ssel = (int32_t *)malloc((size_t)(W > 0 ? W : 1) * sizeof *ssel);
    cand_t *bc = (cand_t *)malloc(((size_t)(W > 0 ? W : 1) * G) * sizeof *bc);
    int32_t *sel = (int32_t *)malloc((size_t)(m > 0 ? m : 1) * sizeof *sel);
    if (!rep || !kids || !cnt || !sc || !ssel || !bc || !sel) {
        free(rep); free(kids); free(cnt); free(sc); free(ssel); free(bc); free(sel);
        return -1;
    }
    /* level 1: every super-block, summarised over its tokens j <= t through
     * its children (complete blocks B keys each, the own block t+1-bt*B) */
    for (int64_t u = 0; u < ns; ++u) {
        int64_t b1 = (u < st) ? (u + 1) * G : bt + 1;     /* children u*G .. b1-1 */
        for (int64_t b = u * G; b < b1; ++b) {
            block_rep_at(K, b, t, B, d, mode, kids + (size_t)(b - u * G) * d);
            cnt[b - u * G] = b < bt ? B : t + 1 - bt * B;
        }
        super_rep(kids, cnt, b1 - u * G, d, mode, rep);
        sc[u].s = oracle_score(q, w, rep, H, d);
        sc[u].i = u;
        if (out_sscore) out_sscore[u] = sc[u].s;
    }
    qsort(sc, (size_t)ns, sizeof *sc, by_score_then_index);
    int weff = ns < W ? (int)ns : W;
    for (int i = 0; i < weff; ++i) ssel[i] = (int32_t)sc[i].i;
    qsort(ssel, (size_t)weff, sizeof *ssel, by_index);
    if (out_sblk)
        for (int i = 0; i < W; ++i) out_sblk[i] = i < weff ? ssel[i] : -1;
    /* level 2: the blocks of the kept super-blocks */
    int64_t nc = 0;
    for (int i = 0; i < weff; ++i) {
        for (int64_t b = (int64_t)ssel[i] * G; b < (int64_t)(ssel[i] + 1) * G && b <= bt; ++b) {
            block_rep_at(K, b, t, B, d, mode, rep);
            bc[nc].s = oracle_score(q, w, rep, H, d);
            bc[nc].i = b;
            ++nc;
        }
    }
    qsort(bc, (size_t)nc, sizeof *bc, by_score_then_index);
    int meff = nc < m ? (int)nc : m;
    for (int i = 0; i < meff; ++i) sel[i] = (int32_t)bc[i].i;
    qsort(sel, (size_t)meff, sizeof *sel, by_index);
    for (int i = 0; i < m; ++i) out_blk[i] = i < meff ? sel[i] : -1;
    /* level 3: the original indexer on the tokens of the kept blocks */
    int keff = oracle_refine_query(q, w, K, H, d, t, B, sel, meff, k, out_idx, out_score, NULL);
    free(rep); free(kids); free(cnt); free(sc); free(ssel); free(bc); free(sel);
    return keff;
}

/* ---------- batched drivers (OpenMP over queries) ---------- */

/* Queries are q[S][T][H][d], w[S][T][H], qpos[S][T]; K row j of sequence s at
 * K + s*k_seq_stride + j*d.  sel (nullable): list of nsel flat query ids
 * (s*T + i) to evaluate; null = all S*T.  Outputs are indexed by flat id.
 * Returns 0, or -1 on a bad position or allocation failure. */
/*
 * Block-sparse baseline (the comparison the pages make: HISA is said to beat
 * block-sparse selection -- arXiv abstract; gptget.net English summary, "Key
 * Results"; Chinese summary, experiment design).  The pages do not define it;
 * the reading here: with the same token budget k, keep the floor(k/B) best
 * blocks by the same block score as HISA's first stage (representatives and
 * ranking as in oracle_hisa_query), and select every token j <= t of those
 * blocks.  out_idx [k]: the tokens in increasing order, then -1.  Returns the
 * number of tokens, or -1 (k < B, or out of memory).
 */
int oracle_block_sparse_query(const uint16_t *q, const float *w, const uint16_t *K, int H, int d,
                              int64_t t, int B, int k, int32_t *out_idx, int32_t *out_blk)
{
    int mb = k / B;              /* whole blocks that fit the budget */
    if (mb < 1) return -1;
    int64_t bt = t / B;
    int64_t nb = bt + 1;
    uint16_t *rep = (uint16_t *)malloc((size_t)d * sizeof *rep);
    cand_t *bc = (cand_t *)malloc((size_t)nb * sizeof *bc);
    int32_t *sel = (int32_t *)malloc((size_t)mb * sizeof *sel);
    if (!rep || !bc || !sel) {
        free(rep); free(bc); free(sel);
        return -1;
    }
    for (int64_t b = 0; b < nb; ++b) {
        int64_t r1 = (b < bt) ? (b + 1) * B : t + 1;
        oracle_mean_rows(K, b * B, r1, d, rep);
        bc[b].s = oracle_score(q, w, rep, H, d);
        bc[b].i = b;
    }
    qsort(bc, (size_t)nb, sizeof *bc, by_score_then_index);
    int keep = nb < mb ? (int)nb : mb;
    for (int i = 0; i < keep; ++i) sel[i] = (int32_t)bc[i].i;
    qsort(sel, (size_t)keep, sizeof *sel, by_index);
    int n = 0;
    for (int i = 0; i < keep; ++i) {
        for (int64_t j = (int64_t)sel[i] * B; j < (int64_t)(sel[i] + 1) * B && j <= t; ++j)
            out_idx[n++] = (int32_t)j;
    }
    for (int i = n; i < k; ++i) out_idx[i] = -1;
    if (out_blk)
        for (int i = 0; i < mb; ++i) out_blk[i] = i < keep ? sel[i] : -1;
    free(rep); free(bc); free(sel);
    return n;
}

int oracle_hisa_batch_mode(const uint16_t *q, const float *w, const int32_t *qpos,
                           const uint16_t *K, int64_t k_seq_stride, int64_t L, int S, int T, int H,
                           int d, int B, int m, int k, int mode, const int32_t *sel, int nsel,
                           int32_t *out_idx, float *out_score, int32_t *out_blk)
{
    int n = sel ? nsel : S * T;
    int64_t nfull = L / B;       /* blocks complete within the cache */
    uint16_t *means = (uint16_t *)malloc((size_t)S * (nfull > 0 ? nfull : 1) * d * sizeof *means);
    if (!means) return -1;
    for (int s = 0; s < S; ++s) {
        const uint16_t *Ks = K + (size_t)s * k_seq_stride;
#pragma omp parallel for schedule(static)
        for (int64_t b = 0; b < nfull; ++b)
            rep_rows(Ks, b * B, (b + 1) * B, d, mode, means + ((size_t)s * nfull + b) * d);
    }
    int bad = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(|| : bad)
    for (int e = 0; e < n; ++e) {
        int id = sel ? sel[e] : e;
        int s = id / T;
        int64_t t = qpos[id];
        if (t < 0 || t >= L) { bad = 1; continue; }
        int r = oracle_hisa_query_mode(q + (size_t)id * H * d, w + (size_t)id * H,
                                       K + (size_t)s * k_seq_stride, means + (size_t)s * nfull * d,
                                       H, d, t, B, m, k, mode, out_idx + (size_t)id * k,
                                       out_score ? out_score + (size_t)id * k : NULL,
                                       out_blk + (size_t)id * m, NULL);
        if (r < 0) bad = 1;
    }
    free(means);
    return bad ? -1 : 0;
}

int oracle_hisa_batch(const uint16_t *q, const float *w, const int32_t *qpos, const uint16_t *K,
                      int64_t k_seq_stride, int64_t L, int S, int T, int H, int d, int B, int m,
                      int k, const int32_t *sel, int nsel, int32_t *out_idx, float *out_score,
                      int32_t *out_blk)
{
    return oracle_hisa_batch_mode(q, w, qpos, K, k_seq_stride, L, S, T, H, d, B, m, k, 0, sel, nsel,
                                  out_idx, out_score, out_blk);
}

int oracle_flat_batch(const uint16_t *q, const float *w, const int32_t *qpos, const uint16_t *K,
                      int64_t k_seq_stride, int64_t L, int S, int T, int H, int d, int k,
                      const int32_t *sel, int nsel, int32_t *out_idx, float *out_score)
{
    int n = sel ? nsel : S * T;
    int bad = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(|| : bad)
    for (int e = 0; e < n; ++e) {
        int id = sel ? sel[e] : e;
        int s = id / T;
        int64_t t = qpos[id];
        if (t < 0 || t >= L) { bad = 1; continue; }
        int r = oracle_flat_query(q + (size_t)id * H * d, w + (size_t)id * H,
                                  K + (size_t)s * k_seq_stride, H, d, t, k,
                                  out_idx + (size_t)id * k,
                                  out_score ? out_score + (size_t)id * k : NULL, NULL);
        if (r < 0) bad = 1;
    }
    return bad ? -1 : 0;
}

int oracle_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
