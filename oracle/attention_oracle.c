/*
 * Sparse attention over a selected token set -- CPU ORACLE.
 *
 * TEST INFRASTRUCTURE ONLY (same rules as hisa_oracle.c: only the tests, the
 * smoke check and the benchmark's CPU-baseline leg load it; it shares nothing
 * with the HIP library).
 *
 * What it computes.  The indexer's token set is consumed by the downstream
 * sparse attention, which attends only over the selected keys ([Abstract]:
 * the arXiv abstract, mlsanity.com page; the set is the token-level top-k
 * pattern the Sparse MLA operator takes).  The pages give no formula for that
 * operator.  Reading taken here: ordinary softmax attention restricted to the
 * set, in the decode form of multi-head latent attention, where every token
 * stores one latent row shared by all heads -- its first Dk entries are the
 * key and its first Dv entries (Dv <= Dk) the value:
 *     s_j   = scale * (q_h . kv_j[0..Dk))              for j in the set
 *     o_h   = sum_j exp(s_j) kv_j[0..Dv) / sum_j exp(s_j)
 *     lse_h = ln sum_j exp(s_j)
 * Set entries outside [0, L) (the -1 padding) are skipped; an index listed
 * twice counts twice.  An empty set gives o = 0 and lse = -inf.
 * Also returned: absw_h = sum_j softmax(s)_j |kv_j[0..Dv)|, the weighted mean
 * of the values' magnitudes, from which the tests derive the error bound of
 * a bf16-weighted GPU sum.
 *
 * Arithmetic: fp64 throughout from the exact bf16 inputs; the exponentials
 * are taken relative to the largest score.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#include <omp.h>

static double bf16_value(uint16_t h)
{
    union { uint32_t u; float f; } v;
    v.u = (uint32_t)h << 16;
    return (double)v.f;
}

/* One query: q [Ha][Dk], kv row j at kv + j*row_stride, idx [k].
 * out, absw: [Ha][Dv]; lse: [Ha] (nullable).  Returns 0, or -1 on allocation failure. */
int oracle_sparse_attention(const uint16_t *q, int Ha, int Dk, int Dv, const uint16_t *kv, int64_t row_stride,
                            int64_t L, const int32_t *idx, int k, double scale, double *out, double *lse,
                            double *absw)
{
    double *s = (double *)malloc((size_t)(k > 0 ? k : 1) * sizeof *s);
    if (!s) return -1;
    for (int h = 0; h < Ha; ++h) {
        const uint16_t *qh = q + (size_t)h * Dk;
        double *oh = out + (size_t)h * Dv;
        double *ah = absw + (size_t)h * Dv;
        for (int e = 0; e < Dv; ++e) oh[e] = ah[e] = 0.0;
        /* scores of the listed tokens, and their maximum */
        double smax = -INFINITY;
        for (int i = 0; i < k; ++i) {
            const int64_t j = idx[i];
            if (j < 0 || j >= L) continue;
            const uint16_t *x = kv + j * row_stride;
            double dot = 0.0;
            for (int c = 0; c < Dk; ++c) dot += bf16_value(qh[c]) * bf16_value(x[c]);
            s[i] = scale * dot;
            if (s[i] > smax) smax = s[i];
        }
        if (smax == -INFINITY) {                 /* nothing to attend to */
            if (lse) lse[h] = -INFINITY;
            continue;
        }
        double l = 0.0;
        for (int i = 0; i < k; ++i) {
            const int64_t j = idx[i];
            if (j < 0 || j >= L) continue;
            const double p = exp(s[i] - smax);
            const uint16_t *x = kv + j * row_stride;
            l += p;
            for (int e = 0; e < Dv; ++e) {
                const double v = bf16_value(x[e]);
                oh[e] += p * v;
                ah[e] += p * fabs(v);
            }
        }
        for (int e = 0; e < Dv; ++e) {
            oh[e] /= l;
            ah[e] /= l;
        }
        if (lse) lse[h] = smax + log(l);
    }
    free(s);
    return 0;
}

/* A batch of S*T queries: q [S*T][Ha][Dk], query i of sequence s attends over
 * idx [s*T + i][k] in the cache kv + s*seq_stride.  sel (nullable): the query
 * ids to compute (nsel of them); out/absw [S*T][Ha][Dv], lse [S*T][Ha]. */
int oracle_sparse_attention_batch(const uint16_t *q, int S, int T, int Ha, int Dk, int Dv, const uint16_t *kv,
                                  int64_t seq_stride, int64_t row_stride, int64_t L, const int32_t *idx, int k,
                                  double scale, const int32_t *sel, int nsel, double *out, double *lse, double *absw)
{
    const int n = sel ? nsel : S * T;
    int bad = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(|| : bad)
    for (int i = 0; i < n; ++i) {
        const int qi = sel ? sel[i] : i;
        const int s = qi / T;
        if (oracle_sparse_attention(q + (size_t)qi * Ha * Dk, Ha, Dk, Dv, kv + (size_t)s * seq_stride, row_stride,
                                    L, idx + (size_t)qi * k, k, scale, out + (size_t)qi * Ha * Dv,
                                    lse ? lse + (size_t)qi * Ha : NULL, absw + (size_t)qi * Ha * Dv) != 0)
            bad = 1;
    }
    return bad ? -1 : 0;
}
