// The HISA indexing path with the block stage fused into one kernel.
//
// The pages' procedure (gptget.net English summary, "Methodology"; Chinese
// summary, method details): score the mean-pooled block representatives with
// the original indexer, keep the top m blocks, re-score every token of the kept
// blocks with the original indexer, keep the top k tokens.
//
// K1 hisa_blocks_topm_kernel -- one workgroup (8 waves) per query:
//    * stages q in LDS and the rows of the query's own block b_t = t / B
//      (rows b_t*B .. t); the own-block representative is their mean,
//      bf16(fp32(fp64 sum in row order / count)), the same arithmetic as the
//      block pool, so the pool entry of the own block is never read;
//    * scores the pooled means of the complete blocks b < b_t and the own
//      representative with the shared MFMA scorer;
//    * keeps the top min(m, b_t + 1) blocks (ascending ids): one wave selects
//      when b_t + 1 <= 2048 (no barriers), the whole workgroup otherwise.
// K2 hisa_refine_kernel -- one workgroup (4 waves) per 128 candidate positions
//    of a query (position p = slot*B + r: row r of the slot-th kept block,
//    masked past t): scores its rows with q staged in LDS and writes their keys.
// The final top k runs as the selection kernel (select.hip).  Limits (checked
// by the host): B*d <= 16384, ceil(L/B) <= 8192.

#include "hisa_internal.h"
#include "scorer.h"
#include "select_core.h"

namespace hisa {
namespace {

constexpr int kK1Threads = 512;
constexpr int kK1R = kFusedMaxBlocks / kK1Threads;        // block keys per thread, block-wide select
constexpr int kK1WaveMax = 64 * 32;                       // rows the one-wave select takes
constexpr int kK2Threads = 256;

// LDS slot of block position p: the keys are stored so that the select's
// owner of a contiguous run of positions reads it as conflict-free rows.
__device__ __forceinline__ int k1_slot(int p, int nb) {
    if (nb <= kK1WaveMax) {
        const int rd = (nb + 63) / 64;                        // positions per lane
        return (p % rd) * 64 + p / rd;
    }
    return (p % kK1R) * kK1Threads + p / kK1R;
}

template <int R>
__device__ __forceinline__ void k1_wave_select(const uint32_t *s_keys, int nb, int m, uint32_t *hist,
                                               int32_t *sel, int32_t *ob, uint32_t &keff_out) {
    const int lane = threadIdx.x & 63;
    const int rd = (nb + 63) / 64;
    uint32_t kv[R];
#pragma unroll
    for (int r = 0; r < R; ++r) kv[r] = (r < rd && lane * rd + r < nb) ? s_keys[r * 64 + lane] : kNoCandidate;
    const SelectResult res = wave_radix_select<R>(kv, static_cast<uint32_t>(m), hist);
    if (res.keff > 0)
        wave_compact<R>(kv, res, [&](uint32_t op, int r, uint32_t) {
            const int pos = lane * rd + r;
            sel[op] = pos;
            if (ob) ob[op] = pos;
        });
    keff_out = res.keff;
}

template <int MT, int KS>
__global__ __launch_bounds__(kK1Threads) void hisa_blocks_topm_kernel(FusedArgs a) {
    constexpr int D = 32 * KS;
    constexpr int QST = QStage<KS>::kStride;
    constexpr int kOwnWords = kFusedOwnElems / 2 > kWaveHistWords ? kFusedOwnElems / 2 : kWaveHistWords;
    __shared__ __attribute__((aligned(16))) uint16_t s_q[64 * QST];
    // own-block rows; after the mean they hold the one-wave select's histograms
    __shared__ __attribute__((aligned(16))) uint32_t s_own_raw[kOwnWords];
    __shared__ __attribute__((aligned(16))) uint16_t s_mean[128];
    __shared__ __attribute__((aligned(16))) uint32_t s_keys[kFusedMaxBlocks];   // by k1_slot()
    __shared__ __attribute__((aligned(16))) SelectScratch sc;
    __shared__ uint32_t s_keff;
    uint16_t *s_own = reinterpret_cast<uint16_t *>(s_own_raw);

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int n = lane & 15, g = lane >> 4;
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
    const int64_t bt = t / a.B;
    const int nb = static_cast<int>(bt + 1);
    const int64_t r0 = bt * a.B;
    const int own_rows = static_cast<int>(t + 1 - r0);
    const uint16_t *Ks = a.K + s * a.k_seq_stride;

    // own-block rows (contiguous in the cache) and the query into LDS
    {
        const int chunks = own_rows * D / 8;
        const u32x4 *src = reinterpret_cast<const u32x4 *>(Ks + r0 * D);
        u32x4 *dst = reinterpret_cast<u32x4 *>(s_own);
        for (int c = tid; c < chunks; c += kK1Threads) dst[c] = src[c];
    }
    stage_query<MT, KS>(a.q + static_cast<int64_t>(qi) * a.H * D, a.H, s_q, tid, kK1Threads);
    __syncthreads();

    QFrag<MT, KS> f;
    load_qfrag_lds<MT, KS>(f, s_q, a.w + static_cast<int64_t>(qi) * a.H, a.H, lane);

    // own-block representative: the last D threads (whole waves), one column
    // each, rows in order, fp64; the other waves score complete blocks meanwhile
    constexpr int kWaves1 = kK1Threads / 64;
    constexpr int kScoreWaves = kWaves1 - D / 64;
    const int mean_tid = tid - kScoreWaves * 64;
    if (mean_tid >= 0) {
        double sum = 0.0;
        int r = 0;
        for (; r + 32 <= own_rows; r += 32) {          // 32 LDS reads in flight per batch
            float x[32];
#pragma unroll
            for (int j = 0; j < 32; ++j) x[j] = bf16_to_f32(s_own[(r + j) * D + mean_tid]);
#pragma unroll
            for (int j = 0; j < 32; ++j) sum += static_cast<double>(x[j]);
        }
        for (; r < own_rows; ++r) sum += static_cast<double>(bf16_to_f32(s_own[r * D + mean_tid]));
        s_mean[mean_tid] = f32_to_bf16_rne(static_cast<float>(sum / static_cast<double>(own_rows)));
    } else {
        // complete blocks b < b_t from the pool, 16 per tile; each wave issues
        // the loads of up to four tiles before scoring them
        const uint16_t *pool = a.pool + s * a.pool_seq_stride;
        const int full = static_cast<int>(bt);
        const int ntiles = (full + 15) / 16;
        for (int base = wave; base < ntiles; base += 4 * kScoreWaves) {
            bf16x8 kb[4][KS];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int p = (base + u * kScoreWaves) * 16 + n;
                load_row_frag<KS>(kb[u], p < full ? pool + static_cast<int64_t>(p) * D : nullptr, lane);
            }
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int tile = base + u * kScoreWaves;
                if (tile < ntiles) {
                    const int p = tile * 16 + n;
                    const float v = score_rows<MT, KS>(f, kb[u]);
                    if (g == 0 && p < full) s_keys[k1_slot(p, nb)] = score_to_key(v);
                }
            }
        }
    }
    __syncthreads();
    if (wave == 0) {
        bf16x8 kb[KS];
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) kb[ks] = n == 0 ? load_bf16x8(s_mean + 32 * ks + 8 * g) : zero_bf16x8();
        const float v = score_rows<MT, KS>(f, kb);
        if (lane == 0) s_keys[k1_slot(nb - 1, nb)] = score_to_key(v);
    }
    __syncthreads();

    uint32_t keff;
    if (nb <= kK1WaveMax) {
        // short rows: one wave, no barriers
        if (wave == 0) {
            const int rd = (nb + 63) / 64;
            uint32_t ke;
            if (rd <= 4) k1_wave_select<4>(s_keys, nb, a.m, s_own_raw, sel, ob, ke);
            else if (rd <= 8) k1_wave_select<8>(s_keys, nb, a.m, s_own_raw, sel, ob, ke);
            else if (rd <= 16) k1_wave_select<16>(s_keys, nb, a.m, s_own_raw, sel, ob, ke);
            else k1_wave_select<32>(s_keys, nb, a.m, s_own_raw, sel, ob, ke);
            if (lane == 0) s_keff = ke;
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
        const uint16_t *row = nullptr;
        if (p < npos) {
            const int slot = p / a.B;
            const int64_t tok = static_cast<int64_t>(selq[slot]) * a.B + (p - slot * a.B);
            if (tok <= t) row = a.K + s * a.k_seq_stride + tok * D;
        }
        valid[nt] = row != nullptr;
        load_row_frag<KS>(kb[nt], row, lane);
    }
    stage_query<MT, KS>(a.q + static_cast<int64_t>(qi) * a.H * D, a.H, s_q, tid, kK2Threads);
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

template <int MT>
hipError_t launch_fused_mt(const FusedArgs &a, hipStream_t st) {
    const int nq = a.S * a.T;
    const dim3 g2(static_cast<uint32_t>((static_cast<int64_t>(a.m) * a.B + 127) / 128), nq);
    hipError_t e;
    if (a.d == 64) {
        e = launch(kKindScoreBlocks, hisa_blocks_topm_kernel<MT, 2>, dim3(nq), dim3(kK1Threads), 0, st, a);
        if (e != hipSuccess) return e;
        return launch(kKindScoreRefine, hisa_refine_kernel<MT, 2>, g2, dim3(kK2Threads), 0, st, a);
    }
    e = launch(kKindScoreBlocks, hisa_blocks_topm_kernel<MT, 4>, dim3(nq), dim3(kK1Threads), 0, st, a);
    if (e != hipSuccess) return e;
    return launch(kKindScoreRefine, hisa_refine_kernel<MT, 4>, g2, dim3(kK2Threads), 0, st, a);
}

}  // namespace

bool fused_supported(int d, int64_t L, int B, int m) {
    (void)m;
    return static_cast<int64_t>(B) * d <= kFusedOwnElems && (L + B - 1) / B <= kFusedMaxBlocks;
}

hipError_t launch_fused_blocks_refine(const FusedArgs &a, hipStream_t st) {
    if (a.H <= 16) return launch_fused_mt<1>(a, st);
    if (a.H <= 32) return launch_fused_mt<2>(a, st);
    return launch_fused_mt<4>(a, st);
}

}  // namespace hisa
