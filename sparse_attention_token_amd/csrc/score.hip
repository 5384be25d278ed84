// The indexer scorer on the matrix cores.
//
// For one query (H heads of dimension d) and a tile of 128 rows x_j, computes
//     s_j = sum_h w_h * ReLU(q_h . x_j)
// the DSA lightweight-indexer score that the pages' "original indexer" applies
// both to block representatives (coarse stage) and to tokens (refinement);
// arXiv abstract and gptget.net English summary, "Methodology".
//
// The contraction q_h . x_j over d is a dense [H x d] x [d x 128] product per
// tile, done with v_mfma_f32_16x16x32_bf16 (bf16 inputs, fp32 accumulate):
//   A = q      (M = heads, 16 per M-tile, zero-padded past H)
//   B = rows   (N = 16 rows per N-tile)
//   K = d      (32 per k-step)
// Lane l = 16*g + n supplies A[head 16*mt + n][8 consecutive d] and
// B[8 consecutive d][row n] for the same 8 d values, so the pairing of the
// contraction index is consistent whatever order the unit sums its slots in.
// The fp32 result D[head][row] comes back as 4 heads (4g..4g+3) of row n per
// lane; the epilogue applies ReLU and w in fp32 and sums the heads: first the
// 4*MT values held by the lane, then across the four lane groups g with two
// xor-shuffles.  The same instruction sequence runs for every mode, so a given
// (query, row) gets the same fp32 bits from the block stage, the refinement
// and the flat indexer.
//
// Work split: one workgroup = 4 waves = one 128-row tile of one query; each
// wave owns two N-tiles (32 rows).  Every lane loads its own 16-byte slices of
// q and of its rows straight into registers; the row loads are issued first.
// The 16-row scoring step is score_rows() of scorer.h, shared with the fused
// HISA kernels.
//
// Rows by mode (tile position p, query position t, own block b_t = t / B):
//   blocks: p = block id <= b_t; row = pool mean p for p < b_t, and the
//           query's own-block mean (rows b_t*B .. t, recomputed from K) for p = b_t
//   refine: p = slot*B + r over the kept blocks (ascending); row = key
//           sel[slot]*B + r if that token is <= t, else no candidate
//   flat:   p = token id <= t; row = key p
// Output is an order-preserving uint32 key per position (0 = no candidate).

#include "hisa_internal.h"
#include "scorer.h"

namespace hisa {
namespace {

constexpr int kTileRows = 128;
constexpr int kWaves = 4;
constexpr int kRowsPerWave = kTileRows / kWaves;   // 32 = two N-tiles
constexpr int kNT = kRowsPerWave / 16;

template <int MODE, int MT, int KS>
__global__ __launch_bounds__(256) void score_kernel(ScoreArgs a) {
    constexpr int D = 32 * KS;
    const int qi = blockIdx.y;
    const int s = qi / a.T;
    const int i = qi - s * a.T;
    const int64_t t = query_pos(a.qpos, qi, i, a.L, a.T);
    if (t < 0) return;
    const int64_t bt = t / a.B;
    int64_t npos;
    if (MODE == kScoreBlocks) {
        npos = bt + 1;
    } else if (MODE == kScoreRefine) {
        const int64_t meff = (a.m < bt + 1) ? a.m : bt + 1;
        npos = meff * a.B;
    } else {
        npos = t + 1;
    }
    const int64_t tile0 = static_cast<int64_t>(blockIdx.x) * kTileRows;
    if (tile0 >= npos) return;

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int n = lane & 15;
    const int g = lane >> 4;

    // ---- rows of this lane (issued first: they come from HBM)
    bf16x8 kb[kNT][KS];
    bool valid[kNT];
    int64_t pos[kNT];
#pragma unroll
    for (int nt = 0; nt < kNT; ++nt) {
        const int64_t p = tile0 + wave * kRowsPerWave + nt * 16 + n;
        pos[nt] = p;
        const uint16_t *row = nullptr;
        if (p < npos) {
            if (MODE == kScoreBlocks) {
                row = p == bt ? a.own_rep + static_cast<int64_t>(qi) * D
                              : a.pool + s * a.pool_seq_stride + p * D;
            } else if (MODE == kScoreRefine) {
                const int64_t slot = p / a.B;
                const int64_t r = p - slot * a.B;
                const int64_t tok = static_cast<int64_t>(a.sel_blk[static_cast<int64_t>(qi) * a.m + slot]) * a.B + r;
                if (tok <= t) row = a.K + s * a.k_seq_stride + tok * D;
            } else {
                row = a.K + s * a.k_seq_stride + p * D;
            }
        }
        valid[nt] = row != nullptr;
        load_row_frag<KS>(kb[nt], row, lane);
    }

    QFrag<MT, KS> f;
    load_qfrag_global<MT, KS>(f, a.q + static_cast<int64_t>(qi) * a.H * D,
                              a.w + static_cast<int64_t>(qi) * a.H, a.H, lane);
#pragma unroll
    for (int nt = 0; nt < kNT; ++nt) {
        const float v = score_rows<MT, KS>(f, kb[nt]);
        if (g == 0 && pos[nt] < npos)
            a.keys[static_cast<int64_t>(qi) * a.keys_stride + pos[nt]] =
                valid[nt] ? score_to_key(v) : kNoCandidate;
    }
}

template <int MODE, int MT>
hipError_t launch_mt(KernelKind kind, const ScoreArgs &a, dim3 grid, hipStream_t st) {
    if (a.d == 64) return launch(kind, score_kernel<MODE, MT, 2>, grid, dim3(256), 0, st, a);
    return launch(kind, score_kernel<MODE, MT, 4>, grid, dim3(256), 0, st, a);
}

template <int MODE>
hipError_t launch_mode(KernelKind kind, const ScoreArgs &a, dim3 grid, hipStream_t st) {
    if (a.H <= 16) return launch_mt<MODE, 1>(kind, a, grid, st);
    if (a.H <= 32) return launch_mt<MODE, 2>(kind, a, grid, st);
    return launch_mt<MODE, 4>(kind, a, grid, st);
}

}  // namespace

hipError_t launch_score(ScoreMode mode, const ScoreArgs &a, int64_t max_pos, hipStream_t st) {
    const dim3 grid(static_cast<uint32_t>((max_pos + kTileRows - 1) / kTileRows),
                    static_cast<uint32_t>(a.S * a.T));
    const KernelKind kind = mode == kScoreBlocks ? kKindScoreBlocks
                          : mode == kScoreRefine ? kKindScoreRefine : kKindScoreFlat;
    if (mode == kScoreBlocks) return launch_mode<kScoreBlocks>(kind, a, grid, st);
    if (mode == kScoreRefine) return launch_mode<kScoreRefine>(kind, a, grid, st);
    return launch_mode<kScoreFlat>(kind, a, grid, st);
}

}  // namespace hisa
