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
// Work split (blocks and refine modes, and the general path): one workgroup =
// 4 waves = one 128-row tile of one query; each wave owns two N-tiles (32
// rows).  The flat indexer streams longer runs per workgroup
// (score_flat_kernel).  Every lane loads its own 16-byte slices of
// q and of its rows straight into registers; the row loads are issued first.
// The 16-row scoring step is score_rows() of scorer.h, shared with the fused
// HISA kernels.
//
// Rows by mode (tile position p, query position t, own block b_t = t / B):
//   blocks: p = block id <= b_t; row = pool mean p for p < b_t, and the
//           query's own-block mean (rows b_t*B .. t, recomputed from K) for p = b_t
//   refine: p = slot*B + r over the kept blocks (ascending); row = key
//           sel[slot]*B + r if that slot holds a block and the token is <= t,
//           else no candidate
//   flat:   p = token id <= t; row = key p
//   tree blocks (three-level tree, super-blocks of G blocks): p = slot*G + c
//           over the kept super-blocks u = sel_sb[slot]; block b = u*G + c;
//           row = pool mean b for b < b_t, the own-block mean for b = b_t,
//           no candidate for b > b_t
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
    } else if (MODE == kScoreTreeBlocks) {
        const int64_t ns = bt / a.G + 1;                  // super-blocks visible to the query
        npos = (a.W < ns ? a.W : ns) * a.G;
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
                const int32_t blk = a.sel_blk[static_cast<int64_t>(qi) * a.m + slot];
                const int64_t tok = static_cast<int64_t>(blk) * a.B + r;
                if (blk >= 0 && tok <= t) row = a.K + s * a.k_seq_stride + tok * D;
            } else if (MODE == kScoreTreeBlocks) {
                const int64_t slot = p / a.G;
                const int64_t b = static_cast<int64_t>(a.sel_sb[static_cast<int64_t>(qi) * a.W + slot]) * a.G +
                                  (p - slot * a.G);
                if (b < bt) row = a.pool + s * a.pool_seq_stride + b * D;
                else if (b == bt) row = a.own_rep + static_cast<int64_t>(qi) * D;
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

// Flat indexer: one workgroup streams a run of `rows_per_wg` keys of one
// query (a multiple of 128).  q and w are staged in LDS once and held as
// register fragments; each wave scores two 16-row tiles per 128-row step while
// the next step's rows are already in flight (two register buffers).  The
// per-row arithmetic is score_rows()'s, so the scores equal the other
// kernels' bit for bit.
constexpr int kFlatThreads = 256;

template <int MT, int KS>
__device__ __forceinline__ void flat_load(bf16x8 (&kb)[kNT][KS], const uint16_t *Ks, int64_t base, int64_t npos,
                                          int lane) {
    constexpr int D = 32 * KS;
#pragma unroll
    for (int nt = 0; nt < kNT; ++nt) {
        const int64_t p = base + nt * 16 + (lane & 15);
        load_row_frag<KS>(kb[nt], p < npos ? Ks + p * D : nullptr, lane);
    }
}

template <int MT, int KS>
__device__ __forceinline__ void flat_score_store(const QFrag<MT, KS> &f, const bf16x8 (&kb)[kNT][KS],
                                                 uint32_t *keys, int64_t base, int64_t npos, int lane) {
    float v[kNT];
    score_tiles_frag<MT, KS, kNT>(f, kb, v);
#pragma unroll
    for (int nt = 0; nt < kNT; ++nt) {
        const int64_t p = base + nt * 16 + (lane & 15);
        if ((lane >> 4) == 0 && p < npos) keys[p] = score_to_key(v[nt]);
    }
}

// The leading arguments are what a workgroup needs before its first loads (K
// rows, q, w); this file is built with kernarg preloading, so they arrive in
// scalar registers at dispatch instead of after a memory round trip for the
// argument block.  pk = H | (qpos null) << 8.  EARLY = false (a key stride
// past 2^31 elements): they are ignored and everything comes from a_in.
template <int MT, int KS, bool EARLY>
__global__ __launch_bounds__(kFlatThreads) void score_flat_kernel(const uint16_t *K, const uint16_t *q, const float *w,
                                                                  int32_t k_seq_stride, int32_t Lk, int32_t T,
                                                                  uint32_t pk, int rows_per_wg, ScoreArgs a_in) {
    constexpr int D = 32 * KS;
    __shared__ __attribute__((aligned(16))) uint16_t s_q[64 * QStage<KS>::kStride];
    __shared__ float s_w[64];
    ScoreArgs a = a_in;
    bool qpos_null = a.qpos == nullptr;
    if constexpr (EARLY) {
        a.K = K; a.q = q; a.w = w; a.k_seq_stride = k_seq_stride; a.L = Lk; a.T = T;
        a.H = static_cast<int>(pk & 0xffu);
        qpos_null = ((pk >> 8) & 1u) != 0;
    }
    const int qi = blockIdx.y;
    const int s = qi / a.T;
    int64_t t;
    if (qpos_null) {
        t = a.L - a.T + (qi - s * a.T);
        t = t >= 0 && t < a.L ? t : -1;
    } else {
        t = query_pos(a.qpos, qi, qi - s * a.T, a.L, a.T);
    }
    if (t < 0) return;
    const int64_t npos = t + 1;
    const int64_t row0 = static_cast<int64_t>(blockIdx.x) * rows_per_wg;
    if (row0 >= npos) return;
    const int64_t row1 = row0 + rows_per_wg < npos ? row0 + rows_per_wg : npos;
    const int nsteps = static_cast<int>((row1 - row0 + kTileRows - 1) / kTileRows);
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const uint16_t *Ks = a.K + s * a.k_seq_stride;
    uint32_t *keys = a.keys + static_cast<int64_t>(qi) * a.keys_stride;
    const int64_t wbase = row0 + wave * kRowsPerWave;       // this wave's rows of step 0

    bf16x8 ka[kNT][KS], kc[kNT][KS];
    flat_load<MT, KS>(ka, Ks, wbase, row1, lane);           // first rows in flight before q
    QStager<MT, KS, kFlatThreads> qst;
    qst.load(a.q + static_cast<int64_t>(qi) * a.H * D, a.H, tid);
    const float wq = a.w[static_cast<int64_t>(qi) * a.H + (tid < a.H ? tid : a.H - 1)];   // unconditional load
    pin_loaded(wq);
    qst.store(s_q, a.H, tid);
    if (tid < 64) s_w[tid] = tid < a.H ? wq : 0.0f;
    __syncthreads();
    QFrag<MT, KS> f;
    load_qfrag_lds_w<MT, KS>(f, s_q, s_w, lane);
    for (int st = 0; st < nsteps; st += 2) {
        if (st + 1 < nsteps) flat_load<MT, KS>(kc, Ks, wbase + (st + 1) * kTileRows, row1, lane);
        flat_score_store<MT, KS>(f, ka, keys, wbase + st * kTileRows, row1, lane);
        if (st + 2 < nsteps) flat_load<MT, KS>(ka, Ks, wbase + (st + 2) * kTileRows, row1, lane);
        if (st + 1 < nsteps) flat_score_store<MT, KS>(f, kc, keys, wbase + (st + 1) * kTileRows, row1, lane);
    }
}

template <int MT>
hipError_t launch_flat_mt(const ScoreArgs &a, dim3 grid, int rows_per_wg, hipStream_t st) {
    const bool early = a.k_seq_stride < (int64_t{1} << 31);
    const uint32_t pk = static_cast<uint32_t>(a.H) | (a.qpos == nullptr ? 1u : 0u) << 8;
    auto go = [&](auto kernel) {
        return launch(kKindScoreFlat, kernel, grid, dim3(kFlatThreads), 0, st, a.K, a.q, a.w,
                      early ? static_cast<int32_t>(a.k_seq_stride) : 0, static_cast<int32_t>(a.L), a.T, pk,
                      rows_per_wg, a);
    };
    if (a.d == 64) return early ? go(score_flat_kernel<MT, 2, true>) : go(score_flat_kernel<MT, 2, false>);
    return early ? go(score_flat_kernel<MT, 4, true>) : go(score_flat_kernel<MT, 4, false>);
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
                          : mode == kScoreRefine ? kKindScoreRefine
                          : mode == kScoreTreeBlocks ? kKindScoreTree : kKindScoreFlat;
    if (mode == kScoreBlocks) return launch_mode<kScoreBlocks>(kind, a, grid, st);
    if (mode == kScoreRefine) return launch_mode<kScoreRefine>(kind, a, grid, st);
    if (mode == kScoreTreeBlocks) return launch_mode<kScoreTreeBlocks>(kind, a, grid, st);
    // flat: about 512 workgroups of 128..4096 rows each
    const int64_t nq = static_cast<int64_t>(a.S) * a.T;
    int64_t rows = (max_pos * nq / 512 + kTileRows - 1) / kTileRows * kTileRows;
    rows = rows < kTileRows ? kTileRows : (rows > 4096 ? 4096 : rows);
    const dim3 fgrid(static_cast<uint32_t>((max_pos + rows - 1) / rows), static_cast<uint32_t>(nq));
    const int r = static_cast<int>(rows);
    if (a.H <= 16) return launch_flat_mt<1>(a, fgrid, r, st);
    if (a.H <= 32) return launch_flat_mt<2>(a, fgrid, r, st);
    return launch_flat_mt<4>(a, fgrid, r, st);
}

}  // namespace hisa
