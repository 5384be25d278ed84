// The block stage and the token refinement for many queries per sequence
// (prefill chunks), block by block.
//
// The refinement step re-scores, with the original indexer, every token of the
// blocks each query kept (gptget.net English summary, "Methodology"; Chinese
// summary, method details).  Done query by query, every (query, kept block)
// pair gathers the block's B key rows again: with thousands of queries over
// the same cache the key rows are fetched from the memory fabric once per pair.
// Here the pairs are grouped by block instead, per chunk of up to
// kChunkQueries consecutive queries of one sequence:
//
//   hisa_blocks_bm_kernel / hisa_topm_kernel: the block stage the same way --
//                        256 pooled means per workgroup in registers, the
//                        chunk's queries streamed through LDS -- then one wave
//                        per query scores its own block's representative
//                        (own_mean_kernel) and keeps the top m.
//   hisa_bucket_kernel   one workgroup per chunk: counting sort of the chunk's
//                        (query, slot) pairs by kept block id, in LDS.
//   hisa_refine_bm_kernel one 2-wave workgroup per (block, chunk) (bm_tile()): the block's
//                        B rows stay in registers as MFMA operands (each wave
//                        owns B/2 rows), and the queries that kept the block
//                        stream through an LDS stage filled by direct
//                        buffer-to-LDS loads; eight such workgroups per CU
//                        cover each other's load latency.
//
// Each (query, row) score comes from score_tiles_lds(), whose per-tile
// arithmetic is that of score_rows() in every other kernel, so the results are
// bit-identical to the query-major refinement's; candidate position p = slot*B + r of query qi gets the key of
// row r of its slot-th kept block, or "no candidate" past the query position.

#include "hisa_internal.h"
#include "scorer.h"
#include "select_core.h"

namespace hisa {
namespace {

constexpr int kBucketThreads = 1024;
constexpr int kBucketR = kFusedMaxBlocks / kBucketThreads;   // bins per thread in the scan
constexpr int kBucketU = 16;                                 // kept-block entries per thread in flight
constexpr int kBMThreads = 128;                              // two waves

// ALL: the flat indexer's form -- every query takes every block b <= b_t, in
// slot b (a.m = nblk slots per query), instead of its kept blocks.
template <bool ALL>
__global__ __launch_bounds__(kBucketThreads) void hisa_bucket_kernel(FusedArgs a) {
    __shared__ uint32_t s_cnt[kFusedMaxBlocks];
    __shared__ uint32_t s_wave[kBucketThreads / 64];
    __shared__ int32_t s_bt[kChunkQueries];
    // a chunk of at most kBucketU * kBucketThreads pairs (the kept blocks of
    // 256 queries with m <= 64) is sorted in one pass: its block ids stay in
    // registers, and the sorted pairs are gathered in LDS and stored in order
    // (stored where they fall they took 16 scattered stores per thread)
    constexpr int kStagePairs = ALL ? 1 : kBucketU * kBucketThreads;
    __shared__ uint32_t s_stage[kStagePairs];
    __shared__ uint32_t s_total;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int c = blockIdx.x;
    const int cps = (a.T + kChunkQueries - 1) / kChunkQueries;
    const int s = c / cps;
    const int i0 = (c - s * cps) * kChunkQueries;
    const int nqc = min(kChunkQueries, a.T - i0);
    const int nblk = a.nblk;
    const int32_t *sel = ALL ? nullptr : a.sel_blk + (static_cast<int64_t>(s) * a.T + i0) * a.m;
    const int n = nqc * a.m;

    for (int b = tid; b < nblk; b += kBucketThreads) s_cnt[b] = 0u;
    if (ALL)
        for (int i = tid; i < nqc; i += kBucketThreads) {
            const int64_t t = query_pos(a.qpos, s * a.T + i0 + i, i0 + i, a.L, a.T);
            s_bt[i] = t < 0 ? -1 : static_cast<int32_t>(t / a.B);
        }
    __syncthreads();
    // slot e of the chunk: the kept block sel[e], or with ALL block e % m of
    // query e / m while it is <= that query's own block
    auto block_of = [&](int e) -> int {
        if (!ALL) return sel[e];
        const int ql = e / a.m, j = e - ql * a.m;
        return j <= s_bt[ql] ? j : -1;
    };
    // the chunk's kept blocks, kBucketU per thread at a time with every load
    // issued before the first atomic (a load per iteration would serialise
    // n / kBucketThreads memory round trips)
    const bool one_pass = !ALL && n <= kStagePairs;
    int bb1[kBucketU];                            // one_pass: the chunk's block ids, kept for the fill
#pragma unroll
    for (int u = 0; u < kBucketU; ++u) bb1[u] = -1;
    for (int e0 = 0; e0 < n; e0 += kBucketU * kBucketThreads) {
        int bb[kBucketU];
#pragma unroll
        for (int u = 0; u < kBucketU; ++u) {
            const int e = e0 + u * kBucketThreads + tid;
            bb[u] = e < n ? block_of(e) : -1;
        }
#pragma unroll
        for (int u = 0; u < kBucketU; ++u) {
            if (bb[u] >= 0) atomicAdd(&s_cnt[bb[u]], 1u);
            bb1[u] = bb[u];
        }
    }
    __syncthreads();

    // exclusive scan of the bins: thread t owns bins [t*R, t*R + R)
    uint32_t v[kBucketR];
    uint32_t sum = 0;
#pragma unroll
    for (int r = 0; r < kBucketR; ++r) {
        const int b = tid * kBucketR + r;
        v[r] = b < nblk ? s_cnt[b] : 0u;
        sum += v[r];
    }
    const uint32_t incl = wave_prefix_incl(sum);
    if (lane == 63) s_wave[wave] = incl;
    __syncthreads();
    uint32_t run = incl - sum;
    for (int w = 0; w < wave; ++w) run += s_wave[w];
    int32_t *off = a.bucket_off + static_cast<int64_t>(c) * (nblk + 1);
#pragma unroll
    for (int r = 0; r < kBucketR; ++r) {
        const int b = tid * kBucketR + r;
        if (b < nblk) {
            off[b] = static_cast<int32_t>(run);
            s_cnt[b] = run;              // becomes the fill cursor
        }
        run += v[r];
    }
    if (tid == kBucketThreads - 1) {
        off[nblk] = static_cast<int32_t>(run);
        s_total = run;                            // the pair count
    }
    __syncthreads();

    uint32_t *ent = a.bucket_ent + static_cast<int64_t>(c) * kChunkQueries * a.m;
    if (one_pass) {
        const uint32_t total = s_total;
#pragma unroll
        for (int u = 0; u < kBucketU; ++u) {
            if (bb1[u] >= 0) {
                const int e = u * kBucketThreads + tid;
                const uint32_t pos = atomicAdd(&s_cnt[bb1[u]], 1u);
                const int ql = e / a.m;
                s_stage[pos] = (static_cast<uint32_t>(ql) << 16) | static_cast<uint32_t>(e - ql * a.m);
            }
        }
        __syncthreads();
        for (uint32_t i = tid; i < total; i += kBucketThreads) ent[i] = s_stage[i];
        return;
    }
    for (int e0 = 0; e0 < n; e0 += kBucketU * kBucketThreads) {
        int bb[kBucketU];
#pragma unroll
        for (int u = 0; u < kBucketU; ++u) {
            const int e = e0 + u * kBucketThreads + tid;
            bb[u] = e < n ? block_of(e) : -1;
        }
#pragma unroll
        for (int u = 0; u < kBucketU; ++u) {
            if (bb[u] >= 0) {
                const int e = e0 + u * kBucketThreads + tid;
                const uint32_t pos = atomicAdd(&s_cnt[bb[u]], 1u);
                const int ql = e / a.m;
                ent[pos] = (static_cast<uint32_t>(ql) << 16) | static_cast<uint32_t>(e - ql * a.m);
            }
        }
    }
}

// The direct global-to-LDS loads, behind plain device functions: named
// directly inside a kernel template, the target builtins keep the host pass
// from emitting some of the template's launch stubs.  Buffer form: the base
// address and size live in scalar registers (a buffer resource), each lane
// adds its own byte offset, and M0 holds the LDS destination of lane 0.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), static_cast<short>(0), static_cast<int>(bytes),
                                             0x00020000);
}
__device__ __forceinline__ void lds_load_b128(__amdgpu_buffer_rsrc_t r, uint32_t voff, void *lds) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, reinterpret_cast<__attribute__((address_space(3))) void *>(
                                                    reinterpret_cast<uintptr_t>(lds)),
                                             16, voff, 0, 0, 0);
}
__device__ __forceinline__ void lds_load_b32(__amdgpu_buffer_rsrc_t r, uint32_t voff, void *lds) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, reinterpret_cast<__attribute__((address_space(3))) void *>(
                                                    reinterpret_cast<uintptr_t>(lds)),
                                             4, voff, 0, 0, 0);
}

// Direct-to-LDS staging of one query (q and w) into the swizzled layout of
// QSwz that score_tiles_lds() reads.  One 16-byte buffer load to LDS fills 64
// consecutive 16-byte slots, one per lane; lane p's slot is slot p % CPR of
// head row p / CPR, so the lane loads the chunk that the swizzle places
// there.  Lanes of rows past H write nothing: those rows are zeroed once.
template <int MT, int KS, int NW>
struct QDirect {
    using L = QSwz<KS>;
    static constexpr int D = L::D, CPR = L::CPR;
    static constexpr int kSlots = MT * 16 * CPR;
    static constexpr int kInstr = kSlots / 64;
    static constexpr int kPerWave = (kInstr + NW - 1) / NW;   // wave w takes instructions w, w+NW, ...
    static_assert(kSlots % 64 == 0, "every wave issues whole loads");
    int src[kPerWave];                                        // byte offset in q, or -1: no load

    __device__ __forceinline__ void init(int H, int wave, int lane) {
#pragma unroll
        for (int u = 0; u < kPerWave; ++u) {
            const int p = 64 * (wave + u * NW) + lane;
            const int row = p / CPR, slot = p - row * CPR;
            src[u] = wave + u * NW < kInstr && row < H ? 2 * (row * D + 8 * (slot ^ L::swz(row))) : -1;
        }
    }
    __device__ __forceinline__ void issue(const uint16_t *__restrict__ q, const float *__restrict__ w, int H,
                                          uint16_t *s_q, float *s_w, int wave, int lane) const {
        const __amdgpu_buffer_rsrc_t rq = make_rsrc(q, static_cast<uint32_t>(H * D * 2));
#pragma unroll
        for (int u = 0; u < kPerWave; ++u)
            if (src[u] >= 0) lds_load_b128(rq, static_cast<uint32_t>(src[u]), s_q + 8 * 64 * (wave + u * NW));
        const __amdgpu_buffer_rsrc_t rw = make_rsrc(w, static_cast<uint32_t>(H * 4));
        if (wave == NW - 1 && lane < H) lds_load_b32(rw, 4u * lane, s_w);
    }
};

// Workgroup -> (block b, chunk c).  With at least 8 chunks, chunk c runs on
// XCD c % 8 (workgroups are dealt to the 8 XCDs in turn): every workgroup of
// an XCD then works on the same chunk, whose queries stay in that XCD's L2
// while the key blocks stream through.  c = -1: nothing to do.
__device__ __forceinline__ void bm_tile(int nblk, int nchunk, int &b, int &c) {
    const int i = blockIdx.x;
    if (nchunk >= 8) {
        const int x = i & 7, r = i >> 3;
        const int cc = r / nblk;
        b = r - cc * nblk;
        c = cc * 8 + x;
        if (c >= nchunk) c = -1;
    } else {
        c = i / nblk;
        b = i - c * nblk;
    }
}

inline uint32_t bm_grid(int nblk, int64_t nchunk) {
    return static_cast<uint32_t>(nchunk >= 8 ? (nchunk + 7) / 8 * 8 * nblk : nchunk * nblk);
}

// Candidate keys of one query for this wave's NTW tiles: every lane of a row's
// column group holds that row's score, so lane (n, g) stores tiles g, g+4, ...
// -- one store per lane per four tiles.  "No candidate" past the query
// position t.
template <int NTW>
__device__ __forceinline__ void store_tiles(uint32_t *cand, const float (&v)[NTW], int tok0, int t, int lane) {
    const int n = lane & 15, g = lane >> 4;
#pragma unroll
    for (int nt0 = 0; nt0 < NTW; nt0 += 4) {
        if (nt0 + g < NTW) {
            // two-level select on the bits of g (kept as selects, not an indexed load)
            const float a0 = v[nt0];
            const float a1 = nt0 + 1 < NTW ? v[nt0 + 1] : a0;
            const float a2 = nt0 + 2 < NTW ? v[nt0 + 2] : a0;
            const float a3 = nt0 + 3 < NTW ? v[nt0 + 3] : a0;
            const float lo = (g & 1) ? a1 : a0;
            const float hi = (g & 1) ? a3 : a2;
            const float x = (g & 2) ? hi : lo;
            const int r = (nt0 + g) * 16 + n;
            cand[r] = tok0 + r <= t ? score_to_key(x) : kNoCandidate;
        }
    }
}

// Block keys of one query for this wave's NTW tiles of means starting at
// block p0: only blocks p < bt are written (the rest of the row is never read,
// and past the last block it may lie beyond the row).
template <int NTW>
__device__ __forceinline__ void store_blocks(uint32_t *out, const float (&v)[NTW], int p0, int bt, int lane) {
    const int n = lane & 15, g = lane >> 4;
#pragma unroll
    for (int nt0 = 0; nt0 < NTW; nt0 += 4) {
        if (nt0 + g < NTW) {
            const float a0 = v[nt0];
            const float a1 = nt0 + 1 < NTW ? v[nt0 + 1] : a0;
            const float a2 = nt0 + 2 < NTW ? v[nt0 + 2] : a0;
            const float a3 = nt0 + 3 < NTW ? v[nt0 + 3] : a0;
            const float lo = (g & 1) ? a1 : a0;
            const float hi = (g & 1) ? a3 : a2;
            const float x = (g & 2) ? hi : lo;
            const int r = (nt0 + g) * 16 + n;
            if (p0 + r < bt) out[r] = score_to_key(x);
        }
    }
}

// NTW 16-row tiles per wave; the workgroup covers B = 2 * 16 * NTW rows.
template <int MT, int KS, int NTW>
__global__ __launch_bounds__(kBMThreads) void hisa_refine_bm_kernel(FusedArgs a) {
    constexpr int D = 32 * KS;
    constexpr int NW = kBMThreads / 64;
    using QD = QDirect<MT, KS, NW>;
    constexpr int kQElems = QD::kSlots * 8;
    constexpr int kRowsPerWave = 16 * NTW;
    __shared__ __attribute__((aligned(16))) uint16_t s_q[kQElems];
    __shared__ __attribute__((aligned(16))) float s_w[64];
    __shared__ uint32_t s_ent[kChunkQueries];
    __shared__ int32_t s_t[kChunkQueries];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int n = lane & 15;
    const int cps = (a.T + kChunkQueries - 1) / kChunkQueries;
    int b, c;
    bm_tile(a.nblk, a.S * cps, b, c);
    if (c < 0) return;
    const int32_t *off = a.bucket_off + static_cast<int64_t>(c) * (a.nblk + 1);
    const int e0 = off[b];
    const int np = off[b + 1] - e0;
    if (np <= 0) return;
    const int s = c / cps;
    const int i0 = (c - s * cps) * kChunkQueries;
    const int qi0 = s * a.T + i0;

    // this wave's rows of block b (rows past the cache end read the last row
    // and are masked when stored; positions fit in int: L < 2^31)
    const int tok0 = b * a.B + wave * kRowsPerWave;
    bf16x8 kb[NTW][KS];
#pragma unroll
    for (int nt = 0; nt < NTW; ++nt) {
        const int tok = tok0 + nt * 16 + n;
        load_row_frag_any<KS>(kb[nt], a.K + s * a.k_seq_stride + static_cast<int64_t>(tok < a.L ? tok : a.L - 1) * D,
                              lane);
    }
    // the pairs (query, slot) and each query's position
    const uint32_t *ent = a.bucket_ent + static_cast<int64_t>(c) * kChunkQueries * a.m + e0;
    for (int i = tid; i < np; i += kBMThreads) {
        const uint32_t e = ent[i];
        const int ql = static_cast<int>(e >> 16);
        s_ent[i] = e;
        s_t[i] = static_cast<int32_t>(query_pos(a.qpos, qi0 + ql, i0 + ql, a.L, a.T));
    }
    // rows past H read as zero (q) with weight zero
    if (a.H < MT * 16) {
        for (int x = tid; x < (MT * 16 - a.H) * D; x += kBMThreads) s_q[a.H * D + x] = 0;
        if (tid < 64) s_w[tid] = 0.0f;
    }
    __syncthreads();

    QD qd;
    qd.init(a.H, wave, lane);
    // One LDS stage per workgroup: the next query's loads wait until every
    // wave has scored the current one.  The loads' latency is covered by the
    // other workgroups on the CU (the small stage lets eight fit, four waves
    // per SIMD), which measured faster than double-buffering with half as
    // many workgroups per CU (514 against 647 us on a 4096-query chunk).
    // Scores of query i are stored while query i+1 is scored, after the wait,
    // so the wait never covers stores issued just before it.
    float v[NTW];
    uint32_t *cand = nullptr;
    int t = -1;
    for (int i = 0; i < np; ++i) {
        if (i > 0) __syncthreads();          // every wave is done reading the stage
        const int qn = qi0 + static_cast<int>(s_ent[i] >> 16);
        qd.issue(a.q + static_cast<int64_t>(qn) * a.H * D, a.w + static_cast<int64_t>(qn) * a.H, a.H, s_q, s_w,
                 wave, lane);
        __builtin_amdgcn_s_waitcnt(0);       // this query's LDS loads (and older stores) are done
        __syncthreads();                     // ... in every wave
        if (cand) store_tiles<NTW>(cand, v, tok0, t, lane);
        const uint32_t e = s_ent[i];
        const int ql = static_cast<int>(e >> 16);
        const int slot = static_cast<int>(e & 0xffffu);
        t = s_t[i];
        score_tiles_lds<MT, KS, NTW>(s_q, s_w, kb, v, lane);
        cand = a.cand_keys + static_cast<int64_t>(qi0 + ql) * a.cand_stride + slot * a.B + wave * kRowsPerWave;
    }
    store_tiles<NTW>(cand, v, tok0, t, lane);
}

// ---------------------------------------------------------------- block stage, block by block
// Block scores of every query of a chunk (kBlkChunk queries) against 128
// pooled means at once: one 2-wave workgroup per (128-block tile, chunk), the tile's means held in
// registers as MFMA operands and the chunk's queries streamed through LDS as
// in the refinement.  Only complete blocks b < b_t are scored here (the own
// block's representative differs per query; hisa_topm_kernel scores it).
// blk_keys[qi][b] receives the key of block b for b < b_t.
// Four waves of 64 pooled means each: every query staged in LDS serves 256
// means (with two waves and 128 means, each query's 16 KB of q was fetched
// from L2 twice as often for the same matrix-core work).
constexpr int kBlkThreads = 256;
constexpr int kBlkTileRows = 256;
constexpr int kBlkChunk = 16;          // queries per workgroup: enough workgroups to fill the GPU

template <int MT, int KS>
__global__ __launch_bounds__(kBlkThreads) void hisa_blocks_bm_kernel(FusedArgs a) {
    constexpr int D = 32 * KS;
    constexpr int NW = kBlkThreads / 64;
    constexpr int NTW = kBlkTileRows / (16 * NW);
    using QD = QDirect<MT, KS, NW>;
    constexpr int kQElems = QD::kSlots * 8;
    __shared__ __attribute__((aligned(16))) uint16_t s_q[kQElems];
    __shared__ __attribute__((aligned(16))) float s_w[64];
    __shared__ int32_t s_qi[kBlkChunk];
    __shared__ int32_t s_bt[kBlkChunk];
    __shared__ uint32_t s_n;

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int n = lane & 15;
    const int cps = (a.T + kBlkChunk - 1) / kBlkChunk;
    int j, c;
    bm_tile((a.nblk + kBlkTileRows - 1) / kBlkTileRows, a.S * cps, j, c);
    if (c < 0) return;
    const int s = c / cps;
    const int i0 = (c - s * cps) * kBlkChunk;
    const int nqc = min(kBlkChunk, a.T - i0);
    const int b0 = j * kBlkTileRows;

    // the chunk's queries that have a complete block in this tile (b_t > b0)
    if (tid == 0) s_n = 0u;
    __syncthreads();
    for (int i = tid; i < nqc; i += kBlkThreads) {
        const int qi = s * a.T + i0 + i;
        const int64_t t = query_pos(a.qpos, qi, i0 + i, a.L, a.T);
        if (t >= 0 && t / a.B > b0) {
            const uint32_t x = atomicAdd(&s_n, 1u);
            s_qi[x] = qi;
            s_bt[x] = static_cast<int32_t>(t / a.B);
        }
    }
    // this wave's means (rows past the pool end read the first mean and are
    // never stored; the loads are unconditional so none waits for another)
    const uint16_t *pool = a.pool + s * a.pool_seq_stride;
    const int p0 = b0 + wave * 16 * NTW;
    bf16x8 kb[NTW][KS];
#pragma unroll
    for (int nt = 0; nt < NTW; ++nt) {
        const int p = p0 + nt * 16 + n;
        load_row_frag_any<KS>(kb[nt], pool + static_cast<int64_t>(p < a.nblk ? p : 0) * D, lane);
    }
    if (a.H < MT * 16) {
        for (int x = tid; x < (MT * 16 - a.H) * D; x += kBlkThreads) s_q[a.H * D + x] = 0;
        if (tid < 64) s_w[tid] = 0.0f;
    }
    __syncthreads();
    const int np = static_cast<int>(s_n);
    if (np == 0) return;

    // One LDS stage, as in the refinement: a second stage gains nothing here,
    // since every LDS read issued after a direct-to-LDS load waits for it,
    // while it would halve the workgroups that fit on a CU.
    QD qd;
    qd.init(a.H, wave, lane);
    float v[NTW];
    uint32_t *out = nullptr;
    int bt = 0;
    for (int i = 0; i < np; ++i) {
        if (i > 0) __syncthreads();          // every wave is done reading the stage
        const int qn = s_qi[i];
        qd.issue(a.q + static_cast<int64_t>(qn) * a.H * D, a.w + static_cast<int64_t>(qn) * a.H, a.H, s_q, s_w,
                 wave, lane);
        __builtin_amdgcn_s_waitcnt(0);       // this query's LDS loads (and older stores) are done
        __syncthreads();                     // ... in every wave
        if (out) store_blocks<NTW>(out, v, p0, bt, lane);
        out = a.blk_keys + static_cast<int64_t>(qn) * a.blk_stride + p0;
        bt = s_bt[i];
        score_tiles_lds<MT, KS, NTW>(s_q, s_w, kb, v, lane);
    }
    store_blocks<NTW>(out, v, p0, bt, lane);
}

// Per query (one wave each, four per workgroup): score the own block's
// representative own_rep[qi], read the complete blocks' keys, and keep the
// top min(m, b_t + 1) blocks (ascending ids) with the one-wave select.
constexpr int kTopMThreads = 256;

// The block keys of one lane (positions lane*rd .. lane*rd + R - 1), every
// load issued at once before anything waits on them (positions past the
// complete blocks read the row's first key and are masked by topm_select):
// a load under a branch makes the wave wait for it on the spot, and R of them
// in a row were as many serial memory round trips.
template <int R>
__device__ __forceinline__ void topm_load(const uint32_t *keys, int nb, int lane, uint32_t (&kv)[R]) {
    const int rd = (nb + 63) / 64;
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const int p = lane * rd + r;
        kv[r] = keys[(r < rd && p < nb - 1) ? p : 0];
    }
}

template <int R, typename Emit>
__device__ __forceinline__ uint32_t topm_select(uint32_t (&kv)[R], uint32_t own_key, int nb, int m, int lane,
                                                uint32_t *win, Emit &&emit) {
    const int rd = (nb + 63) / 64;
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const int p = lane * rd + r;
        kv[r] = (r < rd && p < nb) ? (p == nb - 1 ? own_key : kv[r]) : kNoCandidate;
    }
    // the ballot select up to 1024 blocks (R <= 16): with sixteen waves per
    // compute unit it measured slightly faster than the LDS histogram of
    // wave_window_select (4096-query chunk, 1008-1024 blocks: 32.8 -> 31.4 us
    // in a same-box A/B); beyond, its rounds grow with R and the window wins
    const SelectResult res = R <= 16 ? wave_ballot_select<R>(kv, static_cast<uint32_t>(m))
                                     : wave_window_select<R>(kv, static_cast<uint32_t>(m), win);
    if (res.keff > 0) wave_compact<R>(kv, res, [&](uint32_t op, int r, uint32_t) { emit(op, lane * rd + r); });
    return res.keff;
}

// The own-block score, then the top m of one query.  The block keys (R per
// lane) are loaded after the score, all at once: loaded together with q the
// keys and the query's fragments were live together, which cost a wave per
// SIMD in occupancy and measured slower.
template <int R, int MT, int KS, typename Emit>
__device__ __forceinline__ uint32_t topm_query(const FusedArgs &a, int qi, int nb, const uint32_t *keys, int lane,
                                               uint32_t *win, Emit &&emit) {
    constexpr int D = 32 * KS;
    QFrag<MT, KS> f;
    load_qfrag_global_any<MT, KS>(f, a.q + static_cast<int64_t>(qi) * a.H * D, a.w + static_cast<int64_t>(qi) * a.H,
                                  a.H, lane);
    bf16x8 kbm[KS];
    // every lane reads the representative; only row 0's score (lane 0) is used
    load_row_frag_any<KS>(kbm, a.own_rep + static_cast<int64_t>(qi) * D, lane);
    const float v = score_rows<MT, KS>(f, kbm);
    const uint32_t own_key = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int>(score_to_key(v))));
    uint32_t kv[R];
    topm_load<R>(keys, nb, lane, kv);
    return topm_select<R>(kv, own_key, nb, a.m, lane, win, emit);
}

// R: block keys per lane, at least ceil(n_b / 64) for every query of the
// launch (one instantiation per R keeps the register budget of the short
// rows' variants small: all four in one kernel took 194 registers).
template <int MT, int KS, int R>
__global__ __launch_bounds__(kTopMThreads) void hisa_topm_kernel(FusedArgs a) {
    __shared__ __attribute__((aligned(16))) uint32_t s_win[kTopMThreads / 64][kWindowWords];
    const int lane = threadIdx.x & 63;
    const int qi = blockIdx.x * (kTopMThreads / 64) + (threadIdx.x >> 6);
    if (qi >= a.S * a.T) return;                       // whole wave
    const int s = qi / a.T;
    const int64_t t = query_pos(a.qpos, qi, qi - s * a.T, a.L, a.T);
    int32_t *sel = a.sel_blk + static_cast<int64_t>(qi) * a.m;
    int32_t *ob = a.out_blk ? a.out_blk + static_cast<int64_t>(qi) * a.m : nullptr;
    uint32_t keff = 0;
    if (t >= 0) {
        const int nb = static_cast<int>(t / a.B + 1);
        const uint32_t *keys = a.blk_keys + static_cast<int64_t>(qi) * a.blk_stride;
        auto emit = [&](uint32_t op, int pos) {
            sel[op] = pos;
            if (ob) ob[op] = pos;
        };
        keff = topm_query<R, MT, KS>(a, qi, nb, keys, lane, s_win[threadIdx.x >> 6], emit);
    }
    for (int j = static_cast<int>(keff) + lane; j < a.m; j += 64) {
        sel[j] = -1;
        if (ob) ob[j] = -1;
    }
}

template <int MT, int KS>
hipError_t launch_topm(const FusedArgs &a, dim3 g_top, hipStream_t st) {
    const int rd = (a.nblk + 63) / 64;                 // n_b <= nblk for every query
    if (rd <= 4) return launch(kKindSelectBlocks, hisa_topm_kernel<MT, KS, 4>, g_top, dim3(kTopMThreads), 0, st, a);
    if (rd <= 8) return launch(kKindSelectBlocks, hisa_topm_kernel<MT, KS, 8>, g_top, dim3(kTopMThreads), 0, st, a);
    if (rd <= 16) return launch(kKindSelectBlocks, hisa_topm_kernel<MT, KS, 16>, g_top, dim3(kTopMThreads), 0, st, a);
    return launch(kKindSelectBlocks, hisa_topm_kernel<MT, KS, 32>, g_top, dim3(kTopMThreads), 0, st, a);
}

template <int MT>
hipError_t launch_blocks_mt(const FusedArgs &a, dim3 g_blk, dim3 g_top, hipStream_t st) {
    hipError_t e;
    if (a.d == 64) {
        e = launch(kKindScoreBlocks, hisa_blocks_bm_kernel<MT, 2>, g_blk, dim3(kBlkThreads), 0, st, a);
        if (e != hipSuccess) return e;
        return launch_topm<MT, 2>(a, g_top, st);
    }
    e = launch(kKindScoreBlocks, hisa_blocks_bm_kernel<MT, 4>, g_blk, dim3(kBlkThreads), 0, st, a);
    if (e != hipSuccess) return e;
    return launch_topm<MT, 4>(a, g_top, st);
}

template <int MT, int KS>
hipError_t launch_bm_ks(const FusedArgs &a, dim3 grid, KernelKind kind, hipStream_t st) {
    if (a.B == 64) return launch(kind, hisa_refine_bm_kernel<MT, KS, 2>, grid, dim3(kBMThreads), 0, st, a);
    return launch(kind, hisa_refine_bm_kernel<MT, KS, 4>, grid, dim3(kBMThreads), 0, st, a);
}

template <int MT>
hipError_t launch_bm_mt(const FusedArgs &a, dim3 grid, hipStream_t st, KernelKind kind = kKindScoreRefine) {
    return a.d == 64 ? launch_bm_ks<MT, 2>(a, grid, kind, st) : launch_bm_ks<MT, 4>(a, grid, kind, st);
}

}  // namespace

bool block_major_mode(int S, int T, int d, int64_t L, int B, int m) {
    (void)S;
    return T >= kChunkQueries / 2 && (B == 64 || B == 128) && m <= 65535 && fused_supported(d, L, B, m);
}

hipError_t launch_block_major_blocks(const FusedArgs &a, hipStream_t st) {
    hipError_t e = a.qpos ? launch_own_mean(a.K, a.k_seq_stride, a.qpos, a.L, a.S, a.T, a.d, a.B, a.pool_max != 0,
                                            a.own_rep, st)
                          : launch_own_prefix_mean(a.K, a.k_seq_stride, a.L, a.S, a.T, a.d, a.B, a.pool_max != 0,
                                                   a.own_rep, st);
    if (e != hipSuccess) return e;
    const int64_t nchunk = static_cast<int64_t>(a.S) * ((a.T + kBlkChunk - 1) / kBlkChunk);
    const dim3 g_blk(bm_grid((a.nblk + kBlkTileRows - 1) / kBlkTileRows, nchunk));
    const int nq = a.S * a.T;
    const dim3 g_top(static_cast<uint32_t>((nq + kTopMThreads / 64 - 1) / (kTopMThreads / 64)));
    if (a.H <= 16) return launch_blocks_mt<1>(a, g_blk, g_top, st);
    if (a.H <= 32) return launch_blocks_mt<2>(a, g_blk, g_top, st);
    return launch_blocks_mt<4>(a, g_blk, g_top, st);
}

hipError_t launch_block_major_refine(const FusedArgs &a, hipStream_t st) {
    const int64_t nchunk = bucket_chunks(a.S, a.T);
    hipError_t e = launch(kKindBucket, hisa_bucket_kernel<false>, dim3(static_cast<uint32_t>(nchunk)),
                          dim3(kBucketThreads), 0, st, a);
    if (e != hipSuccess) return e;
    const dim3 grid(bm_grid(a.nblk, nchunk));
    if (a.H <= 16) return launch_bm_mt<1>(a, grid, st);
    if (a.H <= 32) return launch_bm_mt<2>(a, grid, st);
    return launch_bm_mt<4>(a, grid, st);
}

bool flat_block_major_mode(int S, int T, int d, int64_t L) {
    return block_major_mode(S, T, d, L, kFlatBlock, static_cast<int>((L + kFlatBlock - 1) / kFlatBlock));
}

hipError_t launch_flat_block_major(const FusedArgs &a, hipStream_t st) {
    const int64_t nchunk = bucket_chunks(a.S, a.T);
    hipError_t e = launch(kKindBucketFlat, hisa_bucket_kernel<true>, dim3(static_cast<uint32_t>(nchunk)),
                          dim3(kBucketThreads), 0, st, a);
    if (e != hipSuccess) return e;
    const dim3 grid(bm_grid(a.nblk, nchunk));
    if (a.H <= 16) return launch_bm_mt<1>(a, grid, st, kKindScoreFlat);
    if (a.H <= 32) return launch_bm_mt<2>(a, grid, st, kKindScoreFlat);
    return launch_bm_mt<4>(a, grid, st, kKindScoreFlat);
}

}  // namespace hisa
