// Block representatives: mean (or max) pooling of contiguous key blocks.
//
// Mean pooling of contiguous blocks of B keys is how the pages build the
// coarse-stage block representatives (gptget.net English summary,
// "Methodology"; Chinese summary, method details).  The representative is
// bf16 so that the block stage feeds the same bf16 matrix-core scorer as the
// token stage; it is rounded once from the exact-order fp64 sum:
//     mean = bf16_RNE( fp32_RNE( (sum over rows, increasing row, in fp64) / count ) ).
// Max pooling, the alternative one page names for the coarse summaries ("Hierarchical
// Indexing Makes Sparse Attention Actually Fast", section on the hierarchical
// summarization of the KV cache), takes per column the largest key value,
// the earliest row among equal values (+0 and -0), with no rounding at all.
//
// Blocks of up to 128 rows: one thread per column loads its column into
// registers and adds it in row order (pool_append_direct_kernel).  Longer runs
// (B = 256, and a query's own block in the general path): all 256 threads
// first copy the rows into LDS with 16-byte loads (every load in flight at
// once), then one thread per column adds its column from LDS in row order.  The sequential fp64 order is what makes the result
// independent of how the rows were appended.

#include "block_rep.h"
#include "hisa_internal.h"

namespace hisa {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kPoolThreads = 256;
constexpr int kMaxRows = 256;                       // largest supported B
constexpr int kMaxD = 128;

// Running representative of one column, rows added in row order: the fp64
// sum (mean) or the largest value so far, the earliest kept on equal values.
template <bool MAX>
struct ColumnRep {
    double sum = 0.0;
    float bestf = -__builtin_huge_valf();
    uint16_t best = 0;
    __device__ __forceinline__ void add(uint16_t h) {
        const float x = bf16_to_f32(h);
        if (MAX) {
            if (x > bestf) {
                bestf = x;
                best = h;
            }
        } else {
            sum += static_cast<double>(x);
        }
    }
    // representative of the n rows added so far
    __device__ __forceinline__ uint16_t get(int64_t n) const {
        return MAX ? best : f32_to_bf16_rne(static_cast<float>(sum / static_cast<double>(n)));
    }
};

// Running summary of one column of a tree super-block over its child blocks,
// added in block order, each child's representative h covering cnt keys: the
// count-weighted fp64 sum (mean over the super-block's tokens; cnt * x is
// exact, so a fused multiply-add rounds exactly as the product then the sum),
// or the largest value so far, the earliest kept on equal values.
template <bool MAX>
struct SuperRep {
    double sum = 0.0;
    int64_t total = 0;
    float bestf = -__builtin_huge_valf();
    uint16_t best = 0;
    __device__ __forceinline__ void add(uint16_t h, int64_t cnt) {
        const float x = bf16_to_f32(h);
        if (MAX) {
            if (x > bestf) {
                bestf = x;
                best = h;
            }
        } else {
            sum += static_cast<double>(x) * static_cast<double>(cnt);
            total += cnt;
        }
    }
    __device__ __forceinline__ uint16_t get() const {
        return MAX ? best : f32_to_bf16_rne(static_cast<float>(sum / static_cast<double>(total)));
    }
};

// Copy rows [0, rows) of `src` (row stride d elements) into LDS and return the
// bf16 representative of column threadIdx.x (threads >= d return 0 and write nothing).
template <bool MAX>
__device__ __forceinline__ uint16_t staged_column_rep(const uint16_t *__restrict__ src,
                                                      int rows, int d, uint16_t *lds) {
    constexpr int kMaxChunks = kMaxRows * kMaxD / 8 / kPoolThreads;   // 16-byte chunks per thread
    const int chunks_per_row = d / 8;
    const int total = rows * chunks_per_row;
    u32x4 v[kMaxChunks];
#pragma unroll
    for (int it = 0; it < kMaxChunks; ++it) {          // all loads in flight before any store
        const int c = threadIdx.x + it * kPoolThreads;
        if (c < total) {
            const int r = c / chunks_per_row;
            v[it] = *reinterpret_cast<const u32x4 *>(src + static_cast<int64_t>(r) * d + 8 * (c - r * chunks_per_row));
        }
    }
#pragma unroll
    for (int it = 0; it < kMaxChunks; ++it) {
        const int c = threadIdx.x + it * kPoolThreads;
        if (c < total) {
            const int r = c / chunks_per_row;
            *reinterpret_cast<u32x4 *>(lds + r * d + 8 * (c - r * chunks_per_row)) = v[it];
        }
    }
    __syncthreads();
    const int col = threadIdx.x;
    if (col >= d) return 0;
    ColumnRep<MAX> acc;
    int r = 0;
    for (; r + 8 <= rows; r += 8) {                    // 8 LDS reads in flight, added in row order
        uint16_t x[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) x[j] = lds[(r + j) * d + col];
#pragma unroll
        for (int j = 0; j < 8; ++j) acc.add(x[j]);
    }
    for (; r < rows; ++r) acc.add(lds[r * d + col]);
    return acc.get(rows);
}

// Blocks of at most kDirectRows rows: one thread per column loads its whole
// column straight into registers, then adds it in row order -- no LDS stage
// and no barrier.  The loads are buffer loads whose row offset is a uniform
// scalar (rows past the end re-read the last row and are not added), so all
// of them issue back to back with no per-load address arithmetic; each row's
// loads across the threads form one coalesced read.
constexpr int kDirectRows = 128;

template <bool MAX>
__global__ __launch_bounds__(kMaxD) void pool_append_direct_kernel(
        const uint16_t *__restrict__ K, int64_t k_seq_stride, int d, int B, int64_t blk0,
        int64_t L_new, uint16_t *__restrict__ pool, int64_t pool_seq_stride) {
    const int s = blockIdx.y;
    const int col = threadIdx.x;
    if (col >= d) return;
    const int64_t b = blk0 + blockIdx.x;
    const int64_t r0 = b * B;
    const int rows = static_cast<int>(((r0 + B < L_new) ? r0 + B : L_new) - r0);
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<uint16_t *>(K + s * k_seq_stride + r0 * d), static_cast<short>(0),
            rows * d * 2, 0x00020000);
    uint16_t x[kDirectRows];
#pragma unroll
    for (int r = 0; r < kDirectRows; ++r)
        x[r] = __builtin_amdgcn_raw_buffer_load_b16(rs, 2 * col, (r < rows ? r : rows - 1) * d * 2, 0);
    ColumnRep<MAX> acc;
#pragma unroll
    for (int r = 0; r < kDirectRows; ++r)
        if (r < rows) acc.add(x[r]);
    pool[s * pool_seq_stride + b * d + col] = acc.get(rows);
}

// Blocks of at most kFusedOwnElems keys' worth of rows (B*d <= 16384): one
// 512-thread workgroup per block, every thread summing a run of rows of two
// columns straight from global memory (OwnRowsPar: exact fp64 part sums whose
// total is the row-order sum whenever a column's exponents span at most 37
// binades, the row-order sum itself otherwise), so a block costs a few
// dozen dependent additions per thread instead of B.  A step's append
// touches few blocks, so their latency is the append's time (a prefill chunk
// of 4096 rows: 32 blocks).
constexpr int kParThreads = 512;

template <int D, bool MAX>
__global__ __launch_bounds__(kParThreads) void pool_append_par_kernel(
        const uint16_t *__restrict__ K, int64_t k_seq_stride, int B, int64_t blk0, int64_t L_new,
        uint16_t *__restrict__ pool, int64_t pool_seq_stride) {
    using Own = OwnRowsPar<D, kParThreads>;
    __shared__ __attribute__((aligned(16))) typename Own::Scratch sc;
    const int s = blockIdx.y;
    const int tid = threadIdx.x;
    const int64_t b = blk0 + blockIdx.x;
    const int64_t r0 = b * B;
    const int rows = static_cast<int>(((r0 + B < L_new) ? r0 + B : L_new) - r0);
    const uint16_t *src = K + s * k_seq_stride + r0 * D;
    Own own;
    own.load(src, rows, tid);
    own.template partial<MAX>(rows, tid, sc);
    __syncthreads();
    if (tid < D) own.template combine<MAX>(src, rows, tid, sc, nullptr, pool + s * pool_seq_stride + b * D);
}

// grid: (S).  tree_append_one_kernel's work with block b's mean spread over
// all kParThreads threads (OwnRowsPar: the bits of the row-order mean) for
// B*D <= kFusedOwnElems; threads c < D then pool the super-block column c as
// that kernel does, the first round of children loaded with the block's rows.
// At 4 sequences of 1M keys: 8.6 us with one thread per column (two
// dependent memory round trips after a long load queue per thread), 4.8 us
// spread.
template <int D, bool MAX>
__global__ __launch_bounds__(kParThreads) void tree_append_par_kernel(
        const uint16_t *__restrict__ K, int64_t k_seq_stride, int B, int G, int64_t b, int64_t L_new,
        uint16_t *__restrict__ pool, int64_t pool_seq_stride, uint16_t *__restrict__ spool,
        int64_t spool_seq_stride) {
    using Own = OwnRowsPar<D, kParThreads>;
    __shared__ __attribute__((aligned(16))) typename Own::Scratch sc;
    __shared__ uint16_t s_rep[D];
    constexpr int kChildRound = 64;
    const int s = blockIdx.x;
    const int tid = threadIdx.x;
    const int64_t r0 = b * B;
    const int rows = static_cast<int>(((r0 + B < L_new) ? r0 + B : L_new) - r0);
    const uint16_t *src = K + s * k_seq_stride + r0 * D;
    Own own;
    own.load(src, rows, tid);
    // the complete children b0 .. b-1 of column c = tid (threads c < D, whole
    // waves), the first round in flight with the rows; reads past the last
    // child re-read child b0 and are not added
    const int64_t b0 = b / G * G;
    const int nchild = static_cast<int>(b - b0);
    const uint16_t *pcol = pool + s * pool_seq_stride + b0 * D + (tid & (D - 1));
    uint16_t y[kChildRound];
    if (tid < D) {
#pragma unroll
        for (int j = 0; j < kChildRound; ++j) y[j] = pcol[(j < nchild ? j : 0) * D];
    }
    own.template partial<MAX>(rows, tid, sc);
    __syncthreads();
    if (tid < D) {
        SuperRep<MAX> sup;
#pragma unroll
        for (int j = 0; j < kChildRound; ++j)
            if (j < nchild) sup.add(y[j], B);
        for (int c0 = kChildRound; c0 < nchild; c0 += kChildRound) {
#pragma unroll
            for (int j = 0; j < kChildRound; ++j) y[j] = pcol[(c0 + j < nchild ? c0 + j : 0) * D];
#pragma unroll
            for (int j = 0; j < kChildRound; ++j)
                if (c0 + j < nchild) sup.add(y[j], B);
        }
        own.template combine<MAX>(src, rows, tid, sc, s_rep, pool + s * pool_seq_stride + b * D);
        sup.add(s_rep[tid], rows);                      // written by this thread
        spool[s * spool_seq_stride + (b / G) * D + tid] = sup.get();
    }
}

// grid: (S).  Both levels of the three-level tree when the new rows all lie
// in block b (B <= kDirectRows, b the cache's last block): block b is
// recomputed as in pool_append_direct_kernel, then its super-block u = b / G,
// whose children are the blocks u*G .. b, from their pool entries in order
// (B keys each) with block b's new representative last (its row count).
template <bool MAX>
__global__ __launch_bounds__(kMaxD) void tree_append_one_kernel(
        const uint16_t *__restrict__ K, int64_t k_seq_stride, int d, int B, int G, int64_t b, int64_t L_new,
        uint16_t *__restrict__ pool, int64_t pool_seq_stride, uint16_t *__restrict__ spool,
        int64_t spool_seq_stride) {
    const int s = blockIdx.x;
    const int col = threadIdx.x;
    if (col >= d) return;
    const int64_t r0 = b * B;
    const int rows = static_cast<int>(((r0 + B < L_new) ? r0 + B : L_new) - r0);
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<uint16_t *>(K + s * k_seq_stride + r0 * d), static_cast<short>(0),
            rows * d * 2, 0x00020000);
    uint16_t x[kDirectRows];
#pragma unroll
    for (int r = 0; r < kDirectRows; ++r)
        x[r] = __builtin_amdgcn_raw_buffer_load_b16(rs, 2 * col, (r < rows ? r : rows - 1) * d * 2, 0);
    // the complete children b0 .. b-1, kChildRound loads in flight per round
    // (the first round's issued with the block's rows); a round may re-read
    // child b0 past the last one, and such reads are not added
    constexpr int kChildRound = 64;
    const int64_t b0 = b / G * G;
    const int nchild = static_cast<int>(b - b0);
    const uint16_t *pcol = pool + s * pool_seq_stride + b0 * d + col;
    SuperRep<MAX> sup;
    for (int c0 = 0; c0 < nchild; c0 += kChildRound) {
        uint16_t y[kChildRound];
#pragma unroll
        for (int j = 0; j < kChildRound; ++j) y[j] = pcol[(c0 + j < nchild ? c0 + j : 0) * d];
#pragma unroll
        for (int j = 0; j < kChildRound; ++j)
            if (c0 + j < nchild) sup.add(y[j], B);
    }
    ColumnRep<MAX> acc;
#pragma unroll
    for (int r = 0; r < kDirectRows; ++r)
        if (r < rows) acc.add(x[r]);
    const uint16_t rep = acc.get(rows);
    pool[s * pool_seq_stride + b * d + col] = rep;
    sup.add(rep, rows);
    spool[s * spool_seq_stride + (b / G) * d + col] = sup.get();
}

// grid: (nsb, S), d threads.  Super-blocks [sb0, sb0 + nsb) of the three-level
// tree from the block pool of a cache holding L_new rows: super-block u pools
// its blocks u*G .. min(u*G + G, nblk) - 1 in order, each weighted by its key
// count (B, and L_new - b*B for a short last block).
template <bool MAX>
__global__ __launch_bounds__(kMaxD) void super_append_kernel(
        const uint16_t *__restrict__ pool, int64_t pool_seq_stride, int d, int B, int G, int64_t sb0, int64_t L_new,
        uint16_t *__restrict__ spool, int64_t spool_seq_stride) {
    const int s = blockIdx.y;
    const int col = threadIdx.x;
    if (col >= d) return;
    const int64_t u = sb0 + blockIdx.x;
    const int64_t nblk = (L_new + B - 1) / B;
    const int64_t b0 = u * G;
    const int64_t b1 = (b0 + G < nblk) ? b0 + G : nblk;
    const uint16_t *pcol = pool + s * pool_seq_stride + col;
    SuperRep<MAX> sup;
    constexpr int kRound = 16;                          // loads in flight, added in block order
    for (int64_t c0 = b0; c0 < b1; c0 += kRound) {
        uint16_t y[kRound];
#pragma unroll
        for (int j = 0; j < kRound; ++j) y[j] = pcol[(c0 + j < b1 ? c0 + j : b0) * d];
#pragma unroll
        for (int j = 0; j < kRound; ++j) {
            const int64_t b = c0 + j;
            if (b < b1) sup.add(y[j], (b + 1) * B <= L_new ? B : L_new - b * B);
        }
    }
    spool[s * spool_seq_stride + u * d + col] = sup.get();
}

// grid: (nblk, S).  Recomputes blocks [blk0, blk0 + nblk) over rows < L_new.
template <bool MAX>
__global__ __launch_bounds__(kPoolThreads) void pool_append_kernel(
        const uint16_t *__restrict__ K, int64_t k_seq_stride, int d, int B, int64_t blk0,
        int64_t L_new, uint16_t *__restrict__ pool, int64_t pool_seq_stride) {
    __shared__ __attribute__((aligned(16))) uint16_t lds[kMaxRows * kMaxD];
    const int s = blockIdx.y;
    const int64_t b = blk0 + blockIdx.x;
    const int64_t r0 = b * B;
    const int rows = static_cast<int>(((r0 + B < L_new) ? r0 + B : L_new) - r0);
    const uint16_t m = staged_column_rep<MAX>(K + s * k_seq_stride + r0 * d, rows, d, lds);
    if (static_cast<int>(threadIdx.x) < d) pool[s * pool_seq_stride + b * d + threadIdx.x] = m;
}

// grid: (S*T).  Writes the representative of the query's own block
// b_t = floor(t/B) -- over rows [b_t*B, t] -- to own_rep[qi].
template <bool MAX>
__global__ __launch_bounds__(kPoolThreads) void own_mean_kernel(
        const uint16_t *__restrict__ K, int64_t k_seq_stride, const int32_t *__restrict__ qpos,
        int64_t L, int T, int d, int B, uint16_t *__restrict__ own_rep) {
    __shared__ __attribute__((aligned(16))) uint16_t lds[kMaxRows * kMaxD];
    const int qi = blockIdx.x;
    const int s = qi / T;
    const int i = qi - s * T;
    const int64_t t = query_pos(qpos, qi, i, L, T);
    if (t < 0) return;
    const int64_t r0 = (t / B) * B;
    const uint16_t m = staged_column_rep<MAX>(K + s * k_seq_stride + r0 * d,
                                              static_cast<int>(t + 1 - r0), d, lds);
    if (static_cast<int>(threadIdx.x) < d) own_rep[static_cast<int64_t>(qi) * d + threadIdx.x] = m;
}

// grid: (blocks b_lo .. b_lo + gridDim.x - 1, S, kPrefixSegments),
// kPrefixThreads threads.  Consecutive query positions t = L - T + i: the
// own-block representative of the query at t is the running fp64 sum (or
// running maximum) down its block's rows in row order, taken at row t -- the
// same arithmetic as staged_column_rep().  The block's rows are split into
// kPrefixSegments runs of outputs, one workgroup each; the workgroup stages
// the block's rows up to its run's end in LDS, and thread (g, c) takes column
// c and outputs g*per .. g*per + per - 1 of the run: it sums the column from
// the block's first row in row order, then writes a representative after each
// of its own rows.  The prefix before a thread's outputs is summed again by
// every thread that needs it (at most B additions from LDS), which costs less
// than the divisions of a whole run done one after another by a single thread
// per column: 16 us for a 4096-query chunk that way.
constexpr int kPrefixSegments = 4;
constexpr int kPrefixThreads = 1024;

template <bool MAX>
__global__ __launch_bounds__(kPrefixThreads) void own_prefix_mean_kernel(
        const uint16_t *__restrict__ K, int64_t k_seq_stride, int64_t L, int T, int d, int B,
        int64_t b_lo, uint16_t *__restrict__ own_rep) {
    __shared__ __attribute__((aligned(16))) uint16_t lds[kMaxRows * kMaxD];
    const int s = blockIdx.y;
    const int tid = threadIdx.x;
    const int64_t t0 = L - T;                                  // position of query 0
    const int64_t r0 = (b_lo + blockIdx.x) * B;
    const int seg = B / kPrefixSegments;
    const int64_t out_lo = r0 + static_cast<int64_t>(blockIdx.z) * seg;
    const int64_t blk_end = (r0 + B < L) ? r0 + B : L;
    const int64_t r_end = (out_lo + seg < blk_end) ? out_lo + seg : blk_end;   // rows summed: r0 .. r_end-1
    const int64_t r_first = out_lo > t0 ? out_lo : t0;         // first row written
    if (r_first >= r_end) return;                              // whole workgroup
    // stage rows r0 .. r_end-1 (16-byte chunks; d is a multiple of 8)
    const int rows = static_cast<int>(r_end - r0);
    const int cpr = d / 8;
    const u32x4 *src = reinterpret_cast<const u32x4 *>(K + s * k_seq_stride + r0 * d);
    for (int c = tid; c < rows * cpr; c += kPrefixThreads)
        *reinterpret_cast<u32x4 *>(lds + 8 * c) = src[c];
    __syncthreads();
    const int groups = kPrefixThreads / d;                     // 8 (d = 128) or 16 (d = 64)
    const int col = tid % d, g = tid / d;
    const int per = (seg + groups - 1) / groups;
    const int64_t o_lo = out_lo + static_cast<int64_t>(g) * per;
    const int64_t o_hi = (o_lo + per < r_end) ? o_lo + per : r_end;
    if (o_lo >= o_hi) return;
    ColumnRep<MAX> acc;
    const int pre = static_cast<int>(o_lo - r0);               // rows before this thread's outputs
    int r = 0;
    for (; r + 8 <= pre; r += 8) {                             // 8 LDS reads in flight, added in row order
        uint16_t x[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) x[j] = lds[(r + j) * d + col];
#pragma unroll
        for (int j = 0; j < 8; ++j) acc.add(x[j]);
    }
    for (; r < pre; ++r) acc.add(lds[r * d + col]);
    for (int64_t o = o_lo; o < o_hi; ++o) {
        acc.add(lds[(o - r0) * d + col]);
        if (o >= r_first) own_rep[(static_cast<int64_t>(s) * T + (o - t0)) * d + col] = acc.get(o + 1 - r0);
    }
}

// grid: (S*T), d threads.  Own super-block representative of the three-level
// tree: a super-block pools the representatives of its G blocks in block
// order, each weighted by its key count, and the one holding t covers its
// blocks up to b_t: the complete ones (B keys each), then the query's
// own-block representative own_rep[qi] (t + 1 - b_t*B keys).
template <bool MAX>
__global__ __launch_bounds__(kMaxD) void own_super_kernel(
        const uint16_t *__restrict__ pool, int64_t pool_seq_stride, const uint16_t *__restrict__ own_rep,
        const int32_t *__restrict__ qpos, int64_t L, int T, int d, int B, int G,
        uint16_t *__restrict__ own_srep) {
    const int qi = blockIdx.x;
    const int s = qi / T;
    const int64_t t = query_pos(qpos, qi, qi - s * T, L, T);
    const int col = threadIdx.x;
    if (t < 0 || col >= d) return;
    const int64_t bt = t / B;
    const int64_t b0 = bt / G * G;
    const uint16_t *src = pool + s * pool_seq_stride + col;
    SuperRep<MAX> acc;
    int64_t b = b0;
    for (; b + 8 <= bt; b += 8) {                      // 8 loads in flight, added in block order
        uint16_t x[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) x[j] = src[(b + j) * d];
#pragma unroll
        for (int j = 0; j < 8; ++j) acc.add(x[j], B);
    }
    for (; b < bt; ++b) acc.add(src[b * d], B);
    acc.add(own_rep[static_cast<int64_t>(qi) * d + col], t + 1 - bt * B);
    own_srep[static_cast<int64_t>(qi) * d + col] = acc.get();
}

}  // namespace

hipError_t launch_own_super(const uint16_t *pool, int64_t pool_seq_stride, const uint16_t *own_rep,
                            const int32_t *qpos, int64_t L, int S, int T, int d, int B, int G, bool pool_max,
                            uint16_t *own_srep, hipStream_t st) {
    if (pool_max)
        return launch(kKindOwnSuper, own_super_kernel<true>, dim3(S * T), dim3(kMaxD), 0, st, pool, pool_seq_stride,
                      own_rep, qpos, L, T, d, B, G, own_srep);
    return launch(kKindOwnSuper, own_super_kernel<false>, dim3(S * T), dim3(kMaxD), 0, st, pool, pool_seq_stride,
                  own_rep, qpos, L, T, d, B, G, own_srep);
}

hipError_t launch_own_prefix_mean(const uint16_t *K, int64_t k_seq_stride, int64_t L, int S, int T, int d, int B,
                                  bool pool_max, uint16_t *own_rep, hipStream_t st) {
    const int64_t b_lo = (L - T) / B, b_hi = (L - 1) / B;
    const dim3 g(static_cast<uint32_t>(b_hi - b_lo + 1), S, kPrefixSegments);
    if (pool_max)
        return launch(kKindOwnMean, own_prefix_mean_kernel<true>, g, dim3(kPrefixThreads), 0, st, K, k_seq_stride, L,
                      T, d, B, b_lo, own_rep);
    return launch(kKindOwnMean, own_prefix_mean_kernel<false>, g, dim3(kPrefixThreads), 0, st, K, k_seq_stride, L, T,
                  d, B, b_lo, own_rep);
}

hipError_t launch_pool_append(const uint16_t *K, int64_t k_seq_stride, int S, int d, int B,
                              int64_t blk0, int64_t nblk, int64_t L_new, bool pool_max, uint16_t *pool,
                              int64_t pool_seq_stride, hipStream_t st) {
    const dim3 g(static_cast<uint32_t>(nblk), S);
    if (static_cast<int64_t>(B) * d <= kFusedOwnElems) {
        if (d == 64)
            return pool_max ? launch(kKindPoolAppend, pool_append_par_kernel<64, true>, g, dim3(kParThreads), 0, st,
                                     K, k_seq_stride, B, blk0, L_new, pool, pool_seq_stride)
                            : launch(kKindPoolAppend, pool_append_par_kernel<64, false>, g, dim3(kParThreads), 0, st,
                                     K, k_seq_stride, B, blk0, L_new, pool, pool_seq_stride);
        return pool_max ? launch(kKindPoolAppend, pool_append_par_kernel<128, true>, g, dim3(kParThreads), 0, st, K,
                                 k_seq_stride, B, blk0, L_new, pool, pool_seq_stride)
                        : launch(kKindPoolAppend, pool_append_par_kernel<128, false>, g, dim3(kParThreads), 0, st, K,
                                 k_seq_stride, B, blk0, L_new, pool, pool_seq_stride);
    }
    if (B <= kDirectRows) {
        if (pool_max)
            return launch(kKindPoolAppend, pool_append_direct_kernel<true>, g, dim3(kMaxD), 0, st, K, k_seq_stride,
                          d, B, blk0, L_new, pool, pool_seq_stride);
        return launch(kKindPoolAppend, pool_append_direct_kernel<false>, g, dim3(kMaxD), 0, st, K, k_seq_stride, d,
                      B, blk0, L_new, pool, pool_seq_stride);
    }
    if (pool_max)
        return launch(kKindPoolAppend, pool_append_kernel<true>, g, dim3(kPoolThreads), 0, st, K, k_seq_stride, d,
                      B, blk0, L_new, pool, pool_seq_stride);
    return launch(kKindPoolAppend, pool_append_kernel<false>, g, dim3(kPoolThreads), 0, st, K, k_seq_stride, d, B,
                  blk0, L_new, pool, pool_seq_stride);
}

hipError_t launch_super_append(const uint16_t *pool, int64_t pool_seq_stride, int S, int d, int B, int G,
                               int64_t sb0, int64_t nsb, int64_t L_new, bool pool_max, uint16_t *spool,
                               int64_t spool_seq_stride, hipStream_t st) {
    const dim3 g(static_cast<uint32_t>(nsb), S);
    if (pool_max)
        return launch(kKindPoolAppend, super_append_kernel<true>, g, dim3(kMaxD), 0, st, pool, pool_seq_stride, d, B,
                      G, sb0, L_new, spool, spool_seq_stride);
    return launch(kKindPoolAppend, super_append_kernel<false>, g, dim3(kMaxD), 0, st, pool, pool_seq_stride, d, B, G,
                  sb0, L_new, spool, spool_seq_stride);
}

bool tree_append_one_supported(int B) { return B <= kDirectRows; }

hipError_t launch_tree_append_one(const uint16_t *K, int64_t k_seq_stride, int S, int d, int B, int G, int64_t blk,
                                  int64_t L_new, bool pool_max, uint16_t *pool, int64_t pool_seq_stride,
                                  uint16_t *spool, int64_t spool_seq_stride, hipStream_t st) {
    if ((d == 64 || d == 128) && static_cast<int64_t>(B) * d <= kFusedOwnElems) {
        const dim3 g(S), blk_(kParThreads);
        if (d == 64)
            return pool_max ? launch(kKindPoolAppend, tree_append_par_kernel<64, true>, g, blk_, 0, st, K, k_seq_stride,
                                     B, G, blk, L_new, pool, pool_seq_stride, spool, spool_seq_stride)
                            : launch(kKindPoolAppend, tree_append_par_kernel<64, false>, g, blk_, 0, st, K,
                                     k_seq_stride, B, G, blk, L_new, pool, pool_seq_stride, spool, spool_seq_stride);
        return pool_max ? launch(kKindPoolAppend, tree_append_par_kernel<128, true>, g, blk_, 0, st, K, k_seq_stride, B,
                                 G, blk, L_new, pool, pool_seq_stride, spool, spool_seq_stride)
                        : launch(kKindPoolAppend, tree_append_par_kernel<128, false>, g, blk_, 0, st, K, k_seq_stride,
                                 B, G, blk, L_new, pool, pool_seq_stride, spool, spool_seq_stride);
    }
    if (pool_max)
        return launch(kKindPoolAppend, tree_append_one_kernel<true>, dim3(S), dim3(kMaxD), 0, st, K, k_seq_stride, d,
                      B, G, blk, L_new, pool, pool_seq_stride, spool, spool_seq_stride);
    return launch(kKindPoolAppend, tree_append_one_kernel<false>, dim3(S), dim3(kMaxD), 0, st, K, k_seq_stride, d, B,
                  G, blk, L_new, pool, pool_seq_stride, spool, spool_seq_stride);
}

hipError_t launch_own_mean(const uint16_t *K, int64_t k_seq_stride, const int32_t *qpos,
                           int64_t L, int S, int T, int d, int B, bool pool_max, uint16_t *own_rep,
                           hipStream_t st) {
    if (pool_max)
        return launch(kKindOwnMean, own_mean_kernel<true>, dim3(S * T), dim3(kPoolThreads), 0, st, K, k_seq_stride,
                      qpos, L, T, d, B, own_rep);
    return launch(kKindOwnMean, own_mean_kernel<false>, dim3(S * T), dim3(kPoolThreads), 0, st, K, k_seq_stride,
                  qpos, L, T, d, B, own_rep);
}

}  // namespace hisa
