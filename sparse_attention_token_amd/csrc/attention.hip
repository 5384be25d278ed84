// Sparse attention over the selected token set, on the matrix cores.
//
// The indexer's token set is consumed by the downstream sparse attention,
// which attends only over the selected keys (arXiv abstract, mlsanity.com
// page).  Here it is softmax attention restricted to the set, in the decode
// form of multi-head latent attention: every token stores one latent row that
// all heads share, its first Dk entries being the key and its first Dv the
// value.  For head h of a query with set I (entries outside [0, L) skipped):
//     s_j = scale * (q_h . kv_j[0..Dk)),   o_h = sum_j softmax(s)_j kv_j[0..Dv),
//     lse_h = ln sum_j exp(s_j).
//
// One workgroup (4 waves) takes one query, a group of HG = 16*HT heads and a
// run of the set, in steps of 64/HT tokens:
//   1. the step's latent rows are gathered into LDS (16-byte loads; rows
//      padded to Dk + 8 elements so 16 consecutive rows start on distinct
//      banks); the next step's rows are loaded into registers while the
//      current step is computed and stored to the second row buffer;
//   2. each wave scores one 16-token tile of the step against one 16-head
//      tile: S^T = K Q^T with v_mfma_f32_16x16x32_bf16 (A = the token rows
//      from LDS, M = tokens; B = q, held in registers for the whole run,
//      N = heads);
//   3. online softmax in the exp2 domain: the step's maximum per head is
//      combined across the waves through LDS, P = exp2(s - m) is rounded to
//      bf16 and written to LDS as P^T [head][token];
//   4. wave w accumulates its quarter of the value columns for every head:
//      O^T += V^T P^T (A = V^T, read with the gfx950 transposing LDS load
//      ds_read_b64_tr_b16 straight from the token-major rows; B = P^T; K = the
//      step's tokens).  O^T keeps one head per lane column, so the per-head
//      rescale of the online softmax is a per-lane scalar.
// The denominator sums the bf16-rounded weights, so the result is an exact
// convex combination of the values with weights within a bf16 rounding of the
// softmax.  When the set is split over several workgroups (few queries), each
// writes its unnormalised partial (O, m, l) and a combine kernel merges them.

#include "hisa_internal.h"
#include "scorer.h"

namespace hisa {
namespace {

constexpr int kAttnThreads = 256;
constexpr int kAttnStep = 64;                 // splits hold whole multiples of this many entries
constexpr float kLn2 = 0.6931471805599453f;

typedef short v4s __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) v4s lds_v4s;

// max over the four 16-lane rows of a wave (lanes n, n+16, n+32, n+48)
__device__ __forceinline__ float rows_max(float x) {
    const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    const float y = fmaxf(__uint_as_float(p[0]), __uint_as_float(p[1]));
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(y), __float_as_uint(y), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __forceinline__ float rows_add(float x) {
    const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    const float y = __uint_as_float(p[0]) + __uint_as_float(p[1]);
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(y), __float_as_uint(y), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// A fragment of V^T for 16 value columns from dv0 and the 8 tokens tok0..tok0+7:
// lane (g, n) gets V[tok0 + e][dv0 + n], e = 0..7.  Within each 16-lane group,
// lane s reads 4 columns dv0 + 4(s%4).. of token tok0 + s/4 (+4 for the second
// read), and the transposing load hands lane n column n of the four tokens.
__device__ __forceinline__ bf16x8 load_vt_frag(const uint16_t *rows, int stride, int tok0, int dv0, int lane) {
    const int s = lane & 15;
    const uint16_t *p0 = rows + (tok0 + (s >> 2)) * stride + dv0 + 4 * (s & 3);
    const u32x2 a = __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s *)(p0)));
    const u32x2 b = __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s *)(p0 + 4 * stride)));
    const u32x4 u = {a.x, a.y, b.x, b.y};
    return as_bf16x8(u);
}

template <int HT, int KSK, int DVW>
struct AttnLds {
    static constexpr int kDk = 32 * KSK;
    static constexpr int kRowStride = kDk + 8;
    static constexpr int kTT = 4 / HT;                  // token tiles per step (one per wave and head tile)
    static constexpr int kStep = 16 * kTT;              // tokens per step: 32 (HT = 2) or 64 (HT = 1)
    static constexpr int kPStride = kStep + 8;
    uint16_t rows[1][kStep * kRowStride];
    uint16_t pt[16 * HT * kPStride];
    float wmax[kTT][16 * HT];
    float wsum[kTT][16 * HT];
    int32_t tok[2][kStep];                              // token of each row of a step, -1 if none
};

// grid: attn_grid(npair, nhg) with npair = S*T*nsplit; workgroup (pair, hg)
// takes query pair / nsplit, heads hg*16*HT.., and set entries
// [split*tps, min(k, split*tps + tps)).  Wave w scores token tile w % kTT of
// each step against head tile w / kTT, and accumulates value columns
// 16*DVW*w .. for every head of the group.  The next step's rows are loaded
// into registers while the current step is computed (every load is issued,
// rows of no candidate re-read the cache's first row and are masked), and its
// set entries one step further ahead.
// The leading arguments are what a workgroup needs before its first loads
// (the set, the latent rows and q): this file is built with kernarg
// preloading, so they arrive in scalar registers at dispatch and the set's
// loads go out without waiting a memory round trip for the argument block.
// pk = Ha | nsplit << 16.  EARLY = false (latent strides past 2^31 elements):
// they are ignored and everything comes from a_in.
template <int HT, int KSK, int DVW, bool EARLY>
__global__ __launch_bounds__(kAttnThreads, HT == 2 ? 2 : 1) void sparse_attn_kernel(
        const int32_t *idx_, const uint16_t *kv_, const uint16_t *q_, int32_t kv_seq_stride, int32_t kv_row_stride,
        int32_t Lk, int32_t k_, int32_t tps, uint32_t pk, int32_t T_, int32_t npair, AttnArgs a_in) {
    AttnArgs a = a_in;
    if constexpr (EARLY) {
        a.idx = idx_; a.kv = kv_; a.q = q_;
        a.kv_seq_stride = kv_seq_stride; a.kv_row_stride = kv_row_stride; a.L = Lk;
        a.k = k_; a.tps = tps; a.T = T_; a.npair = npair;
        a.Ha = static_cast<int>(pk & 0xffffu);
        a.nsplit = static_cast<int>(pk >> 16);
    }
    constexpr int Dk = 32 * KSK;
    constexpr int HG = 16 * HT;
    using Lds = AttnLds<HT, KSK, DVW>;
    constexpr int RS = Lds::kRowStride;
    constexpr int TT = Lds::kTT;
    constexpr int STEP = Lds::kStep;
    constexpr int PS = Lds::kPStride;
    constexpr int KST = STEP / 32;                              // value k-steps per step
    constexpr int CPR = Dk / 8;                                 // 16-byte chunks per row
    constexpr int kPer = (STEP * CPR + kAttnThreads - 1) / kAttnThreads;
    __shared__ __attribute__((aligned(16))) Lds L;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int n = lane & 15, g = lane >> 4;
    const int tt = wave % TT, hw = wave / TT;                  // this wave's token tile and head tile
    // workgroup -> (pair, head group): the head groups of one pair share an XCD
    const int nhg = a.Ha / HG;
    const int bx = blockIdx.x, x = bx & 7, j8 = bx >> 3;
    const int hg = j8 % nhg;
    const int pair = (j8 / nhg) * 8 + x;
    if (pair >= a.npair) return;
    const int qi = pair / a.nsplit;
    const int split = pair - qi * a.nsplit;
    const int s = qi / a.T;
    const int e0 = split * a.tps;
    const int e1 = min(a.k, e0 + a.tps);
    const int nsteps = (e1 - e0 + STEP - 1) / STEP;
    const int32_t *idx = a.idx + static_cast<int64_t>(qi) * a.k;
    const uint16_t *kv = a.kv + s * a.kv_seq_stride;

    auto entry = [&](int e) -> int32_t {                       // the set entry e as a row, or -1
        const int32_t t = e < e1 ? idx[e] : -1;
        return (t >= 0 && t < a.L) ? t : -1;
    };
    // 16-byte chunk of the rows this thread moves in round i: a wave covers 64
    // consecutive chunks, its upper half interleaved with the lower, so the 16
    // lanes one LDS cycle serves (8 from each half) write 64 consecutive dwords
    const int cbase = wave * 64 + (((lane & 31) << 1) | (lane >> 5));
    u32x4 v[kPer];
    auto load_rows = [&](const int32_t *toks) {
#pragma unroll
        for (int i = 0; i < kPer; ++i) {
            const int c = cbase + i * kAttnThreads;
            const bool in = c < STEP * CPR;
            const int r = in ? c / CPR : 0;
            const int32_t t = toks[r];
            v[i] = *reinterpret_cast<const u32x4 *>(kv + static_cast<int64_t>(t < 0 ? 0 : t) * a.kv_row_stride +
                                                    (in ? 8 * (c - r * CPR) : 0));
        }
    };
    auto store_rows = [&](uint16_t *rows) {
#pragma unroll
        for (int i = 0; i < kPer; ++i) {
            const int c = cbase + i * kAttnThreads;
            if (c < STEP * CPR) {
                const int r = c / CPR;
                *reinterpret_cast<u32x4 *>(rows + r * RS + 8 * (c - r * CPR)) = v[i];
            }
        }
    };

    // q fragments of this wave's head tile (B operand of S^T = K Q^T)
    bf16x8 qb[KSK];
    {
        const uint16_t *qh = a.q + (static_cast<int64_t>(qi) * a.Ha + hg * HG + 16 * hw + n) * Dk;
#pragma unroll
        for (int ks = 0; ks < KSK; ++ks) qb[ks] = load_bf16x8(qh + 32 * ks + 8 * g);
    }
    f32x4 oacc[DVW][HT];
#pragma unroll
    for (int dt = 0; dt < DVW; ++dt)
#pragma unroll
        for (int ht = 0; ht < HT; ++ht) oacc[dt][ht] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    float mrun[HT];
#pragma unroll
    for (int ht = 0; ht < HT; ++ht) mrun[ht] = -__builtin_huge_valf();
    float lpart = 0.0f;

    // prologue: entries of steps 0 and 1, rows of step 0
    if (tid < STEP) {
        L.tok[0][tid] = entry(e0 + tid);
        L.tok[1][tid] = entry(e0 + STEP + tid);
    }
    __syncthreads();
    load_rows(L.tok[0]);
    store_rows(L.rows[0]);
    __syncthreads();

    for (int i = 0; i < nsteps; ++i) {
        const int cur = i & 1;
        // ---- in flight during this step: the next step's rows, entries two steps ahead
        if (i + 1 < nsteps) load_rows(L.tok[cur ^ 1]);
        int32_t ahead = -1;
        if (tid < STEP) ahead = entry(e0 + (i + 2) * STEP + tid);

        // ---- scores of token tile tt against head tile hw
        // two accumulator chains (even and odd k-steps) halve the dependent MFMA latency
        f32x4 sacc = {0.0f, 0.0f, 0.0f, 0.0f}, sacc1 = {0.0f, 0.0f, 0.0f, 0.0f};
        const uint16_t *rows = L.rows[0];
        const uint16_t *krow = rows + (16 * tt + n) * RS + 8 * g;
#pragma unroll
        for (int ks = 0; ks < KSK; ks += 2) {
            sacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(load_bf16x8(krow + 32 * ks), qb[ks], sacc, 0, 0, 0);
            if (ks + 1 < KSK)
                sacc1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(load_bf16x8(krow + 32 * ks + 32), qb[ks + 1], sacc1, 0,
                                                                0, 0);
        }
        sacc += sacc1;
        // lane (g, n): tokens 16*tt + 4g + r of the step, head n of tile hw
        bool ok[4];
        float sv[4];
        float mx = -__builtin_huge_valf();
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            ok[r] = L.tok[cur][16 * tt + 4 * g + r] >= 0;
            sv[r] = ok[r] ? sacc[r] * a.scale_log2 : -__builtin_huge_valf();
            mx = fmaxf(mx, sv[r]);
        }
        mx = rows_max(mx);
        if (g == 0) L.wmax[tt][16 * hw + n] = mx;
        __syncthreads();

        // ---- online softmax: running max of every head tile, rescale, P^T into LDS
        float alpha[HT];
#pragma unroll
        for (int ht = 0; ht < HT; ++ht) {
            float mstep = L.wmax[0][16 * ht + n];
#pragma unroll
            for (int u = 1; u < TT; ++u) mstep = fmaxf(mstep, L.wmax[u][16 * ht + n]);
            const float mnew = fmaxf(mrun[ht], mstep);
            alpha[ht] = mnew == -__builtin_huge_valf() ? 1.0f : __builtin_amdgcn_exp2f(mrun[ht] - mnew);
            mrun[ht] = mnew;
        }
        {
            const float mw = mrun[hw];
            uint32_t packed[2];
            float psum = 0.0f;
#pragma unroll
            for (int r = 0; r < 4; r += 2) {
                const float p0 = ok[r] ? __builtin_amdgcn_exp2f(sv[r] - mw) : 0.0f;
                const float p1 = ok[r + 1] ? __builtin_amdgcn_exp2f(sv[r + 1] - mw) : 0.0f;
                const uint16_t b0 = f32_to_bf16_rne(p0), b1 = f32_to_bf16_rne(p1);
                psum += bf16_to_f32(b0) + bf16_to_f32(b1);
                packed[r / 2] = static_cast<uint32_t>(b0) | (static_cast<uint32_t>(b1) << 16);
            }
            lpart = lpart * alpha[hw] + psum;
            *reinterpret_cast<uint2 *>(L.pt + (16 * hw + n) * PS + 16 * tt + 4 * g) = make_uint2(packed[0], packed[1]);
        }
#pragma unroll
        for (int dt = 0; dt < DVW; ++dt)
#pragma unroll
            for (int ht = 0; ht < HT; ++ht) oacc[dt][ht] *= alpha[ht];
        __syncthreads();

        // ---- O^T += V^T P^T over the step's tokens
#pragma unroll
        for (int kk = 0; kk < KST; ++kk) {
            bf16x8 pb[HT];
#pragma unroll
            for (int ht = 0; ht < HT; ++ht) pb[ht] = load_bf16x8(L.pt + (16 * ht + n) * PS + 32 * kk + 8 * g);
#pragma unroll
            for (int dt = 0; dt < DVW; ++dt) {
                const bf16x8 va = load_vt_frag(rows, RS, 32 * kk + 8 * g, (wave * DVW + dt) * 16, lane);
#pragma unroll
                for (int ht = 0; ht < HT; ++ht)
                    oacc[dt][ht] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, pb[ht], oacc[dt][ht], 0, 0, 0);
            }
        }
        __syncthreads();                                        // rows, P^T and this step's entries are free
        if (i + 1 < nsteps) store_rows(L.rows[0]);
        if (tid < STEP) L.tok[cur][tid] = ahead;
        __syncthreads();
    }

    // ---- the denominators: this lane's tokens, then the wave, then the workgroup
    {
        const float l = rows_add(lpart);
        if (g == 0) L.wsum[tt][16 * hw + n] = l;
    }
    __syncthreads();
#pragma unroll
    for (int ht = 0; ht < HT; ++ht) {
        const int head = hg * HG + 16 * ht + n;
        float lsum = 0.0f;
#pragma unroll
        for (int u = 0; u < TT; ++u) lsum += L.wsum[u][16 * ht + n];
        if (a.nsplit == 1) {
            float *orow = a.out + (static_cast<int64_t>(qi) * a.Ha + head) * a.Dv;
            const float inv = lsum > 0.0f ? 1.0f / lsum : 0.0f;
#pragma unroll
            for (int dt = 0; dt < DVW; ++dt)
                *reinterpret_cast<f32x4 *>(orow + (wave * DVW + dt) * 16 + 4 * g) = oacc[dt][ht] * inv;
            if (a.lse && wave == 0 && g == 0)
                a.lse[static_cast<int64_t>(qi) * a.Ha + head] =
                    lsum > 0.0f ? (mrun[ht] + __builtin_log2f(lsum)) * kLn2 : -__builtin_huge_valf();
        } else {
            const int64_t prow = static_cast<int64_t>(pair) * a.Ha + head;
            float *orow = a.part_o + prow * a.Dv;
#pragma unroll
            for (int dt = 0; dt < DVW; ++dt)
                *reinterpret_cast<f32x4 *>(orow + (wave * DVW + dt) * 16 + 4 * g) = oacc[dt][ht];
            if (wave == 0 && g == 0) {
                a.part_m[prow] = mrun[ht];
                a.part_l[prow] = lsum;
            }
        }
    }
}

// grid: (S*T*Ha), Dv/4 threads: merges the nsplit partials of one (query, head).
// Every load is issued before any value is used, 16 splits at a time (a load
// under a test of an earlier one waits for it).  Up to 16 splits everything is
// read in one round; beyond, the maxima first, then the weighted sums, in the
// same split order either way.
// Leading arguments preloaded at dispatch (pk = Ha | nsplit << 16), the rest
// of the struct used only for the outputs.
__global__ __launch_bounds__(128) void attn_combine_kernel(float *part_o, float *part_m, float *part_l, uint32_t pk,
                                                           int32_t Dv, AttnArgs a_in) {
    AttnArgs a = a_in;
    a.part_o = part_o; a.part_m = part_m; a.part_l = part_l; a.Dv = Dv;
    a.Ha = static_cast<int>(pk & 0xffffu);
    a.nsplit = static_cast<int>(pk >> 16);
    constexpr int U = 16;
    const int qh = blockIdx.x;                      // query * Ha + head
    const int qi = qh / a.Ha, head = qh - qi * a.Ha;
    const int c = threadIdx.x * 4;
    if (c >= a.Dv) return;
    const int64_t row0 = static_cast<int64_t>(qi) * a.nsplit * a.Ha + head;    // split sp at row0 + sp*Ha
    float M = -__builtin_huge_valf();
    f32x4 o = {0.0f, 0.0f, 0.0f, 0.0f};
    float lsum = 0.0f;
    // splits sp0 .. sp0+U-1: partial rows (when `rows`), weights and maxima;
    // splits past nsplit re-read split sp0 and get weight 0
    auto load = [&](int sp0, bool rows, f32x4 (&po)[U], float (&wl)[U], float (&ll)[U]) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int sp = sp0 + u < a.nsplit ? sp0 + u : sp0;
            const int64_t prow = row0 + static_cast<int64_t>(sp) * a.Ha;
            if (rows) po[u] = *reinterpret_cast<const f32x4 *>(a.part_o + prow * a.Dv + c);
            const float l = a.part_l[prow];
            ll[u] = sp0 + u < a.nsplit ? l : 0.0f;
            wl[u] = a.part_m[prow];
        }
    };
    auto accumulate = [&](const f32x4 (&po)[U], const float (&wl)[U], const float (&ll)[U]) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            if (!(ll[u] > 0.0f)) continue;
            const float wgt = __builtin_amdgcn_exp2f(wl[u] - M);
            lsum += wgt * ll[u];
            o += wgt * po[u];
        }
    };
    f32x4 po[U];
    float wl[U], ll[U];
    if (a.nsplit <= U) {
        load(0, true, po, wl, ll);
#pragma unroll
        for (int u = 0; u < U; ++u)
            if (ll[u] > 0.0f) M = fmaxf(M, wl[u]);
        if (M != -__builtin_huge_valf()) accumulate(po, wl, ll);
    } else {
        for (int sp0 = 0; sp0 < a.nsplit; sp0 += U) {
            load(sp0, false, po, wl, ll);
#pragma unroll
            for (int u = 0; u < U; ++u)
                if (ll[u] > 0.0f) M = fmaxf(M, wl[u]);
        }
        if (M != -__builtin_huge_valf())
            for (int sp0 = 0; sp0 < a.nsplit; sp0 += U) {
                load(sp0, true, po, wl, ll);
                accumulate(po, wl, ll);
            }
    }
    const float inv = lsum > 0.0f ? 1.0f / lsum : 0.0f;
    *reinterpret_cast<f32x4 *>(a.out + static_cast<int64_t>(qh) * a.Dv + c) = o * inv;
    if (a.lse && c == 0) a.lse[qh] = lsum > 0.0f ? (M + __builtin_log2f(lsum)) * kLn2 : -__builtin_huge_valf();
}

template <int HT, int KSK, int DVW>
hipError_t launch_attn(const AttnArgs &a, hipStream_t st) {
    const int nhg = a.Ha / (16 * HT);
    const dim3 grid(static_cast<uint32_t>((a.npair + 7) / 8 * 8 * nhg));
    // Ha <= 128 and nsplit <= k / 64 < 2^16 (the ABI's limits): pk holds both
    const uint32_t pk = static_cast<uint32_t>(a.Ha) | static_cast<uint32_t>(a.nsplit) << 16;
    const bool fits = a.kv_seq_stride < (int64_t{1} << 31) && a.kv_row_stride < (int64_t{1} << 31);
    hipError_t e = fits
        ? launch(kKindAttention, sparse_attn_kernel<HT, KSK, DVW, true>, grid, dim3(kAttnThreads), 0, st, a.idx,
                 a.kv, a.q, static_cast<int32_t>(a.kv_seq_stride), static_cast<int32_t>(a.kv_row_stride),
                 static_cast<int32_t>(a.L), a.k, a.tps, pk, a.T, a.npair, a)
        : launch(kKindAttention, sparse_attn_kernel<HT, KSK, DVW, false>, grid, dim3(kAttnThreads), 0, st,
                 static_cast<const int32_t *>(nullptr), static_cast<const uint16_t *>(nullptr),
                 static_cast<const uint16_t *>(nullptr), 0, 0, 0, 0, 0, 0u, 0, 0, a);
    if (e != hipSuccess || a.nsplit == 1) return e;
    return launch(kKindAttnCombine, attn_combine_kernel, dim3(static_cast<uint32_t>(a.S * a.T * a.Ha)),
                  dim3(128), 0, st, a.part_o, a.part_m, a.part_l, pk, a.Dv, a);
}

template <int KSK, int DVW>
hipError_t launch_attn_heads(const AttnArgs &a, hipStream_t st) {
    if (a.Ha % 32 == 0) return launch_attn<2, KSK, DVW>(a, st);
    return launch_attn<1, KSK, DVW>(a, st);
}

}  // namespace

bool attention_shape_supported(int Dk, int Dv) {
    return (Dk == 64 && Dv == 64) || (Dk == 128 && Dv == 128) || (Dk == 192 && Dv == 128) ||
           (Dk == 576 && Dv == 512);
}

void attention_split(int nq, int Ha, int Dk, int Dv, int k, int &nsplit, int &tps) {
    const int hg = Ha % 32 == 0 ? 32 : 16;
    const int64_t base = static_cast<int64_t>(nq) * (Ha / hg);
    const int64_t steps = (k + kAttnStep - 1) / kAttnStep;
    // enough workgroups for two per compute unit, but the partials one split
    // writes (Ha*Dv fp32 per query) no larger than twice the rows it reads (Dk
    // bf16 per entry).  At 8 queries x 128 heads x 2048 entries (Dk 576, Dv
    // 512) that is 16 splits: the attention kernel 27 -> 23 us, the combine
    // 4.4 -> 7.4 us, the call 32.9 -> 31.1 us against the cap at the rows' own
    // size (8 splits)
    int64_t want = (512 + base - 1) / base;
    const int64_t cap = static_cast<int64_t>(k) * Dk * 2 / (static_cast<int64_t>(Ha) * Dv * 4);
    want = want < 2 * cap ? want : 2 * cap;
    want = want < 1 ? 1 : (want > steps ? steps : want);
    tps = static_cast<int>((steps + want - 1) / want * kAttnStep);
    nsplit = static_cast<int>((k + tps - 1) / tps);
}

hipError_t launch_attention(const AttnArgs &a, hipStream_t st) {
    if (a.Dk == 64) return launch_attn_heads<2, 1>(a, st);
    if (a.Dk == 128) return launch_attn_heads<4, 2>(a, st);
    if (a.Dk == 192) return launch_attn_heads<6, 2>(a, st);
    return launch_attn_heads<18, 8>(a, st);
}

}  // namespace hisa
