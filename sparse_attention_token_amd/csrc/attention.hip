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
// run of the set, in steps of 64 tokens:
//   1. the step's 64 latent rows are gathered into LDS (16-byte loads; rows
//      padded to Dk + 8 elements so 16 consecutive rows start on distinct
//      banks);
//   2. wave w scores tokens 16w..16w+15 against the group's heads:
//      S^T = K Q^T with v_mfma_f32_16x16x32_bf16 (A = the token rows from LDS,
//      M = tokens; B = q, held in registers for the whole run, N = heads), so
//      each latent row is read from LDS once per workgroup;
//   3. online softmax in the exp2 domain: the step's maximum per head is
//      combined across the waves through LDS, P = exp2(s - m) is rounded to
//      bf16 and written to LDS as P^T [head][token];
//   4. wave w accumulates its quarter of the value columns for every head:
//      O^T += V^T P^T (A = V^T, read with the gfx950 transposing LDS load
//      ds_read_b64_tr_b16 straight from the token-major rows; B = P^T; K = 64
//      tokens).  O^T keeps one head per lane column, so the per-head rescale
//      of the online softmax is a per-lane scalar.
// The denominator sums the bf16-rounded weights, so the result is an exact
// convex combination of the values with weights within a bf16 rounding of the
// softmax.  When the set is split over several workgroups (few queries), each
// writes its unnormalised partial (O, m, l) and a combine kernel merges them.

#include "hisa_internal.h"
#include "scorer.h"

namespace hisa {
namespace {

constexpr int kAttnThreads = 256;
constexpr int kAttnStep = 64;                 // tokens per step
constexpr int kAttnPStride = kAttnStep + 8;   // P^T row stride (elements)
constexpr float kLn2 = 0.6931471805599453f;

typedef short v4s __attribute__((ext_vector_type(4)));
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
    const v4s a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s *)(p0));
    const v4s b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s *)(p0 + 4 * stride));
    const u32x4 u = {static_cast<uint32_t>(static_cast<uint16_t>(a[0])) | (static_cast<uint32_t>(static_cast<uint16_t>(a[1])) << 16),
                     static_cast<uint32_t>(static_cast<uint16_t>(a[2])) | (static_cast<uint32_t>(static_cast<uint16_t>(a[3])) << 16),
                     static_cast<uint32_t>(static_cast<uint16_t>(b[0])) | (static_cast<uint32_t>(static_cast<uint16_t>(b[1])) << 16),
                     static_cast<uint32_t>(static_cast<uint16_t>(b[2])) | (static_cast<uint32_t>(static_cast<uint16_t>(b[3])) << 16)};
    return as_bf16x8(u);
}

template <int HT, int KSK, int DVW>
struct AttnLds {
    static constexpr int kDk = 32 * KSK;
    static constexpr int kRowStride = kDk + 8;
    uint16_t rows[kAttnStep * kRowStride];
    uint16_t pt[16 * HT * kAttnPStride];
    float wmax[4][16 * HT];
    float wsum[4][16 * HT];
    int valid[kAttnStep];
};

// grid: attn_grid(npair, nhg) with npair = S*T*nsplit; workgroup (pair, hg)
// takes query pair / nsplit, heads hg*16*HT.., and set entries
// [split*tps, min(k, split*tps + tps)).
template <int HT, int KSK, int DVW>
__global__ __launch_bounds__(kAttnThreads) void sparse_attn_kernel(AttnArgs a) {
    constexpr int Dk = 32 * KSK;
    constexpr int HG = 16 * HT;
    using Lds = AttnLds<HT, KSK, DVW>;
    constexpr int RS = Lds::kRowStride;
    constexpr int CPR = Dk / 8;                                 // 16-byte chunks per row
    constexpr int kPer = (kAttnStep * CPR + kAttnThreads - 1) / kAttnThreads;
    __shared__ __attribute__((aligned(16))) Lds L;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int n = lane & 15, g = lane >> 4;
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
    const int32_t *idx = a.idx + static_cast<int64_t>(qi) * a.k;
    const uint16_t *kv = a.kv + s * a.kv_seq_stride;

    // q fragments (B operand of S^T = K Q^T): lane (g, n) holds head n's 8
    // entries 32*ks + 8g .. of each k-step
    bf16x8 qb[HT][KSK];
#pragma unroll
    for (int ht = 0; ht < HT; ++ht) {
        const uint16_t *qh = a.q + (static_cast<int64_t>(qi) * a.Ha + hg * HG + 16 * ht + n) * Dk;
#pragma unroll
        for (int ks = 0; ks < KSK; ++ks) qb[ht][ks] = load_bf16x8(qh + 32 * ks + 8 * g);
    }

    f32x4 oacc[DVW][HT];
#pragma unroll
    for (int dt = 0; dt < DVW; ++dt)
#pragma unroll
        for (int ht = 0; ht < HT; ++ht) oacc[dt][ht] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    float mrun[HT], lpart[HT];
#pragma unroll
    for (int ht = 0; ht < HT; ++ht) {
        mrun[ht] = -__builtin_huge_valf();
        lpart[ht] = 0.0f;
    }

    for (int base = e0; base < e1; base += kAttnStep) {
        __syncthreads();                                        // the previous step's LDS reads are done
        // ---- gather the step's rows (invalid entries: zero rows)
        {
            u32x4 v[kPer];
#pragma unroll
            for (int i = 0; i < kPer; ++i) {
                const int c = tid + i * kAttnThreads;
                v[i] = u32x4{0u, 0u, 0u, 0u};
                if (c < kAttnStep * CPR) {
                    const int r = c / CPR;
                    const int e = base + r;
                    const int32_t tok = e < e1 ? idx[e] : -1;
                    if (tok >= 0 && tok < a.L)
                        v[i] = *reinterpret_cast<const u32x4 *>(kv + static_cast<int64_t>(tok) * a.kv_row_stride +
                                                                8 * (c - r * CPR));
                }
            }
#pragma unroll
            for (int i = 0; i < kPer; ++i) {
                const int c = tid + i * kAttnThreads;
                if (c < kAttnStep * CPR) {
                    const int r = c / CPR;
                    *reinterpret_cast<u32x4 *>(L.rows + r * RS + 8 * (c - r * CPR)) = v[i];
                }
            }
            if (tid < kAttnStep) {
                const int e = base + tid;
                const int32_t tok = e < e1 ? idx[e] : -1;
                L.valid[tid] = tok >= 0 && tok < a.L;
            }
        }
        __syncthreads();

        // ---- scores of this wave's 16 tokens for every head of the group
        f32x4 sacc[HT];
#pragma unroll
        for (int ht = 0; ht < HT; ++ht) sacc[ht] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
        const uint16_t *krow = L.rows + (16 * wave + n) * RS + 8 * g;
#pragma unroll
        for (int ks = 0; ks < KSK; ++ks) {
            const bf16x8 kfrag = load_bf16x8(krow + 32 * ks);
#pragma unroll
            for (int ht = 0; ht < HT; ++ht)
                sacc[ht] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kfrag, qb[ht][ks], sacc[ht], 0, 0, 0);
        }
        // lane (g, n): tokens 16w + 4g + r (r = 0..3), head n of each tile
        bool ok[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) ok[r] = L.valid[16 * wave + 4 * g + r] != 0;
        float sv[HT][4];
#pragma unroll
        for (int ht = 0; ht < HT; ++ht) {
            float mx = -__builtin_huge_valf();
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                sv[ht][r] = ok[r] ? sacc[ht][r] * a.scale_log2 : -__builtin_huge_valf();
                mx = fmaxf(mx, sv[ht][r]);
            }
            mx = rows_max(mx);
            if (g == 0) L.wmax[wave][16 * ht + n] = mx;
        }
        __syncthreads();

        // ---- online softmax: new running max, rescale, P^T into LDS
        float alpha[HT];
#pragma unroll
        for (int ht = 0; ht < HT; ++ht) {
            float mstep = L.wmax[0][16 * ht + n];
#pragma unroll
            for (int w = 1; w < 4; ++w) mstep = fmaxf(mstep, L.wmax[w][16 * ht + n]);
            const float mnew = fmaxf(mrun[ht], mstep);
            alpha[ht] = mnew == -__builtin_huge_valf() ? 1.0f : __builtin_amdgcn_exp2f(mrun[ht] - mnew);
            mrun[ht] = mnew;
            uint32_t packed[2];
            float psum = 0.0f;
#pragma unroll
            for (int r = 0; r < 4; r += 2) {
                const float p0 = ok[r] ? __builtin_amdgcn_exp2f(sv[ht][r] - mnew) : 0.0f;
                const float p1 = ok[r + 1] ? __builtin_amdgcn_exp2f(sv[ht][r + 1] - mnew) : 0.0f;
                const uint16_t b0 = f32_to_bf16_rne(p0), b1 = f32_to_bf16_rne(p1);
                psum += bf16_to_f32(b0) + bf16_to_f32(b1);
                packed[r / 2] = static_cast<uint32_t>(b0) | (static_cast<uint32_t>(b1) << 16);
            }
            lpart[ht] = lpart[ht] * alpha[ht] + psum;
            *reinterpret_cast<uint2 *>(L.pt + (16 * ht + n) * kAttnPStride + 16 * wave + 4 * g) =
                make_uint2(packed[0], packed[1]);
        }
#pragma unroll
        for (int dt = 0; dt < DVW; ++dt)
#pragma unroll
            for (int ht = 0; ht < HT; ++ht) oacc[dt][ht] *= alpha[ht];
        __syncthreads();

        // ---- O^T += V^T P^T over the step's 64 tokens (two k-steps of 32)
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
            bf16x8 pb[HT];
#pragma unroll
            for (int ht = 0; ht < HT; ++ht)
                pb[ht] = load_bf16x8(L.pt + (16 * ht + n) * kAttnPStride + 32 * kk + 8 * g);
#pragma unroll
            for (int dt = 0; dt < DVW; ++dt) {
                const bf16x8 va = load_vt_frag(L.rows, RS, 32 * kk + 8 * g, (wave * DVW + dt) * 16, lane);
#pragma unroll
                for (int ht = 0; ht < HT; ++ht)
                    oacc[dt][ht] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, pb[ht], oacc[dt][ht], 0, 0, 0);
            }
        }
    }

    // ---- the denominators: this lane's tokens, then the wave, then the workgroup
    __syncthreads();
#pragma unroll
    for (int ht = 0; ht < HT; ++ht) {
        const float l = rows_add(lpart[ht]);
        if (g == 0) L.wsum[wave][16 * ht + n] = l;
    }
    __syncthreads();
#pragma unroll
    for (int ht = 0; ht < HT; ++ht) {
        const int head = hg * HG + 16 * ht + n;
        const float lsum = L.wsum[0][16 * ht + n] + L.wsum[1][16 * ht + n] + L.wsum[2][16 * ht + n] +
                           L.wsum[3][16 * ht + n];
        if (a.nsplit == 1) {
            float *orow = a.out + (static_cast<int64_t>(qi) * a.Ha + head) * a.Dv;
            const float inv = lsum > 0.0f ? 1.0f / lsum : 0.0f;
#pragma unroll
            for (int dt = 0; dt < DVW; ++dt) {
                const f32x4 o = oacc[dt][ht] * inv;
                *reinterpret_cast<f32x4 *>(orow + (wave * DVW + dt) * 16 + 4 * g) = o;
            }
            if (a.lse && wave == 0 && g == 0)
                a.lse[static_cast<int64_t>(qi) * a.Ha + head] =
                    lsum > 0.0f ? (mrun[ht] + __builtin_log2f(lsum)) * kLn2 : -__builtin_huge_valf();
        } else {
            const int64_t prow = (static_cast<int64_t>(pair) * a.Ha + head);
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
__global__ __launch_bounds__(128) void attn_combine_kernel(AttnArgs a) {
    const int qh = blockIdx.x;                      // query * Ha + head
    const int qi = qh / a.Ha, head = qh - qi * a.Ha;
    const int c = threadIdx.x * 4;
    if (c >= a.Dv) return;
    float M = -__builtin_huge_valf();
    for (int sp = 0; sp < a.nsplit; ++sp) {
        const int64_t prow = (static_cast<int64_t>(qi) * a.nsplit + sp) * a.Ha + head;
        if (a.part_l[prow] > 0.0f) M = fmaxf(M, a.part_m[prow]);
    }
    f32x4 o = {0.0f, 0.0f, 0.0f, 0.0f};
    float lsum = 0.0f;
    if (M != -__builtin_huge_valf()) {
        for (int sp = 0; sp < a.nsplit; ++sp) {
            const int64_t prow = (static_cast<int64_t>(qi) * a.nsplit + sp) * a.Ha + head;
            const float l = a.part_l[prow];
            if (!(l > 0.0f)) continue;
            const float wgt = __builtin_amdgcn_exp2f(a.part_m[prow] - M);
            lsum += wgt * l;
            o += wgt * *reinterpret_cast<const f32x4 *>(a.part_o + prow * a.Dv + c);
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
    hipError_t e = launch(kKindAttention, sparse_attn_kernel<HT, KSK, DVW>, grid, dim3(kAttnThreads), 0, st, a);
    if (e != hipSuccess || a.nsplit == 1) return e;
    return launch(kKindAttnCombine, attn_combine_kernel, dim3(static_cast<uint32_t>(a.S * a.T * a.Ha)),
                  dim3(128), 0, st, a);
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

void attention_split(int nq, int Ha, int k, int &nsplit, int &tps) {
    const int hg = Ha % 32 == 0 ? 32 : 16;
    const int64_t base = static_cast<int64_t>(nq) * (Ha / hg);
    const int steps = (k + kAttnStep - 1) / kAttnStep;
    int want = static_cast<int>((512 + base - 1) / base);
    want = want < 1 ? 1 : (want > steps ? steps : want);
    tps = (steps + want - 1) / want * kAttnStep;
    nsplit = (k + tps - 1) / tps;
}

hipError_t launch_attention(const AttnArgs &a, hipStream_t st) {
    if (a.Dk == 64) return launch_attn_heads<2, 1>(a, st);
    if (a.Dk == 128) return launch_attn_heads<4, 2>(a, st);
    if (a.Dk == 192) return launch_attn_heads<6, 2>(a, st);
    return launch_attn_heads<18, 8>(a, st);
}

}  // namespace hisa
