// The indexer scorer on the matrix cores, as device building blocks shared by
// every kernel that scores rows (block stage, refinement, flat indexer).
//
// For one query (H heads of dimension d = 32*KS) and 16 rows x_j,
//     s_j = sum_h w_h * ReLU(q_h . x_j)
// -- the DSA lightweight-indexer score that the pages' "original indexer"
// applies both to block representatives (coarse stage) and to tokens
// (refinement); arXiv abstract and gptget.net English summary, "Methodology".
//
// The contraction over d runs on v_mfma_f32_16x16x32_bf16 (bf16 inputs, fp32
// accumulation):  A = q (M = heads, 16 per M-tile, zero past H),
// B = rows (N = 16), K = d (32 per k-step).  Lane l = 16*g + n supplies
// A[head 16*mt + n][8 consecutive d] and B[same 8 d][row n], so the pairing of
// the contraction index is the same whatever order the unit sums its slots in.
// D[head][row] comes back as heads 4g..4g+3 of row n in each lane; the fp32
// epilogue applies ReLU and w and sums heads: the lane's 4*MT values in a fixed
// order with explicit fused multiply-adds (ReLU as an integer max on the bit
// pattern), then across the four lane groups
// with two xor-shuffles.  Every kernel
// calls score_rows(), so a given (query, row) gets the same fp32 bits wherever
// it is scored.
#pragma once

#include "hisa_internal.h"

namespace hisa {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// Marks x as consumed by every lane at this point.  A value loaded by all
// threads but used only under a branch (a head weight stored to LDS by
// tid < 64) has its load sunk into that branch by the compiler, behind the
// wait for every load issued earlier: one more memory round trip, which the
// next barrier hands on to every wave.  Pinned where those loads are awaited
// anyway, the load issues with them.
__device__ __forceinline__ void pin_loaded(float x) { asm volatile("" ::"v"(x)); }

__device__ __forceinline__ bf16x8 load_bf16x8(const uint16_t *p) {
    return as_bf16x8(*reinterpret_cast<const u32x4 *>(p));
}

__device__ __forceinline__ bf16x8 zero_bf16x8() {
    const u32x4 z = {0u, 0u, 0u, 0u};
    return as_bf16x8(z);
}

// Query fragments and head weights held in registers by one wave.
template <int MT, int KS>
struct QFrag {
    bf16x8 qa[MT][KS];
    float wv[MT][4];
};

// LDS staging of a query: rows of kQStride elements (d + 8 pad keeps the
// 16-byte fragment reads of 16 consecutive heads on distinct banks).
template <int KS>
struct QStage {
    static constexpr int D = 32 * KS;
    static constexpr int kStride = D + 8;
};

// Copy q [H][D] (global) into s_q [MT*16][D+8] with zero rows past H, in two
// halves so that a caller can keep the loads in flight across other work:
// load() issues every global load into registers, store() writes them to LDS.
template <int MT, int KS, int NT>
struct QStager {
    static constexpr int D = QStage<KS>::D, ST = QStage<KS>::kStride;
    static constexpr int kChunks = MT * 16 * D / 8;
    static constexpr int kPer = (kChunks + NT - 1) / NT;
    u32x4 v[kPer];

    // Loads are unconditional (heads past H read head H-1, zeroed by
    // store()): a load under a branch can make the wave wait for it at once.
    __device__ __forceinline__ void load(const uint16_t *__restrict__ q, int H, int tid) {
#pragma unroll
        for (int i = 0; i < kPer; ++i) {
            const int c = tid + i * NT;
            const int h = c / (D / 8);
            const int hc = h < H ? h : H - 1;
            if (kChunks % NT == 0 || c < kChunks)
                v[i] = *reinterpret_cast<const u32x4 *>(q + hc * D + 8 * (c - h * (D / 8)));
        }
    }
    __device__ __forceinline__ void store(uint16_t *s_q, int H, int tid) const {
#pragma unroll
        for (int i = 0; i < kPer; ++i) {
            const int c = tid + i * NT;
            const int h = c / (D / 8);
            if (kChunks % NT == 0 || c < kChunks)
                *reinterpret_cast<u32x4 *>(s_q + h * ST + 8 * (c - h * (D / 8))) =
                    h < H ? v[i] : u32x4{0u, 0u, 0u, 0u};
        }
    }
};

template <int MT, int KS, int NT>
__device__ __forceinline__ void stage_query(const uint16_t *__restrict__ q, int H, uint16_t *s_q, int tid) {
    QStager<MT, KS, NT> st;
    st.load(q, H, tid);
    st.store(s_q, H, tid);
}

template <int MT, int KS>
__device__ __forceinline__ void load_qfrag_lds(QFrag<MT, KS> &f, const uint16_t *s_q,
                                               const float *__restrict__ w, int H, int lane) {
    constexpr int ST = QStage<KS>::kStride;
    const int n = lane & 15, g = lane >> 4;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
            f.qa[mt][ks] = load_bf16x8(s_q + (16 * mt + n) * ST + 32 * ks + 8 * g);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int head = 16 * mt + 4 * g + r;
            f.wv[mt][r] = head < H ? w[head] : 0.0f;
        }
}

// As load_qfrag_lds, with the head weights also read from LDS (s_w[MT*16],
// zero past H).
template <int MT, int KS>
__device__ __forceinline__ void load_qfrag_lds_w(QFrag<MT, KS> &f, const uint16_t *s_q, const float *s_w,
                                                 int lane) {
    constexpr int ST = QStage<KS>::kStride;
    const int n = lane & 15, g = lane >> 4;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
            f.qa[mt][ks] = load_bf16x8(s_q + (16 * mt + n) * ST + 32 * ks + 8 * g);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int r = 0; r < 4; ++r) f.wv[mt][r] = s_w[16 * mt + 4 * g + r];
}

template <int MT, int KS>
__device__ __forceinline__ void load_qfrag_global(QFrag<MT, KS> &f, const uint16_t *__restrict__ q,
                                                  const float *__restrict__ w, int H, int lane) {
    constexpr int D = 32 * KS;
    const int n = lane & 15, g = lane >> 4;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
        const int head = 16 * mt + n;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
            f.qa[mt][ks] = head < H ? load_bf16x8(q + head * D + 32 * ks + 8 * g) : zero_bf16x8();
    }
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int head = 16 * mt + 4 * g + r;
            f.wv[mt][r] = head < H ? w[head] : 0.0f;
        }
}

// As load_qfrag_global with every load issued unconditionally (heads past H
// read head H-1 and are zeroed afterwards, weights past H are zero), so the
// loads do not wait for each other.
template <int MT, int KS>
__device__ __forceinline__ void load_qfrag_global_any(QFrag<MT, KS> &f, const uint16_t *__restrict__ q,
                                                      const float *__restrict__ w, int H, int lane) {
    constexpr int D = 32 * KS;
    const int n = lane & 15, g = lane >> 4;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
        const int head = 16 * mt + n;
        const int hc = head < H ? head : H - 1;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) f.qa[mt][ks] = load_bf16x8(q + hc * D + 32 * ks + 8 * g);
    }
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int head = 16 * mt + 4 * g + r;
            f.wv[mt][r] = w[head < H ? head : H - 1];
        }
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
        const int head = 16 * mt + n;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
            if (head >= H) f.qa[mt][ks] = zero_bf16x8();
#pragma unroll
        for (int r = 0; r < 4; ++r)
            if (16 * mt + 4 * g + r >= H) f.wv[mt][r] = 0.0f;
    }
}

// The row fragment of lane (n, g): 8 consecutive d of row n for each k-step.
template <int KS>
__device__ __forceinline__ void load_row_frag(bf16x8 (&kb)[KS], const uint16_t *row, int lane) {
    const int g = lane >> 4;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
        kb[ks] = row ? load_bf16x8(row + 32 * ks + 8 * g) : zero_bf16x8();
}

// As load_row_frag for a pointer that is always a valid row: the loads are
// unconditional.  A load under a null test compiles to a branch on the exec
// mask, and the register copy that joins its two sides makes the wave wait
// for the load right there (one full memory round trip before the next
// load is even issued); callers that have no row for a lane point it at any
// valid row instead and discard that row's score.
template <int KS>
__device__ __forceinline__ void load_row_frag_any(bf16x8 (&kb)[KS], const uint16_t *row, int lane) {
    const int g = lane >> 4;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) kb[ks] = load_bf16x8(row + 32 * ks + 8 * g);
}

// max(x, 0) for finite x, as one integer max on the bit pattern: every
// negative value (and -0) has a negative two's-complement pattern and becomes
// +0; non-negative values pass unchanged.
__device__ __forceinline__ float relu_bits(float x) {
    return __int_as_float(max(__float_as_int(x), 0));
}

// Sum of x over the four 16-lane rows of a wave, (x_r + x_(r^1)) summed
// across the two halves, returned to every lane.  The two lane swaps
// (v_permlane16_swap, v_permlane32_swap) are VALU operations rather than LDS
// permutes; addition is commutative, so both lanes of a swapped pair compute
// the same bits, as an xor-shuffle sum in the same order would.
__device__ __forceinline__ float rows_sum(float x) {
    const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    const float y = __uint_as_float(p[0]) + __uint_as_float(p[1]);
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(y), __float_as_uint(y), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Score of row (lane & 15) for this query; every lane of the row's column
// group returns the same value.
template <int MT, int KS>
__device__ __forceinline__ float score_rows(const QFrag<MT, KS> &f, const bf16x8 (&kb)[KS]) {
    float part = 0.0f;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
        f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(f.qa[mt][ks], kb[ks], acc, 0, 0, 0);
#pragma unroll
        for (int r = 0; r < 4; ++r) part = __builtin_fmaf(f.wv[mt][r], relu_bits(acc[r]), part);
    }
    return rows_sum(part);
}

// NT 16-row tiles of one query at once with the fragments in registers; per
// tile the arithmetic is exactly score_rows(), with NT accumulators in flight.
template <int MT, int KS, int NT>
__device__ __forceinline__ void score_tiles_frag(const QFrag<MT, KS> &f, const bf16x8 (&kb)[NT][KS],
                                                 float (&out)[NT]) {
    float part[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) part[nt] = 0.0f;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
        f32x4 acc[NT];
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) acc[nt] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
#pragma unroll
            for (int nt = 0; nt < NT; ++nt)
                acc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(f.qa[mt][ks], kb[nt][ks], acc[nt], 0, 0, 0);
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
#pragma unroll
            for (int r = 0; r < 4; ++r) part[nt] = __builtin_fmaf(f.wv[mt][r], relu_bits(acc[nt][r]), part[nt]);
    }
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) out[nt] = rows_sum(part[nt]);
}

// Swizzled LDS stage of one query: head row h holds its D elements at h * D
// with no padding, and its 16-byte chunk c sits in slot c ^ swz(h), where
// swz(h) is the low four bits of h with bits 0 and 1 exchanged (masked to
// the chunks of a row).  The 16x16x32 operand reads (16 rows x 4 chunks per
// wave-wide 16-byte load) then meet no LDS bank twice in one cycle; over
// rows padded to D + 8 elements they did, about 4 extra cycles per load as
// counted by the LDS bank-conflict counter.
template <int KS>
struct QSwz {
    static constexpr int D = 32 * KS, CPR = D / 8;   // 16-byte chunks per row
    __device__ static __forceinline__ int swz(int h) {
        const int r = h & 15;
        return ((r & 12) | ((r & 1) << 1) | ((r >> 1) & 1)) & (CPR - 1);
    }
    // element offset of chunk c of head row h
    __device__ static __forceinline__ int elem(int h, int c) { return h * D + 8 * (c ^ swz(h)); }
};

// NT 16-row tiles of one query at once, q and w read from LDS (swizzled
// layout of QSwz, w zero past H).  Per tile the arithmetic is exactly
// score_rows(): the same MFMA sequence per head group and the same fused
// multiply-add order over heads, then the same row sum.  Working one head
// group at a time over all tiles keeps NT accumulators in flight (independent
// MFMA chains) and needs only one head group's fragments in registers.
template <int MT, int KS, int NT>
__device__ __forceinline__ void score_tiles_lds(const uint16_t *s_q, const float *s_w,
                                                const bf16x8 (&kb)[NT][KS], float (&out)[NT], int lane) {
    using L = QSwz<KS>;
    const int n = lane & 15, g = lane >> 4;
    float part[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) part[nt] = 0.0f;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
        bf16x8 qa[KS];
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) qa[ks] = load_bf16x8(s_q + 16 * mt * L::D + L::elem(n, 4 * ks + g));
        float wv[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) wv[r] = s_w[16 * mt + 4 * g + r];
        f32x4 acc[NT];
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) acc[nt] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
#pragma unroll
            for (int nt = 0; nt < NT; ++nt)
                acc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[ks], kb[nt][ks], acc[nt], 0, 0, 0);
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
#pragma unroll
            for (int r = 0; r < 4; ++r) part[nt] = __builtin_fmaf(wv[r], relu_bits(acc[nt][r]), part[nt]);
    }
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) out[nt] = rows_sum(part[nt]);
}

}  // namespace hisa
