// Device helpers shared by the forward and backward kernels (gfx950).
// Included only by the .hip sources; not part of the public ABI.
#pragma once

#include "linattn_internal.h"

#include <type_traits>

namespace sana {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef short s16x2 __attribute__((ext_vector_type(2)));

// ReLU on two packed bf16: for the sign test a bf16 orders like an int16, so
// max(x, 0) as int16 keeps positives and maps negatives (and -0) to +0.
__device__ __forceinline__ uint32_t relu_bf16x2(uint32_t x) {
    s16x2 s = __builtin_bit_cast(s16x2, x);
    s = __builtin_elementwise_max(s, (s16x2){0, 0});
    return __builtin_bit_cast(uint32_t, s);
}

// ReLU of an fp32 value on its bits: as an int32 a float orders like its
// sign, so max(bits, 0) keeps positives and maps negatives (and -0) to +0 in
// one integer max (fmaxf also canonicalises its input: two instructions).
__device__ __forceinline__ float relu_f32(float x) {
    return __builtin_bit_cast(float, max(__builtin_bit_cast(int, x), 0));
}
// The same on one bf16 or fp16 value's bits (int16 order).
__device__ __forceinline__ uint16_t relu_16(uint16_t h) { return (uint16_t)max((int)(short)h, 0); }

__device__ __forceinline__ u32x4 relu_bf16x8(u32x4 x) {
    return (u32x4){relu_bf16x2(x[0]), relu_bf16x2(x[1]), relu_bf16x2(x[2]), relu_bf16x2(x[3])};
}

__device__ __forceinline__ f32x16 mfma_bf16(u32x4 a, u32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

__device__ __forceinline__ f32x16 mfma_f16(u32x4 a, u32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}

// The 16-bit input formats: bf16 (F16 = false) or IEEE binary16 (F16 = true).
// ReLU on packed values works the same for both: the sign is the top bit.
template <bool F16>
__device__ __forceinline__ f32x16 mfma16(u32x4 a, u32x4 b, f32x16 c) {
    if constexpr (F16)
        return mfma_f16(a, b, c);
    else
        return mfma_bf16(a, b, c);
}

__device__ __forceinline__ float f16_to_f32(uint16_t h) { return (float)__builtin_bit_cast(_Float16, h); }

// Splits two packed finite fp16 values exactly into bf16 terms, x = hi + lo:
// hi keeps the top 8 significant bits of the fp32 widening (truncation toward
// zero), and the remainder, of the same sign, has at most the 3 low
// significant bits of the 11, so it is a bf16 value too.  f0, f1 receive the
// fp32 values.
__device__ __forceinline__ void split_f16x2(uint32_t w, uint32_t& hi, uint32_t& lo, float& f0, float& f1) {
    f0 = f16_to_f32((uint16_t)(w & 0xffffu));
    f1 = f16_to_f32((uint16_t)(w >> 16));
    const uint32_t t0 = __builtin_bit_cast(uint32_t, f0) & 0xffff0000u;
    const uint32_t t1 = __builtin_bit_cast(uint32_t, f1) & 0xffff0000u;
    const float r0 = f0 - __builtin_bit_cast(float, t0);
    const float r1 = f1 - __builtin_bit_cast(float, t1);
    hi = (t0 >> 16) | t1;
    lo = (__builtin_bit_cast(uint32_t, r0) >> 16) | (__builtin_bit_cast(uint32_t, r1) & 0xffff0000u);
}

__device__ __forceinline__ float bf16_to_f32(uint16_t h) {
    return __builtin_bit_cast(float, (uint32_t)h << 16);
}
__device__ __forceinline__ float lo_bf16(uint32_t x) { return __builtin_bit_cast(float, x << 16); }
__device__ __forceinline__ float hi_bf16(uint32_t x) { return __builtin_bit_cast(float, x & 0xffff0000u); }

// Round to nearest, ties to even: gfx950's v_cvt_pk_bf16_f32.
__device__ __forceinline__ uint16_t f32_to_bf16(float f) { return __builtin_bit_cast(uint16_t, (__bf16)f); }

// Element types by ABI code: float (0), bf16 bits in uint16_t (1), _Float16 (2).
__device__ __forceinline__ float load_in(const float* p, long long i) { return p[i]; }
__device__ __forceinline__ float load_in(const uint16_t* p, long long i) { return bf16_to_f32(p[i]); }
__device__ __forceinline__ float load_in(const _Float16* p, long long i) { return (float)p[i]; }

// fp32 -> fp16 conversion rounds to nearest even; outputs lie within the range
// of V, so they never overflow.
__device__ __forceinline__ void store_out(float* p, long long i, float x) { p[i] = x; }
__device__ __forceinline__ void store_out(uint16_t* p, long long i, float x) { p[i] = f32_to_bf16(x); }
__device__ __forceinline__ void store_out(_Float16* p, long long i, float x) { p[i] = (_Float16)x; }

// fp32 output stores are non-temporal: out is written once and never read
// here, and streaming whole lines past the caches raises the write bandwidth
// markedly on gfx950.  A 16-bit row piece here is half of each line an
// instruction touches, and those stores are plain (non-temporal half-line
// stores measured slower: the JVP with bf16 out 148.4 against 151.5 us).
__device__ __forceinline__ void store4(float* p, f32x4 x) {
    __builtin_nontemporal_store(x, reinterpret_cast<f32x4*>(p));
}
__device__ __forceinline__ void store4(uint16_t* p, f32x4 x) {
    const uint32_t lo = (uint32_t)f32_to_bf16(x[0]) | ((uint32_t)f32_to_bf16(x[1]) << 16);
    const uint32_t hi = (uint32_t)f32_to_bf16(x[2]) | ((uint32_t)f32_to_bf16(x[3]) << 16);
    *reinterpret_cast<u32x2*>(p) = (u32x2){lo, hi};
}
__device__ __forceinline__ void store4(_Float16* p, f32x4 x) {
    const uint32_t h0 = __builtin_bit_cast(uint16_t, (_Float16)x[0]), h1 = __builtin_bit_cast(uint16_t, (_Float16)x[1]);
    const uint32_t h2 = __builtin_bit_cast(uint16_t, (_Float16)x[2]), h3 = __builtin_bit_cast(uint16_t, (_Float16)x[3]);
    *reinterpret_cast<u32x2*>(p) = (u32x2){h0 | (h1 << 16), h2 | (h3 << 16)};
}

// Three bf16 terms of an fp32 value, x = t0 + t1 + t2 to about 2^-24 relative:
// each term is the round-to-nearest bf16 of what the previous ones left, and
// each remainder is exact in fp32.
__device__ __forceinline__ void split3_f32(float x, uint16_t t[3]) {
#pragma unroll
    for (int sp = 0; sp < 3; ++sp) {
        t[sp] = f32_to_bf16(x);
        x -= bf16_to_f32(t[sp]);
    }
}

// Packs split terms of 8 consecutive fp32 values into three bf16x8 operands.
__device__ __forceinline__ void split3_f32x8(const float* x, u32x4 out[3]) {
#pragma unroll
    for (int d = 0; d < 4; ++d) {
        uint16_t a[3], b[3];
        split3_f32(x[2 * d], a);
        split3_f32(x[2 * d + 1], b);
#pragma unroll
        for (int sp = 0; sp < 3; ++sp) out[sp][d] = (uint32_t)a[sp] | ((uint32_t)b[sp] << 16);
    }
}

// Three bf16 terms of 8 fp32 values by truncation: t0 keeps the top 8
// significant bits of x, t1 the next 8 of the (exact) remainder, t2 the last
// 8, so x = t0 + t1 + t2 exactly (for x well above the fp32 subnormal range).
// Cheaper than split3_f32x8 (no rounding), for values split per token.
__device__ __forceinline__ void split3_trunc_f32x8(const float* x, u32x4 out[3]) {
#pragma unroll
    for (int d = 0; d < 4; ++d) {
        float a = x[2 * d], b = x[2 * d + 1];
#pragma unroll
        for (int sp = 0; sp < 3; ++sp) {
            const uint32_t ta = __builtin_bit_cast(uint32_t, a) & 0xffff0000u;
            const uint32_t tb = __builtin_bit_cast(uint32_t, b) & 0xffff0000u;
            out[sp][d] = (ta >> 16) | tb;
            a -= __builtin_bit_cast(float, ta);
            b -= __builtin_bit_cast(float, tb);
        }
    }
}

// Token range [c0, c1) of chunk p of a (b, head) unit.
struct ChunkRange { int c0, c1; };
__device__ __forceinline__ ChunkRange chunk_range(int p, int cpb, int chunk, int L, int N) {
    const int beta = p / cpb, s = p - beta * cpb;
    const int blk0 = beta * L;
    const int blk1 = min(blk0 + L, N);
    const int c0 = blk0 + s * chunk;
    return {c0, min(c0 + chunk, blk1)};
}

// ------------------------------------------------------------------ matrix-core helpers
constexpr int kPitch = 36;   // floats per LDS tile row: 32 + 4 keeps rows 16-byte aligned, no bank conflicts

// K-steps of 16 features in a 32-column block's product for head dim HD
// (the kernels see a token row as 32-feature groups: a head of 64 is two, a
// group holds two heads of 16).
template <int HD> struct KSteps { static constexpr int value = HD == 2 * kD ? 4 : 2; };

// Split-term operands (three bf16 terms, each the round-to-nearest bf16 of
// what the previous ones left, remainders exact) of one 32-row block of a
// head-dim HD state S for the matrix cores, K-steps of 16: lane (g, i) gets
// A[i][16 ks + 8 g + e] in out[ks][sp] (element e), with
//   natural:    A[i][kk] = S[row(i)][kk]
//   transposed: A[i][kk] = S[kk][row(i)]
// head(r) points at head r's HD x (HD + 1) state.
//   HD = 32: head grp, row(i) = i.
//   HD = 64: head grp, row(i) = 32 half + i, kk over all 64 features (four
//            K-steps).
//   HD = 16: heads 2 grp (K-step 0) and 2 grp + 1 (K-step 1; zero when there
//            is none, grp's row then being a lone head) as one block-diagonal
//            matrix: K-step ks is nonzero in rows 16 ks .. 16 ks + 15 only.
template <int HD, typename HeadState>
__device__ __forceinline__ void state_operands(HeadState head, int grp, int half, int HR, int lane, bool transposed,
                                               u32x4 (&out)[KSteps<HD>::value][3], const float* kkscale = nullptr) {
    constexpr int KS = KSteps<HD>::value, SW = HD + 1;
    const int g = lane >> 5, i = lane & 31;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
        float x[8];
        if constexpr (HD == kD / 2) {
            const int hr = 2 * grp + ks;
            const bool on = hr < HR && (i >> 4) == ks;
            const float* S = head(min(hr, HR - 1));
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int kk = 8 * g + e, r = i & 15;
                x[e] = on ? (transposed ? S[kk * SW + r] : S[r * SW + kk]) : 0.f;
                if (kkscale) x[e] *= fabsf(kkscale[min(hr, HR - 1) * HD + kk]);
            }
        } else {
            const float* S = head(grp);
            const int ri = (HD == 2 * kD ? kD * half : 0) + i;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int kk = 16 * ks + 8 * g + e;
                x[e] = transposed ? S[kk * SW + ri] : S[ri * SW + kk];
                if (kkscale) x[e] *= fabsf(kkscale[grp * HD + kk]);
            }
        }
        split3_f32x8(x, out[ks]);
    }
}

// The apply kernels' operands of out^T = S^T f^T (state_operands, transposed)
// and the normaliser entries at this lane's features: z[8 ks + e] =
// S[16 ks + 8 g + e][HD] (HD = 16: of head 2 grp + ks, zero when there is none).
// With qscale (qk_norm: the per-channel scales of q, [HR][HD]) every entry of
// feature kk is multiplied by |qscale[head][kk]|, which moves the magnitude of
// the scale from the query onto the state.
template <int HD, typename HeadState>
__device__ __forceinline__ void apply_operands(HeadState head, int grp, int half, int HR, int lane,
                                               u32x4 (&sa)[KSteps<HD>::value][3],
                                               float (&z)[8 * KSteps<HD>::value], const float* qscale = nullptr) {
    constexpr int KS = KSteps<HD>::value, SW = HD + 1;
    const int g = lane >> 5;
    state_operands<HD>(head, grp, half, HR, lane, true, sa, qscale);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            if constexpr (HD == kD / 2) {
                const int hr = 2 * grp + ks;
                z[8 * ks + e] = hr < HR ? head(hr)[(8 * g + e) * SW + HD] : 0.f;
                if (qscale && hr < HR) z[8 * ks + e] *= fabsf(qscale[hr * HD + 8 * g + e]);
            } else {
                z[8 * ks + e] = head(grp)[(16 * ks + 8 * g + e) * SW + HD];
                if (qscale) z[8 * ks + e] *= fabsf(qscale[grp * HD + 16 * ks + 8 * g + e]);
            }
        }
}

// acc += A B over KS K-steps, B a 16-bit operand per K-step (bf16 exact;
// fp16 split exactly into two bf16 terms), A three split terms; small terms
// first.
template <bool F16, int KS>
__device__ __forceinline__ f32x16 mma_split_ks(const u32x4 (&A)[KS][3], const u32x4 (&b)[KS], f32x16 acc) {
    if constexpr (F16) {
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            u32x4 hi, lo;
#pragma unroll
            for (int d = 0; d < 4; ++d) {
                uint32_t h, l;
                float f0, f1;
                split_f16x2(b[ks][d], h, l, f0, f1);
                hi[d] = h;
                lo[d] = l;
            }
#pragma unroll
            for (int sp = 2; sp >= 0; --sp) acc = mfma_bf16(A[ks][sp], lo, acc);
#pragma unroll
            for (int sp = 2; sp >= 0; --sp) acc = mfma_bf16(A[ks][sp], hi, acc);
        }
    } else {
#pragma unroll
        for (int sp = 2; sp >= 0; --sp)
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) acc = mfma_bf16(A[ks][sp], b[ks], acc);
    }
    return acc;
}

// Writes a wave's 32 x 32 accumulator tile (row 8*(r/4) + 4g + r%4 of column
// i in register r of lane (g, i)) token-major through the wave's LDS tile, then
// stores whole rows: dst(t) is the output row of token tt + t.  Rows t >= n
// were computed from the clamped input row n - 1, so they hold exactly row
// n - 1's values: they are stored there again (the same values), which keeps
// the row stores unconditional.  Only the first ncols columns of each row are
// stored (16 for a 32-feature group that is a lone head of dim 16).
template <typename OutT, typename RowPtr>
__device__ __forceinline__ void store_tile(float* ot, const f32x16& acc, int lane, int n, RowPtr dst,
                                           int ncols = 32) {
    const int g = lane >> 5, i = lane & 31;
#pragma unroll
    for (int rr = 0; rr < 4; ++rr)
        *reinterpret_cast<f32x4*>(ot + i * kPitch + 8 * rr + 4 * g) =
            (f32x4){acc[4 * rr], acc[4 * rr + 1], acc[4 * rr + 2], acc[4 * rr + 3]};
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int s4 = 0; s4 < 4; ++s4) {
        const int r = 8 * s4 + (lane >> 3), cc = (lane & 7) * 4;
        const f32x4 x = *reinterpret_cast<const f32x4*>(ot + r * kPitch + cc);
        if (cc < ncols) store4(dst(min(r, n - 1)) + cc, x);
    }
    __builtin_amdgcn_wave_barrier();
}

// fp32 inputs: features 8g..8g+7 and 16+8g..16+8g+7 of an fp32 row (the B
// operand layout), 4 x 16 bytes.  Plain loads: each instruction reads a part
// of each line it touches, and a non-temporal load of part of a line does not
// keep the line for the loads of its other parts (such reads measured at
// half the bandwidth of plain ones); whole-line reads are non-temporal.  upper = false leaves features 16.. as zero
// without reading them (a 32-feature group that is a lone head of dim 16).
struct F32Operand {
    f32x4 x[4];
    __device__ __forceinline__ void load(const float* row, int g, bool upper = true) {
#pragma unroll
        for (int p = 0; p < 4; ++p)
            x[p] = (p < 2 || upper)
                       ? *reinterpret_cast<const f32x4*>(row + 16 * (p >> 1) + 8 * g + 4 * (p & 1))
                       : (f32x4){0.f, 0.f, 0.f, 0.f};
    }
    // the 8 values of half ks (features 16 ks + 8 g ..), optionally ReLU'd
    __device__ __forceinline__ void half(int ks, bool relu, float out[8]) const {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float t = x[2 * ks + (e >> 2)][e & 3];
            out[e] = relu ? relu_f32(t) : t;
        }
    }
    // bit j set when feature j of the token is > 0 (the partner lane, i + 32,
    // holds the other 16 features)
    __device__ __forceinline__ uint32_t positive(int g) const {
        uint32_t m = 0;
#pragma unroll
        for (int p = 0; p < 4; ++p)
#pragma unroll
            for (int e = 0; e < 4; ++e) m |= (uint32_t)(x[p][e] > 0.f) << (16 * (p >> 1) + 8 * g + 4 * (p & 1) + e);
        return m | (uint32_t)__shfl_xor((int)m, 32);
    }
};

// The three truncation terms of half ks of an fp32 operand, optionally ReLU'd.
__device__ __forceinline__ void split_half(const F32Operand& b, int ks, bool relu, u32x4 t[3]) {
    float x[8];
    b.half(ks, relu, x);
    split3_trunc_f32x8(x, t);
}

// acc += A B for one K-step of 16 features, A and B both as three bf16 terms
// (index 0 the largest): the products of terms i + j <= 2, smallest first;
// the others lie below 2^-24 of the product and are dropped.
__device__ __forceinline__ f32x16 mma_terms(const u32x4 A[3], const u32x4 t[3], f32x16 acc) {
    acc = mfma_bf16(A[0], t[2], acc);
    acc = mfma_bf16(A[1], t[1], acc);
    acc = mfma_bf16(A[2], t[0], acc);
    acc = mfma_bf16(A[0], t[1], acc);
    acc = mfma_bf16(A[1], t[0], acc);
    acc = mfma_bf16(A[0], t[0], acc);
    return acc;
}

// acc += A B over 32 features with A given as three split terms (index 0 the
// largest) and B as an fp32 operand split here into three truncation terms.
__device__ __forceinline__ f32x16 mma_split3(const u32x4 A[2][3], const F32Operand& b, bool relu, f32x16 acc) {
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
        u32x4 t[3];
        split_half(b, ks, relu, t);
        acc = mma_terms(A[ks], t, acc);
    }
    return acc;
}

// ------------------------------------------------------------------ transposing LDS gathers
// Operand of v_mfma_f32_32x32x16 with tokens as the reduction dimension, from
// a token-major LDS tile of 16-bit elements (`pitch` per row): lane (g, m)
// gets tile[row0 + 8 g + e][col0 + m], e = 0..7, packed in pairs.
// ds_read_b64_tr_b16 works on groups of 16 lanes: lane r of a group supplies
// the address of 4 consecutive elements (its "row" r), and lane j receives
// element j % 4 of rows j / 4 + 4 q, q = 0..3.  Row r here is tile row
// row0 + 8 g + r / 4 (+ 4 for the second read), columns col0 + 16 h + 4 (r % 4)
// .. + 3, with g and h the group's halves of the wave and of the 32 columns.
// Addresses must be 8-byte aligned (pitch and col0 multiples of 4).
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
__device__ __forceinline__ u32x4 gather_tokens_t16(const uint16_t* tile, int pitch, int row0, int col0, int lane) {
    const int grp = lane >> 4, r = lane & 15;
    const uint16_t* p = tile + (row0 + 8 * (grp >> 1) + (r >> 2)) * pitch + col0 + 16 * (grp & 1) + 4 * (r & 3);
    const s16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)p);
    const s16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p + 4 * pitch));
    const u32x2 a2 = __builtin_bit_cast(u32x2, a), b2 = __builtin_bit_cast(u32x2, b);
    return (u32x4){a2[0], a2[1], b2[0], b2[1]};
}

// ------------------------------------------------------------------ 16-bit head-pair output lines
// With 16-bit outputs one head's row is half a 128-byte line.  The two waves
// of a head pair therefore write their tiles into one shared LDS tile
// [32 tokens][kPairRow] (head hh in elements 32 hh .. 32 hh + 31 of each row),
// and after a work-group barrier the rows are stored as whole lines.
constexpr int kPairRow = 68;   // 16-bit elements per row: 64 + 4 (136 bytes) spreads the banks

// acc of lane (g, i): token i, features 8 (r / 4) + 4 g + r % 4, rounded to
// OutT (nearest-even) into head hh's half of the pair tile.
template <typename OutT>
__device__ __forceinline__ void put_pair_tile(uint16_t* ct, const f32x16& acc, int lane, int hh) {
    const int g = lane >> 5, i = lane & 31;
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
        f32x4 x = {acc[4 * rr], acc[4 * rr + 1], acc[4 * rr + 2], acc[4 * rr + 3]};
        uint32_t p0, p1;
        if constexpr (std::is_same<OutT, _Float16>::value) {
            // pin the fp32 values: otherwise a multiply that produced them and
            // the narrowing can fuse into one mixed-precision FMA that rounds
            // once, and the result would no longer be the fp32 value rounded
#pragma unroll
            for (int e = 0; e < 4; ++e) asm volatile("" : "+v"(x[e]));
            p0 = __builtin_bit_cast(uint16_t, (_Float16)x[0]) | ((uint32_t)__builtin_bit_cast(uint16_t, (_Float16)x[1]) << 16);
            p1 = __builtin_bit_cast(uint16_t, (_Float16)x[2]) | ((uint32_t)__builtin_bit_cast(uint16_t, (_Float16)x[3]) << 16);
        } else {
            p0 = (uint32_t)f32_to_bf16(x[0]) | ((uint32_t)f32_to_bf16(x[1]) << 16);
            p1 = (uint32_t)f32_to_bf16(x[2]) | ((uint32_t)f32_to_bf16(x[3]) << 16);
        }
        *reinterpret_cast<u32x2*>(ct + i * kPairRow + hh * 32 + 8 * rr + 4 * g) = (u32x2){p0, p1};
    }
}

// Rows r0 .. r0 + 15 of a pair tile as whole lines: 8 lanes x 16 bytes per
// row; dst(r) points at the head pair's first element of row r's token; only
// the first nchunk 16-byte chunks of each row are written (4 per head that
// exists).
template <typename OutT, typename RowPtr>
__device__ __forceinline__ void store_pair_rows(const uint16_t* ct, int lane, int r0, int nchunk, RowPtr dst) {
#pragma unroll
    for (int k8 = 0; k8 < 2; ++k8) {
        const int r = r0 + 8 * k8 + (lane >> 3), chunk = lane & 7;
        const u32x4 x = *reinterpret_cast<const u32x4*>(ct + r * kPairRow + chunk * 8);
        if (chunk < nchunk) __builtin_nontemporal_store(x, reinterpret_cast<u32x4*>(dst(r) + chunk * 8));
    }
}

}  // namespace sana
