// gfx950 kernels of the LiteLA forward (ReLU-kernel linear self-attention).
//
// The operator ("Sana: the autoencoder does more of the work than the linear
// attention", section "What LiteLA actually computes"): per (batch, head) a
// D x (D+1) state S = phi(K)^T [V | 1] with phi = ReLU, then
// out_i = phi(q_i) S[:, :D] / (phi(q_i) S[:, D] + eps), all in fp32.
// The pages compute it with two library matmuls on a ones-padded copy of V;
// here it is three kernels on one stream and nothing is padded or copied:
//
//   1. state  (k_state_partial_*) - each work-group reduces one chunk of tokens
//      of one head pair into a partial state; ReLU and the ones column are fused
//      into the reduction.  bf16 inputs use v_mfma_f32_32x32x16_bf16 with the
//      tokens as the reduction dimension (bf16 x bf16 products are exact in
//      fp32); K/V tiles are staged through LDS to turn the token-major HBM rows
//      into token-packed matrix operands.
//   2. merge  (k_merge) - one thread per (b, h, state entry) sums the partials
//      in a fixed order (deterministic, no atomics).  For the block-causal
//      operator it also forms the inclusive prefix over blocks ("cumulative
//      statistics per temporal block", "How Linear Attention Improves
//      Efficiency in DiT for High-Resolution Images", section "Video
//      Generation and Constant-Memory KV Cache").
//   3. apply  (k_apply_*) - q rows go straight from HBM into a matrix operand
//      (the feature axis is already contiguous) and the numerators come from
//      the same MFMA against three bf16 split terms of S, which reproduce the
//      fp32 state to ~2^-24; the normaliser is an fp32 dot product on the
//      vector unit.  Both keep fp32 accuracy, as the pages' fp32 attention
//      policy asks.
//
// fp16 inputs take the same matrix-core kernels (products of fp16 values are
// exact in fp32 as well); in the apply kernel each ReLU(q) element is split
// exactly into two bf16 terms, so the state side stays the bf16 split.  fp32
// inputs (head dim 32) split K, V and q into three bf16 terms each
// (k_state_partial_mfma_f32 and the fp32 branch of k_apply_mfma).  Head dims
// 16 and 64 run the same kernels on 32-feature groups of the token row.  The
// vector kernels (k_*_valu) are a second implementation for cross-checks.
#include "linattn_device.h"

#include <type_traits>

namespace sana {
namespace {

// ------------------------------------------------------------------ state, bf16, MFMA
// LDS tile: [tensor K|V][head 0|1][token 0..63][32 x bf16]; the second head's
// rows are shifted by 64 bytes so that a 16-byte write from each head of one
// token lands in different banks.
constexpr int kPieces = kStateTile / 32;            // 16-byte pieces per thread per tensor
constexpr int kHeadStride = kStateTile * 64 + 64;   // bytes
constexpr int kTensorStride = 2 * kHeadStride;

static_assert(2 * kTensorStride >= 2 * 2 * 16 * 64 * (int)sizeof(float), "reduction area exceeds the LDS tile");

// Head dim 16: the diagonal 16 x 16 blocks of group grp's 32 x 32 sums (this
// wave's accumulators plus the other token half's, staged in red as
// [head][V|O][16][64]) are the states of heads 2 grp and 2 grp + 1, written
// when those heads exist.  Rows 0..15 (r < 8) are the first head's, 16..31
// the second's; the lanes of columns of the same half hold that head's state.
__device__ __forceinline__ void write_diag16(float* part, const float* red, const f32x16& accV, const f32x16& accO,
                                             int b, int HR, int P, int p, int grp, int hh, int lane) {
    constexpr int W16 = kD / 2 + 1;
    const int g = lane >> 5, j = lane & 31;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        const int half = r >> 3, head = 2 * grp + half;
        if ((j >> 4) != half || head >= HR) continue;
        const int row = 8 * ((r >> 2) & 1) + 4 * g + (r & 3);
        float* dst = part + (((size_t)b * HR + head) * P + p) * (kD / 2 * W16);
        dst[row * W16 + (j & 15)] = accV[r] + red[((hh * 2 + 0) * 16 + r) * 64 + lane];
        if ((j & 15) == 0) dst[row * W16 + kD / 2] = accO[r] + red[((hh * 2 + 1) * 16 + r) * 64 + lane];
    }
}

// grid.x = (b * HP + hp) * P + p; one work-group = one chunk of one head pair.
// Wave w reduces head (w & 1) over token half (w >> 1) of each 64-token tile.
// K and V are read once, so their loads are non-temporal.
//
// Other head dims HD reuse the tiles, which only see a token row as 32-feature
// groups ("heads" here: H of them, HP pairs; HR real heads, rows of HR * HD
// elements, pieces past the row read as zero):
//  - HD = 64: a head is a pair of groups.  Its 64 x 65 state is four 32 x 32
//    blocks: wave w accumulates block (K group w & 1, V group w >> 1) over all
//    tokens of each tile, the waves of V group 0 also the ones column of their
//    K group.
//  - HD = 16: a group holds two heads.  The group's 32 x 32 product is formed
//    as for HD = 32 and only its two diagonal 16 x 16 blocks (each head's keys
//    against its own values) are kept.
template <bool F16, int HD>
__global__ __launch_bounds__(kThreads) void k_state_partial_mfma(
    const uint16_t* __restrict__ k, const uint16_t* __restrict__ v, float* __restrict__ part,
    int N, int H, int HP, int HR, int L, int cpb, int P, int chunk, Strides sk, Strides sv) {
    constexpr bool D64 = HD == 2 * kD;
    __shared__ __attribute__((aligned(16))) uint8_t lds[2 * kTensorStride];

    const int p = blockIdx.x % P;
    const int bhp = blockIdx.x / P;
    const int hp = bhp % HP, b = bhp / HP;
    const int h0 = 2 * hp;
    const int nh = min(2, H - h0);
    const ChunkRange cr = chunk_range(p, cpb, chunk, L, N);

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int hh = wave & 1, th = wave >> 1;

    // Global -> register assignment: 16-byte piece id = tid + 256 i; piece
    // (tok, head, part) covers features 8*part..8*part+7 of one head of one
    // token, so a wave reads 8 whole 128-byte rows (both heads of 8 tokens).
    u32x4 rk[kPieces], rv[kPieces];
    auto load_tile = [&](int t0) {
#pragma unroll
        for (int i = 0; i < kPieces; ++i) {
            const int pc = tid + kThreads * i;
            const int part_ = pc & 3, hd = (pc >> 2) & 1, tok = pc >> 3;
            const int n = t0 + tok;
            const int col = (h0 + hd) * kD + part_ * 8;
            if (n < cr.c1 && col < HR * HD) {
                rk[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(k + (b * sk.b + n * sk.n + col)));
                rv[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(v + (b * sv.b + n * sv.n + col)));
            } else {
                rk[i] = (u32x4){0u, 0u, 0u, 0u};
                rv[i] = (u32x4){0u, 0u, 0u, 0u};
            }
        }
    };

    f32x16 accV = {}, accO = {};
    constexpr uint32_t kOne2 = F16 ? 0x3c003c00u : 0x3f803f80u;   // 1.0 in both halves
    const u32x4 ones = {kOne2, kOne2, kOne2, kOne2};
    const int g = lane >> 5, j = lane & 31;

    if (cr.c0 < cr.c1) load_tile(cr.c0);
    for (int t0 = cr.c0; t0 < cr.c1; t0 += kStateTile) {
        __syncthreads();   // the previous tile has been consumed
#pragma unroll
        for (int i = 0; i < kPieces; ++i) {
            const int pc = tid + kThreads * i;
            const int part_ = pc & 3, hd = (pc >> 2) & 1, tok = pc >> 3;
            const int o = hd * kHeadStride + tok * 64 + part_ * 16;
            *reinterpret_cast<u32x4*>(lds + o) = relu_bf16x8(rk[i]);
            *reinterpret_cast<u32x4*>(lds + kTensorStride + o) = rv[i];
        }
        __syncthreads();
        if (t0 + kStateTile < cr.c1) load_tile(t0 + kStateTile);   // in flight during the MFMAs

        if constexpr (D64) {
            const uint16_t* Kt = reinterpret_cast<const uint16_t*>(lds + hh * kHeadStride);
            const uint16_t* Vt = reinterpret_cast<const uint16_t*>(lds + kTensorStride + th * kHeadStride);
            // a token row of one half is 32 contiguous 16-bit values (pitch 32)
            static_assert(kHeadStride % 8 == 0, "transposing reads need 8-byte aligned rows");
#pragma unroll
            for (int st = 0; st < kStateTile / 16; ++st) {
                const u32x4 a = gather_tokens_t16(Kt, kD, 16 * st, 0, lane);   // lane (g, j): tokens 16 st + 8 g + e, feature j
                const u32x4 bv = gather_tokens_t16(Vt, kD, 16 * st, 0, lane);
                accV = mfma16<F16>(a, bv, accV);
                if (th == 0) accO = mfma16<F16>(a, ones, accO);
            }
            continue;
        }
        const uint16_t* Kt = reinterpret_cast<const uint16_t*>(lds + hh * kHeadStride);
        const uint16_t* Vt = reinterpret_cast<const uint16_t*>(lds + kTensorStride + hh * kHeadStride);
#pragma unroll
        for (int st = 0; st < kStateTile / 32; ++st) {
            // 16 tokens per MFMA; element e of lane (g, j) is token tb + 2e + g,
            // the same token for the K (row j) and the V (column j) operand.
            const int tb = (kStateTile / 2) * th + 16 * st;
            u32x4 a, bv;
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const int r0 = (tb + 4 * t + g) * 32 + j;
                const int r1 = r0 + 2 * 32;
                a[t] = (uint32_t)Kt[r0] | ((uint32_t)Kt[r1] << 16);
                bv[t] = (uint32_t)Vt[r0] | ((uint32_t)Vt[r1] << 16);
            }
            accV = mfma16<F16>(a, bv, accV);
            accO = mfma16<F16>(a, ones, accO);
        }
    }

    if constexpr (D64) {
        // each wave owns its block over the whole chunk
        constexpr int W64 = 2 * kD + 1;
        float* dst = part + (((size_t)b * HP + hp) * P + p) * (2 * kD * W64);
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int row = kD * hh + 8 * (r >> 2) + 4 * g + (r & 3);
            dst[row * W64 + kD * th + j] = accV[r];
            if (th == 0 && j == 0) dst[row * W64 + 2 * kD] = accO[r];
        }
        return;
    }
    // Combine the two token halves of each head in a fixed order, then write.
    __syncthreads();
    float* red = reinterpret_cast<float*>(lds);   // [head][V|O][16][64] floats = 16 KiB
    if (th == 1) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            red[((hh * 2 + 0) * 16 + r) * 64 + lane] = accV[r];
            red[((hh * 2 + 1) * 16 + r) * 64 + lane] = accO[r];
        }
    }
    __syncthreads();
    if constexpr (HD == kD / 2) {
        if (th == 0 && hh < nh) write_diag16(part, red, accV, accO, b, HR, P, p, h0 + hh, hh, lane);
        return;
    }
    if (th == 0 && hh < nh) {
        float* dst = part + (((size_t)b * H + h0 + hh) * P + p) * kStateFloats;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            // accumulator r of lane (g, c) holds row 8*(r/4) + 4*g + r%4, column c
            const int row = 8 * (r >> 2) + 4 * g + (r & 3);
            dst[row * kW + j] = accV[r] + red[((hh * 2 + 0) * 16 + r) * 64 + lane];
            if (j == 0) dst[row * kW + kD] = accO[r] + red[((hh * 2 + 1) * 16 + r) * 64 + lane];
        }
    }
}

// ------------------------------------------------------------------ state, matrix cores, fp32 inputs
// grid.x = (b * HP + hp) * P + p, as above.  fp32 K and V: each 64-token tile
// of both heads is loaded as 32-byte pieces (8 features of one head of one
// token; 8 threads read a token's whole 256-byte head-pair row), K through
// ReLU, and each value is split by truncation into three bf16 terms
// (t1 + t2 + t3 = x exactly) staged in LDS as 16-bit term tiles.  Per 16
// tokens each wave gathers, with transposing LDS reads, 8 tokens of one
// feature per lane and accumulates
//   S_v += a_i^T v_j over the term pairs i + j <= 4 (1-based; the dropped
//          products are below 2^-24 of the exact one)
//   S_1 += (a_1 + a_2 + a_3)^T 1 (exact)
// Wave w: head w & 1, token half w >> 1 of each tile.  Head dims 16 and 64
// work on 32-feature groups as the 16-bit kernel does (HD = 64: wave w owns
// state block (K group w & 1, V group w >> 1) over all tokens; HD = 16: the
// diagonal blocks of each group are kept).
constexpr int kF32Tile = 64 * kD;   // 16-bit elements of one term tile [token][feature] of one head

// The same kernel serves the qk_norm prologue (QK) for every input type: a key
// row of head h becomes r_n ReLU(sign(gamma_k) k_n), r_n = 1 / sqrt(mean(k_n^2) +
// norm_eps) over the head's HD features, formed in fp32 and split into three
// terms like an fp32 input (the merge multiplies row j of the state by
// |gamma_k[h][j]|, which completes phi(gamma_k k_n r_n)).  16-bit values are
// exact as bf16 terms (a bf16 value is one term, an fp16 value two), so only
// the products with nonzero terms of V are formed.
template <typename InT> struct Piece;   // 8 consecutive features of one token row
template <> struct Piece<float> {
    f32x4 x[2];
    __device__ __forceinline__ void load(const float* p) {
        x[0] = reinterpret_cast<const f32x4*>(p)[0];   // plain loads: each reads half of a line (see F32Operand)
        x[1] = reinterpret_cast<const f32x4*>(p)[1];
    }
    __device__ __forceinline__ void zero() { x[0] = x[1] = (f32x4){0.f, 0.f, 0.f, 0.f}; }
    __device__ __forceinline__ void get(float f[8]) const {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            f[e] = x[0][e];
            f[4 + e] = x[1][e];
        }
    }
};
template <> struct Piece<uint16_t> {
    u32x4 x;
    __device__ __forceinline__ void load(const uint16_t* p) {
        x = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
    }
    __device__ __forceinline__ void zero() { x = (u32x4){0u, 0u, 0u, 0u}; }
    __device__ __forceinline__ void get(float f[8]) const {
#pragma unroll
        for (int d = 0; d < 4; ++d) {
            const uint32_t w = x[d];
            f[2 * d] = lo_bf16(w);
            f[2 * d + 1] = hi_bf16(w);
        }
    }
};
template <> struct Piece<_Float16> {
    u32x4 x;
    __device__ __forceinline__ void load(const _Float16* p) {
        x = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
    }
    __device__ __forceinline__ void zero() { x = (u32x4){0u, 0u, 0u, 0u}; }
    __device__ __forceinline__ void get(float f[8]) const {
#pragma unroll
        for (int d = 0; d < 4; ++d) {
            const uint32_t w = x[d];
            f[2 * d] = f16_to_f32((uint16_t)(w & 0xffffu));
            f[2 * d + 1] = f16_to_f32((uint16_t)(w >> 16));
        }
    }
};

template <int HD, typename InT = float, bool QK = false>
__global__ __launch_bounds__(kThreads) void k_state_partial_mfma_f32(
    const InT* __restrict__ k, const InT* __restrict__ v, float* __restrict__ part,
    int N, int H, int HP, int HR, int L, int cpb, int P, int chunk, Strides sk, Strides sv,
    const float* __restrict__ gk, float norm_eps) {
    // terms of a V value: bf16 1, fp16 2 (8 + 3 significant bits), fp32 3
    constexpr int VT = std::is_same<InT, uint16_t>::value ? 1 : std::is_same<InT, _Float16>::value ? 2 : 3;
    // term tiles [term][head]: K three terms, V as many as its type needs
    // (24 + 8, 16 or 24 KB), so that 16-bit V leaves room for a fourth
    // work-group per CU
    __shared__ __attribute__((aligned(16))) uint16_t ldk[3][2][kF32Tile];
    __shared__ __attribute__((aligned(16))) uint16_t ldv[VT][2][kF32Tile];

    const int p = blockIdx.x % P;
    const int bhp = blockIdx.x / P;
    const int hp = bhp % HP, b = bhp / HP;
    const int h0 = 2 * hp;
    const int nh = min(2, H - h0);
    const ChunkRange cr = chunk_range(p, cpb, chunk, L, N);

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int hh = wave & 1, th = wave >> 1;
    const int g = lane >> 5, j = lane & 31;

    // piece pc = tid + 256 i: part (pc & 3) = features 8 part .. + 7, head
    // (pc >> 2) & 1, token pc >> 3; a thread's part and group are the same for
    // both of its pieces
    const int part0 = tid & 3, grp0 = (tid >> 2) & 1;
    Piece<InT> rk[2], rv[2];
    auto load_tile = [&](int t0) {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int tok = (tid >> 3) + 32 * i;
            const int n = t0 + tok;
            const int col = (h0 + grp0) * kD + part0 * 8;
            if (n < cr.c1 && col < HR * HD) {
                rk[i].load(k + (b * sk.b + n * sk.n + col));
                rv[i].load(v + (b * sv.b + n * sv.n + col));
            } else {
                rk[i].zero();
                rv[i].zero();
            }
        }
    };
    // qk_norm: the sign of gamma_k at this thread's 8 features, as sign bits
    uint32_t kneg = 0;
    if constexpr (QK) {
        int head, f0;   // the head and first feature this thread's pieces belong to
        if constexpr (HD == 2 * kD) {
            head = hp;
            f0 = kD * grp0 + 8 * part0;
        } else if constexpr (HD == kD) {
            head = h0 + grp0;
            f0 = 8 * part0;
        } else {
            head = 2 * (h0 + grp0) + (part0 >> 1);
            f0 = 8 * (part0 & 1);
        }
        if (head < HR)
#pragma unroll
            for (int e = 0; e < 8; ++e) kneg |= (uint32_t)(gk[head * HD + f0 + e] < 0.f) << e;
    }

    f32x16 accV = {}, accO = {};
    const u32x4 ones = {0x3f803f80u, 0x3f803f80u, 0x3f803f80u, 0x3f803f80u};   // bf16 1.0 pairs

    if (cr.c0 < cr.c1) load_tile(cr.c0);
    for (int t0 = cr.c0; t0 < cr.c1; t0 += 64) {
        __syncthreads();   // the previous tile has been consumed
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int tok = (tid >> 3) + 32 * i;
            float a[8], w[8];
            rk[i].get(a);
            rv[i].get(w);
            if constexpr (QK) {
                // r_n over the head's features: 4 threads hold a 32-feature
                // group row, 8 (both groups) a head of 64, 2 a head of 16
                float ss = 0.f;
#pragma unroll
                for (int e = 0; e < 8; ++e) ss = fmaf(a[e], a[e], ss);
                ss += __shfl_xor(ss, 1);
                if constexpr (HD >= kD) ss += __shfl_xor(ss, 2);
                if constexpr (HD == 2 * kD) ss += __shfl_xor(ss, 4);
                const float r = 1.0f / sqrtf(ss * (1.0f / HD) + norm_eps);
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const uint32_t bits = __builtin_bit_cast(uint32_t, a[e]) ^ (((kneg >> e) & 1u) << 31);
                    a[e] = r * relu_f32(__builtin_bit_cast(float, bits));
                }
            } else {
#pragma unroll
                for (int e = 0; e < 8; ++e) a[e] = relu_f32(a[e]);
            }
            u32x4 ta[3], tv[3];
            split3_trunc_f32x8(a, ta);
            split3_trunc_f32x8(w, tv);
            const int o = tok * kD + part0 * 8;
#pragma unroll
            for (int t = 0; t < 3; ++t) {
                *reinterpret_cast<u32x4*>(&ldk[t][grp0][o]) = ta[t];
                if (t < VT) *reinterpret_cast<u32x4*>(&ldv[t][grp0][o]) = tv[t];
            }
        }
        __syncthreads();
        if (t0 + 64 < cr.c1) load_tile(t0 + 64);   // in flight during the MFMAs

        constexpr bool D64 = HD == 2 * kD;
#pragma unroll
        for (int st = 0; st < (D64 ? 4 : 2); ++st) {
            const int tb = D64 ? 16 * st : 32 * th + 16 * st;   // first token of this K-step in the tile
            u32x4 ta[3], tv[3];
#pragma unroll
            for (int t = 0; t < 3; ++t) {
                ta[t] = gather_tokens_t16(ldk[t][hh], kD, tb, 0, lane);   // lane (g, j): tokens tb + 8g + e, feature j
                if (t < VT) tv[t] = gather_tokens_t16(ldv[t][D64 ? th : hh], kD, tb, 0, lane);   // lane (g, c): tokens tb + 8g + e, channel c
            }
            // term pairs with i + j <= 2, smallest products first
            accV = mfma_bf16(ta[2], tv[0], accV);
            if constexpr (VT > 1) accV = mfma_bf16(ta[1], tv[1], accV);
            if constexpr (VT > 2) accV = mfma_bf16(ta[0], tv[2], accV);
            accV = mfma_bf16(ta[1], tv[0], accV);
            if constexpr (VT > 1) accV = mfma_bf16(ta[0], tv[1], accV);
            accV = mfma_bf16(ta[0], tv[0], accV);
            if (!D64 || th == 0) {
                accO = mfma_bf16(ta[2], ones, accO);
                accO = mfma_bf16(ta[1], ones, accO);
                accO = mfma_bf16(ta[0], ones, accO);
            }
        }
    }

    if constexpr (HD == 2 * kD) {
        // each wave owns its block over the whole chunk
        constexpr int W64 = 2 * kD + 1;
        float* dst = part + (((size_t)b * HP + hp) * P + p) * (2 * kD * W64);
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int row = kD * hh + 8 * (r >> 2) + 4 * g + (r & 3);
            dst[row * W64 + kD * th + j] = accV[r];
            if (th == 0 && j == 0) dst[row * W64 + 2 * kD] = accO[r];
        }
        return;
    }
    // Combine the two token halves of each head in a fixed order, then write.
    __syncthreads();
    static_assert(sizeof(ldk) >= 2 * 2 * 16 * 64 * sizeof(float), "reduction area exceeds the K term tiles");
    float* red = reinterpret_cast<float*>(&ldk[0][0][0]);   // [head][V|O][16][64] floats = 16 KiB
    if (th == 1) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            red[((hh * 2 + 0) * 16 + r) * 64 + lane] = accV[r];
            red[((hh * 2 + 1) * 16 + r) * 64 + lane] = accO[r];
        }
    }
    __syncthreads();
    if constexpr (HD == kD / 2) {
        if (th == 0 && hh < nh) write_diag16(part, red, accV, accO, b, HR, P, p, h0 + hh, hh, lane);
        return;
    }
    if (th == 0 && hh < nh) {
        float* dst = part + (((size_t)b * H + h0 + hh) * P + p) * kStateFloats;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            // accumulator r of lane (g, c) holds row 8*(r/4) + 4*g + r%4, column c
            const int row = 8 * (r >> 2) + 4 * g + (r & 3);
            dst[row * kW + j] = accV[r] + red[((hh * 2 + 0) * 16 + r) * 64 + lane];
            if (j == 0) dst[row * kW + kD] = accO[r] + red[((hh * 2 + 1) * 16 + r) * 64 + lane];
        }
    }
}

// ------------------------------------------------------------------ state, vector path
// grid.x = (b * H + h) * P + p.  Thread t owns state entries t, t+256, ...
// Head dim DD (16, 32 or 64): a state is DD x (DD + 1).
// With gk (qk_norm) each key row is RMS-normalised over its DD features,
// scaled by gamma_k and passed through ReLU here, straight from the definition.
template <typename InT, int DD>
__global__ __launch_bounds__(kThreads) void k_state_partial_valu(
    const InT* __restrict__ k, const InT* __restrict__ v, float* __restrict__ part,
    int N, int H, int L, int cpb, int P, int chunk, Strides stk, Strides stv, const float* __restrict__ gk,
    float norm_eps) {
    constexpr int WW = DD + 1, SF = DD * WW, M = (SF + kThreads - 1) / kThreads;
    __shared__ float sa[kValuTile][DD + 1];   // ReLU(k) tile
    __shared__ float sv[kValuTile][WW];       // [v | 1] tile
    __shared__ float rr[kValuTile];           // qk_norm: 1 / rms of each key row

    const int p = blockIdx.x % P;
    const int bh = blockIdx.x / P;
    const int h = bh % H, b = bh / H;
    const ChunkRange cr = chunk_range(p, cpb, chunk, L, N);
    const int tid = threadIdx.x;

    float acc[M] = {};
    for (int t0 = cr.c0; t0 < cr.c1; t0 += kValuTile) {
        __syncthreads();
        for (int e = tid; e < kValuTile * DD; e += kThreads) {
            const int tok = e / DD, jj = e % DD;
            const int n = t0 + tok;
            float kk = 0.f, vv = 0.f;
            if (n < cr.c1) {
                const long long col = (long long)h * DD + jj;
                kk = load_in(k, b * stk.b + n * stk.n + col);
                vv = load_in(v, b * stv.b + n * stv.n + col);
            }
            sa[tok][jj] = gk ? kk : (kk > 0.f ? kk : 0.f);
            sv[tok][jj] = vv;
        }
        if (tid < kValuTile) sv[tid][DD] = 1.f;
        __syncthreads();
        if (gk) {
            if (tid < kValuTile) {
                float ss = 0.f;
                for (int jj = 0; jj < DD; ++jj) ss += sa[tid][jj] * sa[tid][jj];
                rr[tid] = 1.0f / sqrtf(ss / DD + norm_eps);
            }
            __syncthreads();
            for (int e = tid; e < kValuTile * DD; e += kThreads) {
                const int tok = e / DD, jj = e % DD;
                const float x = gk[h * DD + jj] * sa[tok][jj] * rr[tok];
                sa[tok][jj] = x > 0.f ? x : 0.f;
            }
            __syncthreads();
        }
#pragma unroll
        for (int m = 0; m < M; ++m) {
            const int o = tid + kThreads * m;
            if (o < SF) {
                const int jj = o / WW, c = o - jj * WW;
                float s = acc[m];
                for (int tok = 0; tok < kValuTile; ++tok) s += sa[tok][jj] * sv[tok][c];
                acc[m] = s;
            }
        }
    }
    float* dst = part + ((size_t)bh * P + p) * SF;
#pragma unroll
    for (int m = 0; m < M; ++m) {
        const int o = tid + kThreads * m;
        if (o < SF) dst[o] = acc[m];
    }
}

// ------------------------------------------------------------------ merge / block scan
// grid.x = (b * H + h) * groups + m, groups = ceil(SF / kMergeThreads); thread
// t owns state entry e = m * kMergeThreads + t of the SF = D (D + 1) entries.
// Starting from the carried state (or zero), for each block it sums that
// block's chunk partials (in groups of 8 added as a fixed pairwise tree, the
// groups in order), and adds the block sum to the running state (inclusive
// prefix over blocks); the final running state is the carried state out.
// The kernel is a few load round trips long, so the loads of up to 16
// partials are issued together.  state_in and state_out may be the same
// array: each thread reads its own entry before it writes it.
__device__ __forceinline__ float tree8(const float* x) {
    return ((x[0] + x[1]) + (x[2] + x[3])) + ((x[4] + x[5]) + (x[6] + x[7]));
}

__global__ __launch_bounds__(kMergeThreads) void k_merge(
    const float* __restrict__ part, float* __restrict__ state, const float* state_in, float* state_out,
    int NB, int cpb, int P, int SF, const float* __restrict__ gk, int H, int D) {
    const int groups = (SF + kMergeThreads - 1) / kMergeThreads;
    const size_t bh = blockIdx.x / groups;
    const int e = (blockIdx.x % groups) * kMergeThreads + threadIdx.x;
    if (e >= SF) return;
    // qk_norm: the partials hold sum_n r_n ReLU(sign(gamma_k) k_n) [v_n | 1];
    // row j of the state is that times |gamma_k[h][j]|
    const float gscale = gk ? fabsf(gk[(bh % H) * D + e / (D + 1)]) : 1.f;
    const float* src = part + bh * P * SF + e;
    float* dst = state + bh * NB * SF + e;
    float acc = state_in ? state_in[bh * SF + e] : 0.f;
    // Loads take clamped (always valid) indices and are unconditional, so a
    // thread's loads are all in flight before the first sum; entries past the
    // end are then replaced by zeros, or not stored.
    if (cpb == 1) {
        // one partial per block (the block-causal case): 16 blocks' loads at once
        for (int b0 = 0; b0 < NB; b0 += 16) {
            float x[16];
#pragma unroll
            for (int i = 0; i < 16; ++i) x[i] = src[(size_t)min(b0 + i, NB - 1) * SF];
#pragma unroll
            for (int i = 0; i < 16; ++i) asm volatile("" : "+v"(x[i]));   // all 16 in flight first
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                if (b0 + i < NB) {
                    acc += gscale * (0.f + x[i]);   // the block sum of one partial, as the general path forms it
                    dst[(size_t)(b0 + i) * SF] = acc;
                }
            }
        }
    } else if (cpb <= 8 && NB > 1) {
        // each block: its chunk partials added as a fixed pairwise tree of 8
        // (zeros past cpb); the loads of 4 blocks in flight at once (a
        // streamed call has few blocks of few chunks each: 2 us less per
        // call of 4096 tokens; with one block the general path is faster)
        for (int b0 = 0; b0 < NB; b0 += 4) {
            float x[4][8];
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
                for (int c = 0; c < 8; ++c)
                    x[j][c] = src[((size_t)min(b0 + j, NB - 1) * cpb + min(c, cpb - 1)) * SF];
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
                for (int c = 0; c < 8; ++c) asm volatile("" : "+v"(x[j][c]));   // all in flight first
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                if (b0 + j < NB) {
#pragma unroll
                    for (int c = 0; c < 8; ++c) x[j][c] = c < cpb ? x[j][c] : 0.f;
                    acc += gscale * (0.f + tree8(x[j]));   // the block sum as the general path forms it
                    dst[(size_t)(b0 + j) * SF] = acc;
                }
            }
        }
    } else {
        // each block: its chunk partials in groups of 8 added as a fixed
        // pairwise tree, the groups in order
        for (int beta = 0; beta < NB; ++beta) {
            const float* blk = src + (size_t)beta * cpb * SF;
            float bs = 0.f;
            for (int s0 = 0; s0 < cpb; s0 += 16) {
                float x[16];
#pragma unroll
                for (int i = 0; i < 16; ++i) x[i] = blk[(size_t)min(s0 + i, cpb - 1) * SF];
                // (keeps the compiler from deferring the second group's loads
                // until the first group is summed)
#pragma unroll
                for (int i = 0; i < 16; ++i) asm volatile("" : "+v"(x[i]));
#pragma unroll
                for (int i = 0; i < 16; ++i) x[i] = s0 + i < cpb ? x[i] : 0.f;
                bs += tree8(x);
                if (s0 + 8 < cpb) bs += tree8(x + 8);
            }
            acc += gscale * bs;
            dst[(size_t)beta * SF] = acc;
        }
    }
    if (state_out) state_out[bh * SF + e] = acc;
}

// ------------------------------------------------------------------ apply, bf16, MFMA
// grid.x = (b * HP + hp) * (NB * tpb) + beta * tpb + tile.  Wave w handles head
// 2*hp + (w & 1) and every other 32-token sub-tile (w >> 1) of the work-group's
// token range, which never crosses a block boundary.
//
// Per sub-tile the wave forms the transposed product out^T = S^T f^T with
// f = ReLU(q): A = S^T as three bf16 split terms (built once per work-group
// from the fp32 state), B = 32 q rows straight from HBM (lane (g, i) holds
// features 8g..8g+7 and 16+8g..16+8g+7 of token i, the layout the operand
// needs).  Lane (g, i) then owns 16 numerators of token i (columns
// 8*(r/4) + 4g + r%4), so it computes token i's normaliser itself in fp32 from
// the same registers (half the features here, half from lane i + 32) and takes
// one reciprocal.  The normalised 32 x 32 tile goes through this wave's LDS so
// that every store instruction writes whole 128-byte output rows.
constexpr int kOutPitch = 36;   // floats per LDS output row: 32 + 4 keeps rows 16-byte aligned, no bank conflicts

// q is bf16 (InT uint16_t), fp16 or fp32.  A 16-bit q row half is one exact
// B operand (fp16: split exactly into two bf16 terms); an fp32 q is split by
// truncation into three bf16 terms and the products of S's and q's terms with
// i + j <= 4 (1-based) are summed (the dropped ones are below 2^-24 of the
// exact product).  Occupancy target 5 waves per SIMD (4 for fp16 and fp32 q,
// whose splits need more registers; 3 for head dim 64, 2 with fp32 q; one
// less with qk_norm).
//
// Other head dims HD (16-bit q) use the 32-feature groups of a token row as
// "heads" (H of them, HP pairs; HR real heads of rows HR * HD elements long):
//  - HD = 64: wave w computes output half w & 1 of head hp (columns 32 (w & 1)
//    .. + 31, stored as group 2 hp + (w & 1)), reducing over all 64 features
//    of q in four K-steps against the state's column half.
//  - HD = 16: group h holds heads 2h and 2h + 1; A is the block-diagonal
//    32 x 32 matrix of their two states (zero off the diagonal blocks), so the
//    product gives both heads' numerators, and each head takes its own
//    normaliser (K-step 0 is the first head's features, 1 the second's).
//
// qk_norm (QK): phi(gamma_q q_i rho_i), rho_i = 1 / rms of the head's row of
// q_i, equals rho_i |gamma_q| ReLU(sign(gamma_q) q_i); |gamma_q| goes onto the
// rows of S when its operands are built, the sign flip is exact on the bits,
// and rho_i cancels between numerator and normaliser except against eps, so
// the normaliser becomes den + eps * rms_i (rms_i from the same registers).
template <typename InT, int HD, bool QK>
constexpr int apply_waves_per_simd() {
    const int w = HD == 2 * kD ? (std::is_same<InT, float>::value ? 2 : 3) : std::is_same<InT, uint16_t>::value ? 5 : 4;
    return QK && w > 2 ? w - 1 : w;   // qk_norm keeps sign masks and sums of squares live as well
}

template <typename InT, typename OutT, int HD, bool QK = false>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(apply_waves_per_simd<InT, HD, QK>(), 8))) void k_apply_mfma(
    const InT* __restrict__ q, const float* __restrict__ state, OutT* __restrict__ out,
    int N, int H, int HP, int HR, int L, int NB, int tile, int tpb, float eps, Strides sq, Strides so,
    const float* __restrict__ gq, float norm_eps) {
    constexpr bool F16 = std::is_same<InT, _Float16>::value;
    constexpr bool F32 = std::is_same<InT, float>::value;
    constexpr bool D64 = HD == 2 * kD, D16 = HD == kD / 2;
    constexpr int KS = D64 ? 4 : 2;   // K-steps of 16 features
    constexpr int SW = HD + 1;        // state row
    constexpr int QW = F32 ? 2 * KS : KS;   // 16-byte pieces of a lane's q features (16 ks + 8 g .. + 7)
    __shared__ __attribute__((aligned(16))) float otile[4][32 * kOutPitch];   // fp32 out only

    const int per_unit = NB * tpb;
    const int tau = blockIdx.x % per_unit;
    const int bhp = blockIdx.x / per_unit;
    const int hp = bhp % HP, b = bhp / HP;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int hh = wave & 1, h = 2 * hp + hh;
    const int sub = wave >> 1;
    const int hs = min(h, H - 1);   // a missing second head works on the first (never stored)
    const int beta = tau / tpb, tib = tau - beta * tpb;
    const int blk0 = beta * L;
    const int blk1 = min(blk0 + L, N);
    const int t0 = blk0 + tib * tile;
    const int t1 = min(t0 + tile, blk1);
    if (t0 >= t1) return;

    const int g = lane >> 5, i = lane & 31;
    // A operand: lane (g, c = i), element e of (ks, split) = split term of
    // S[16 ks + 8 g + e][c]; sden: this lane's 8 KS normaliser entries.
    const int SF = HD * SW;
    auto head_state = [&](int hr) { return state + (((size_t)b * HR + hr) * NB + beta) * SF; };
    u32x4 sa[KS][3];
    float sden[8 * KS];
    apply_operands<HD>(head_state, D64 ? hp : hs, hh, HR, lane, sa, sden, QK ? gq : nullptr);
    // qk_norm: sign bits of gamma_q at this lane's features 16 ks + 8 g + e
    // (head dim 16: K-step ks is head 2 hs + ks, features 8 g + e)
    uint32_t qneg[KS] = {};
    if constexpr (QK) {
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const int hr = D64 ? hp : D16 ? 2 * hs + ks : hs;
            const int f0 = D16 ? 8 * g : 16 * ks + 8 * g;
            if (hr < HR)
#pragma unroll
                for (int e = 0; e < 8; ++e) qneg[ks] |= (uint32_t)(gq[hr * HD + f0 + e] < 0.f) << e;
        }
    }
    // the same as 16-bit sign bits of a packed operand
    auto neg16 = [&](int ks) {
        u32x4 m;
#pragma unroll
        for (int d = 0; d < 4; ++d) m[d] = (((qneg[ks] >> (2 * d)) & 1u) << 15) | (((qneg[ks] >> (2 * d + 1)) & 1u) << 31);
        return m;
    };

    // fp32 out: rows past the range read as zero and are not stored.  16-bit
    // out: they are clamped to the range's last row, so every load is
    // unconditional, and a clamped row's output equals the last row's (it is
    // stored there again, with the same bits).
    struct QRow {
        u32x4 x[QW];
    };
    const bool second = !D16 || 2 * hs + 1 < HR;   // head dim 16: group hs has a second head
    auto load_row = [&](const u32x4* src, QRow& r) {
        if constexpr (F32) {   // features 16 ks + 8g..8g+7 = src[4 ks .. 4 ks + 1]
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                const bool on = !D16 || ks == 0 || second;   // head dim 16: the second head only if it exists
                r.x[2 * ks] = on ? src[4 * ks] : (u32x4){0u, 0u, 0u, 0u};
                r.x[2 * ks + 1] = on ? src[4 * ks + 1] : (u32x4){0u, 0u, 0u, 0u};
            }
        } else if constexpr (D16) {   // the second head's features only if it exists
            r.x[0] = src[0];
            r.x[1] = second ? src[2] : (u32x4){0u, 0u, 0u, 0u};
        } else {               // features 16 ks + 8g..8g+7 = src[2 ks]
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) r.x[ks] = src[2 * ks];
        }
    };
    auto load_b = [&](int tt, QRow& r) {
        if constexpr (sizeof(OutT) == 4) {
            const int row = tt + i;
            if (row < t1) {
                load_row(reinterpret_cast<const u32x4*>(q + (b * sq.b + row * sq.n + (D64 ? 2 * hp : h) * kD + 8 * g)), r);
            } else {
#pragma unroll
                for (int c = 0; c < QW; ++c) r.x[c] = (u32x4){0u, 0u, 0u, 0u};
            }
        } else {
            const int row = min(tt + i, t1 - 1);
            load_row(reinterpret_cast<const u32x4*>(q + (b * sq.b + row * sq.n + (D64 ? 2 * hp : hs) * kD + 8 * g)), r);
        }
    };
    // normalised 32 x 32 output tile of one sub-tile: acc row 8 (r / 4) + 4 g + r % 4, column i
    auto compute = [&](const QRow& qr) -> f32x16 {
        f32x16 acc = {};
        float dp = 0.f, dp1 = 0.f;   // dp1: head dim 16, the group's second head
        float ss = 0.f, ss1 = 0.f;   // qk_norm: sums of squares of the row (ss1: second head of dim 16)
        if constexpr (F32) {
            // f = ReLU(q) in fp32 (features 16 ks + 8 g + e at f[8 ks + e])
            float f[8 * KS];
#pragma unroll
            for (int c = 0; c < QW; ++c)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    // through a scalar: bit_cast of a vector element expression
                    // reads the vector's first element with this compiler
                    uint32_t bits = qr.x[c][e];
                    if constexpr (QK) {
                        const float x = __builtin_bit_cast(float, bits);
                        float& t = (D16 && c >= 2) ? ss1 : ss;
                        t = fmaf(x, x, t);
                        bits ^= ((qneg[c >> 1] >> (4 * (c & 1) + e)) & 1u) << 31;
                    }
                    f[4 * c + e] = relu_f32(__builtin_bit_cast(float, bits));
                }
#pragma unroll
            for (int e = 0; e < 8 * KS; ++e) {
                float& t = (D16 && e >= 8) ? dp1 : dp;
                t = fmaf(f[e], sden[e], t);
            }
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                u32x4 fb[3];
                split3_trunc_f32x8(f + 8 * ks, fb);
                // term pairs (S, q) with i + j <= 4, smallest first
                acc = mfma_bf16(sa[ks][2], fb[0], acc);
                acc = mfma_bf16(sa[ks][1], fb[1], acc);
                acc = mfma_bf16(sa[ks][0], fb[2], acc);
                acc = mfma_bf16(sa[ks][1], fb[0], acc);
                acc = mfma_bf16(sa[ks][0], fb[1], acc);
                acc = mfma_bf16(sa[ks][0], fb[0], acc);
            }
        } else if constexpr (F16) {
            // one 16-feature step at a time (fewer live registers); the
            // normaliser takes the fp32 values as they are split
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                if constexpr (QK) {
                    float& t = (D16 && ks == 1) ? ss1 : ss;
#pragma unroll
                    for (int d = 0; d < 4; ++d) {
                        const uint32_t w = qr.x[ks][d];
                        const float x0 = f16_to_f32((uint16_t)(w & 0xffffu)), x1 = f16_to_f32((uint16_t)(w >> 16));
                        t = fmaf(x0, x0, t);
                        t = fmaf(x1, x1, t);
                    }
                }
                const u32x4 x = relu_bf16x8(QK ? (qr.x[ks] ^ neg16(ks)) : qr.x[ks]);   // the sign test is the same for fp16
                u32x4 hi, lo;
#pragma unroll
                for (int d = 0; d < 4; ++d) {
                    uint32_t h, l;
                    float f0, f1;
                    split_f16x2(x[d], h, l, f0, f1);
                    hi[d] = h;
                    lo[d] = l;
                    float& t = (D16 && ks == 1) ? dp1 : dp;
                    t = fmaf(f0, sden[8 * ks + 2 * d], t);
                    t = fmaf(f1, sden[8 * ks + 2 * d + 1], t);
                }
#pragma unroll
                for (int sp = 2; sp >= 0; --sp) acc = mfma_bf16(sa[ks][sp], lo, acc);   // small terms first
#pragma unroll
                for (int sp = 2; sp >= 0; --sp) acc = mfma_bf16(sa[ks][sp], hi, acc);
            }
        } else {
            u32x4 a[KS];
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                if constexpr (QK) {
                    float& t = (D16 && ks == 1) ? ss1 : ss;
#pragma unroll
                    for (int d = 0; d < 4; ++d) {
                        const uint32_t w = qr.x[ks][d];
                        t = fmaf(lo_bf16(w), lo_bf16(w), t);
                        t = fmaf(hi_bf16(w), hi_bf16(w), t);
                    }
                }
                a[ks] = relu_bf16x8(QK ? (qr.x[ks] ^ neg16(ks)) : qr.x[ks]);
            }
#pragma unroll
            for (int sp = 2; sp >= 0; --sp)   // small split terms first
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) acc = mfma_bf16(sa[ks][sp], a[ks], acc);
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
#pragma unroll
                for (int d = 0; d < 4; ++d) {
                    float& t = (D16 && ks == 1) ? dp1 : dp;
                    t = fmaf(lo_bf16(a[ks][d]), sden[8 * ks + 2 * d], t);
                    t = fmaf(hi_bf16(a[ks][d]), sden[8 * ks + 2 * d + 1], t);
                }
        }
        const float den = dp + __shfl_xor(dp, 32);   // same sum on lanes i and i + 32
        // qk_norm: eps meets the normaliser divided by rho_i, i.e. eps * rms_i
        float epsq = eps, epsq1 = eps;
        if constexpr (QK) {
            epsq = eps * sqrtf((ss + __shfl_xor(ss, 32)) * (1.0f / HD) + norm_eps);
            if constexpr (D16) epsq1 = eps * sqrtf((ss1 + __shfl_xor(ss1, 32)) * (1.0f / HD) + norm_eps);
        }
        const float rinv = 1.0f / (den + epsq);
        if constexpr (D16) {
            // rows 0..15 (r < 8) are the first head's outputs, 16..31 the second's
            const float den1 = dp1 + __shfl_xor(dp1, 32);
            const float rinv1 = 1.0f / (den1 + epsq1);
#pragma unroll
            for (int rg = 0; rg < 16; ++rg) acc[rg] *= rg < 8 ? rinv : rinv1;
        } else {
#pragma unroll
            for (int rg = 0; rg < 16; ++rg) acc[rg] *= rinv;
        }
        return acc;
    };

    if constexpr (sizeof(OutT) == 4) {
        // fp32: one head's output row is a whole 128-byte line; each wave
        // stores its own tile through its LDS tile
        if (h >= H) return;
        const int lim = HR * HD - h * kD;   // elements of the row from this group on (16 for a lone head of dim 16)
        float* ot = otile[wave];
        int tt = t0 + 32 * sub;
        QRow cur;
        load_b(tt, cur);
        for (; tt < t1; tt += 64) {
            QRow nxt;
            load_b(tt + 64, nxt);       // next sub-tile of this wave, in flight during the MFMAs
            const f32x16 acc = compute(cur);
            // tile row i = token tt + i; lane (g, i) holds columns 8 rr + 4 g .. +3
#pragma unroll
            for (int rr = 0; rr < 4; ++rr)
                *reinterpret_cast<f32x4*>(ot + i * kOutPitch + 8 * rr + 4 * g) =
                    (f32x4){acc[4 * rr], acc[4 * rr + 1], acc[4 * rr + 2], acc[4 * rr + 3]};
            __builtin_amdgcn_wave_barrier();
            // each store: 8 rows x 8 lanes x 4 columns = 8 whole output rows of this head
#pragma unroll
            for (int s4 = 0; s4 < 4; ++s4) {
                const int r = 8 * s4 + (lane >> 3), cc = (lane & 7) * 4;
                const f32x4 x = *reinterpret_cast<const f32x4*>(ot + r * kOutPitch + cc);
                if (tt + r < t1 && cc < lim) store4(out + (b * so.b + (tt + r) * so.n + h * kD + cc), x);
            }
            __builtin_amdgcn_wave_barrier();
            cur = nxt;
        }
    } else {
        // 16-bit: both heads of a token share one 128-byte output line; the
        // two waves of a sub-tile fill a pair tile and then store whole lines.
        // All waves take the same number of steps (a step past the range
        // works on the clamped last row).
        __shared__ __attribute__((aligned(16))) uint16_t ct[2][32 * kPairRow];
        const int nchunk = min(8, (HR * HD - 2 * hp * kD) / 8);   // 16-byte chunks of the line that exist
        const int steps = (t1 - t0 + 63) / 64;
        int tt = t0 + 32 * sub;
        QRow cur;
        load_b(tt, cur);
        for (int st = 0; st < steps; ++st, tt += 64) {
            QRow nxt;
            load_b(tt + 64, nxt);
            const f32x16 acc = compute(cur);
            put_pair_tile<OutT>(ct[sub], acc, lane, hh);
            __syncthreads();
            // wave (sub, hh) stores rows 16 hh .. 16 hh + 15 of its sub-tile
            // (rows past the range repeat the last row, with its bits)
            store_pair_rows<OutT>(ct[sub], lane, 16 * hh, nchunk, [&](int r) {
                return reinterpret_cast<uint16_t*>(out + (b * so.b + min(tt + r, t1 - 1) * so.n + 2 * hp * kD));
            });
            __syncthreads();
            cur = nxt;
        }
    }
}

// ------------------------------------------------------------------ apply, vector path
// grid.x = ((b * H + h) * NB + beta) * tpb + tile; one thread per token.
template <typename InT, typename OutT, int DD>
__global__ __launch_bounds__(kThreads) void k_apply_valu(
    const InT* __restrict__ q, const float* __restrict__ state, OutT* __restrict__ out,
    int N, int H, int L, int NB, int tpb, float eps, Strides sq, Strides so, const float* __restrict__ gq,
    float norm_eps) {
    constexpr int WW = DD + 1, SF = DD * WW;
    __shared__ float s[SF];
    const int tile = blockIdx.x % tpb;
    const size_t bhb = blockIdx.x / tpb;            // (b * H + h) * NB + beta
    const int beta = (int)(bhb % NB);
    const size_t bh = bhb / NB;
    const int h = (int)(bh % H), b = (int)(bh / H);
    for (int e = threadIdx.x; e < SF; e += kThreads) s[e] = state[bhb * SF + e];
    __syncthreads();
    const int blk0 = beta * L;
    const int blk1 = min(blk0 + L, N);
    const int row = blk0 + tile * kValuApplyTokens + threadIdx.x;
    if (row >= blk1) return;
    const long long qbase = b * sq.b + row * sq.n + (long long)h * DD;
    const long long obase = b * so.b + row * so.n + (long long)h * DD;
    float f[DD];
#pragma unroll
    for (int jj = 0; jj < DD; ++jj) f[jj] = load_in(q, qbase + jj);
    if (gq) {   // qk_norm, from the definition
        float ss = 0.f;
#pragma unroll
        for (int jj = 0; jj < DD; ++jj) ss += f[jj] * f[jj];
        const float r = 1.0f / sqrtf(ss / DD + norm_eps);
#pragma unroll
        for (int jj = 0; jj < DD; ++jj) f[jj] = gq[h * DD + jj] * f[jj] * r;
    }
#pragma unroll
    for (int jj = 0; jj < DD; ++jj) f[jj] = f[jj] > 0.f ? f[jj] : 0.f;
    float den = 0.f;
#pragma unroll
    for (int jj = 0; jj < DD; ++jj) den += f[jj] * s[jj * WW + DD];
    for (int cc = 0; cc < DD; ++cc) {
        float num = 0.f;
#pragma unroll
        for (int jj = 0; jj < DD; ++jj) num += f[jj] * s[jj * WW + cc];
        store_out(out, obase + cc, num / (den + eps));
    }
}

}  // namespace

// ------------------------------------------------------------------ launchers
namespace {
template <typename T> struct Tag { using type = T; };

// Calls f(Tag<T>{}) with T the element type of ABI dtype code `code`.
template <typename F> void by_dtype(int code, F&& f) {
    if (code == 1)
        f(Tag<uint16_t>{});
    else if (code == 2)
        f(Tag<_Float16>{});
    else
        f(Tag<float>{});
}

// Calls f(std::integral_constant<int, D>) for the supported head dims.
}  // namespace

hipError_t launch_state(const Plan& pl, const void* k, const void* v, float* part, hipStream_t stream) {
    const uint16_t* k16 = static_cast<const uint16_t*>(k);
    const uint16_t* v16 = static_cast<const uint16_t*>(v);
    if (pl.mfma) {
        const unsigned grid = (unsigned)((size_t)pl.B * pl.HP * pl.P);
        if (pl.gk)   // qk_norm on the keys: every input type takes the split-term kernel
            by_dtype(pl.in_dtype, [&](auto in) {
                using IT = typename decltype(in)::type;
                by_head_dim(pl.D, [&](auto dd) {
                    constexpr int DD = decltype(dd)::value;
                    hipLaunchKernelGGL((k_state_partial_mfma_f32<DD, IT, true>), dim3(grid), dim3(kThreads), 0, stream,
                                       static_cast<const IT*>(k), static_cast<const IT*>(v), part, pl.N, groups32(pl),
                                       pl.HP, pl.H, pl.L, pl.cpb, pl.P, pl.chunk, pl.sk, pl.sv, pl.gk, pl.norm_eps);
                });
            });
        else if (pl.in_dtype == 0)
            by_head_dim(pl.D, [&](auto dd) {
                constexpr int DD = decltype(dd)::value;
                hipLaunchKernelGGL(k_state_partial_mfma_f32<DD>, dim3(grid), dim3(kThreads), 0, stream,
                                   static_cast<const float*>(k), static_cast<const float*>(v), part, pl.N,
                                   groups32(pl), pl.HP, pl.H, pl.L, pl.cpb, pl.P, pl.chunk, pl.sk, pl.sv,
                                   (const float*)nullptr, 0.f);
            });
        else
            by_head_dim(pl.D, [&](auto dd) {
                constexpr int DD = decltype(dd)::value;
                auto kern = pl.in_dtype == 2 ? k_state_partial_mfma<true, DD> : k_state_partial_mfma<false, DD>;
                hipLaunchKernelGGL(kern, dim3(grid), dim3(kThreads), 0, stream, k16, v16, part, pl.N,
                                   groups32(pl), pl.HP, pl.H, pl.L, pl.cpb, pl.P, pl.chunk, pl.sk, pl.sv);
            });
    } else {
        const unsigned grid = (unsigned)((size_t)pl.B * pl.H * pl.P);
        by_dtype(pl.in_dtype, [&](auto in) {
            by_head_dim(pl.D, [&](auto dd) {
                using IT = typename decltype(in)::type;
                constexpr int DD = decltype(dd)::value;
                hipLaunchKernelGGL((k_state_partial_valu<IT, DD>), dim3(grid), dim3(kThreads), 0, stream,
                                   static_cast<const IT*>(k), static_cast<const IT*>(v), part,
                                   pl.N, pl.H, pl.L, pl.cpb, pl.P, pl.chunk, pl.sk, pl.sv, pl.gk, pl.norm_eps);
            });
        });
    }
    return hipGetLastError();
}

hipError_t launch_merge(const Plan& pl, const float* part, float* state, const float* state_in,
                        float* state_out, hipStream_t stream) {
    const int SF = pl.D * (pl.D + 1);
    const unsigned grid = (unsigned)((size_t)pl.B * pl.H * ((SF + kMergeThreads - 1) / kMergeThreads));
    hipLaunchKernelGGL(k_merge, dim3(grid), dim3(kMergeThreads), 0, stream, part, state, state_in, state_out,
                       pl.NB, pl.cpb, pl.P, SF, pl.mfma ? pl.gk : nullptr, pl.H, pl.D);
    return hipGetLastError();
}

hipError_t launch_apply(const Plan& pl, const void* q, const float* state, void* out, float eps,
                        hipStream_t stream) {
    if (pl.mfma) {
        const unsigned grid = (unsigned)((size_t)pl.B * pl.HP * pl.NB * pl.tpb);
        by_dtype(pl.in_dtype, [&](auto in) {
            by_dtype(pl.out_dtype, [&](auto o) {
                using IT = typename decltype(in)::type;
                using OT = typename decltype(o)::type;
                by_head_dim(pl.D, [&](auto dd) {
                    constexpr int DD = decltype(dd)::value;
                    auto kern = pl.gq ? k_apply_mfma<IT, OT, DD, true> : k_apply_mfma<IT, OT, DD, false>;
                    hipLaunchKernelGGL(kern, dim3(grid), dim3(kThreads), 0, stream,
                                       static_cast<const IT*>(q), state, static_cast<OT*>(out), pl.N, groups32(pl),
                                       pl.HP, pl.H, pl.L, pl.NB, pl.tile, pl.tpb, eps, pl.sq, pl.so, pl.gq,
                                       pl.norm_eps);
                });
            });
        });
    } else {
        const unsigned grid = (unsigned)((size_t)pl.B * pl.H * pl.NB * pl.tpb);
        by_dtype(pl.in_dtype, [&](auto in) {
            by_dtype(pl.out_dtype, [&](auto o) {
              by_head_dim(pl.D, [&](auto dd) {
                using IT = typename decltype(in)::type;
                using OT = typename decltype(o)::type;
                constexpr int DD = decltype(dd)::value;
                hipLaunchKernelGGL((k_apply_valu<IT, OT, DD>), dim3(grid), dim3(kThreads), 0, stream,
                                   static_cast<const IT*>(q), state, static_cast<OT*>(out), pl.N, pl.H, pl.L,
                                   pl.NB, pl.tpb, eps, pl.sq, pl.so, pl.gq, pl.norm_eps);
              });
            });
        });
    }
    return hipGetLastError();
}

}  // namespace sana
