// gfx950 kernels of the LiteLA forward-mode derivative (JVP): the output and
// its tangent for tangents (qt, kt, vt) of the inputs, for the ReLU-kernel
// linear self-attention of "Sana: the autoencoder does more of the work than
// the linear attention", section "What LiteLA actually computes".
//
// With f = ReLU(q), a = ReLU(k), ft = [q > 0] qt, at = [k > 0] kt:
//   S  = sum a [v | 1]^T,   St = sum (at [v | 1]^T + a [vt | 0]^T)
//        (both per chunk, then merged and prefixed over blocks by the
//        forward's merge kernel, which sees them as 2 H heads)
//   num = S_v^T f,  den = S_z . f,  numt = St_v^T f + S_v^T ft,
//   dent = St_z . f + S_z . ft
//   out = num r,  outt = (numt - out dent) r,  r = 1 / (den + eps)
// Everything accumulates in fp32; products of 16-bit inputs are exact.
#include "linattn_device.h"

namespace sana {
namespace {

// Packed 16-bit halves of t where the same half of a is non-zero, else 0
// (a = ReLU(x) is non-zero exactly where x > 0).
__device__ __forceinline__ uint32_t keep_where_nonzero(uint32_t a, uint32_t t) {
    const uint32_t m = ((a & 0xffffu) ? 0xffffu : 0u) | ((a >> 16) ? 0xffff0000u : 0u);
    return t & m;
}
__device__ __forceinline__ u32x4 keep_where_nonzero(u32x4 a, u32x4 t) {
    return (u32x4){keep_where_nonzero(a[0], t[0]), keep_where_nonzero(a[1], t[1]), keep_where_nonzero(a[2], t[2]),
                   keep_where_nonzero(a[3], t[3])};
}

// ------------------------------------------------------------------ state and tangent state, MFMA
// As the forward's state kernel, with four tensors in the LDS tile:
// [a | v | at | vt][head 0|1][token][32 x 16 bit].
constexpr int kJHead = kStateTile * 64 + 64;   // bytes per head (second head shifted by 64 bytes)
constexpr int kJTensor = 2 * kJHead;
constexpr int kJPieces = kStateTile / 32;
static_assert(4 * kJTensor >= 2 * 4 * 16 * 64 * (int)sizeof(float), "reduction area exceeds the LDS tile");

// grid.x = (b * HP + hp) * P + p.  Partials: part[((b * H + h) * 2 + s) * P + p],
// s = 0 the state, s = 1 the tangent state.
template <bool F16>
__global__ __launch_bounds__(kThreads) void k_jvp_state_mfma(
    const uint16_t* __restrict__ k, const uint16_t* __restrict__ v, const uint16_t* __restrict__ kt,
    const uint16_t* __restrict__ vt, float* __restrict__ part, int N, int H, int HP, int L, int cpb, int P,
    int chunk) {
    __shared__ __attribute__((aligned(16))) uint8_t lds[4 * kJTensor];

    const int p = blockIdx.x % P;
    const int bhp = blockIdx.x / P;
    const int hp = bhp % HP, b = bhp / HP;
    const int h0 = 2 * hp;
    const int nh = min(2, H - h0);
    const ChunkRange cr = chunk_range(p, cpb, chunk, L, N);
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int hh = wave & 1, th = wave >> 1;
    const long long hstride = (long long)H * kD;
    const uint16_t* src[4] = {k, v, kt, vt};

    u32x4 r[4][kJPieces];
    auto load_tile = [&](int t0) {
#pragma unroll
        for (int i = 0; i < kJPieces; ++i) {
            const int pc = tid + kThreads * i;
            const int part_ = pc & 3, hd = (pc >> 2) & 1, tok = pc >> 3;
            const int n = t0 + tok;
            const bool ok = n < cr.c1 && hd < nh;
            const long long off = ((long long)b * N + (ok ? n : cr.c0)) * hstride + (h0 + (ok ? hd : 0)) * kD + part_ * 8;
#pragma unroll
            for (int ts = 0; ts < 4; ++ts) {
                const u32x4 x = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(src[ts] + off));
                r[ts][i] = ok ? x : (u32x4){0u, 0u, 0u, 0u};
            }
        }
    };

    f32x16 accV = {}, accO = {}, accVt = {}, accOt = {};
    constexpr uint32_t kOne2 = F16 ? 0x3c003c00u : 0x3f803f80u;
    const u32x4 ones = {kOne2, kOne2, kOne2, kOne2};
    const int g = lane >> 5, j = lane & 31;

    if (cr.c0 < cr.c1) load_tile(cr.c0);
    for (int t0 = cr.c0; t0 < cr.c1; t0 += kStateTile) {
        __syncthreads();
#pragma unroll
        for (int i = 0; i < kJPieces; ++i) {
            const int pc = tid + kThreads * i;
            const int part_ = pc & 3, hd = (pc >> 2) & 1, tok = pc >> 3;
            const int o = hd * kJHead + tok * 64 + part_ * 16;
            const u32x4 a = relu_bf16x8(r[0][i]);
            *reinterpret_cast<u32x4*>(lds + o) = a;
            *reinterpret_cast<u32x4*>(lds + kJTensor + o) = r[1][i];
            *reinterpret_cast<u32x4*>(lds + 2 * kJTensor + o) = keep_where_nonzero(a, r[2][i]);
            *reinterpret_cast<u32x4*>(lds + 3 * kJTensor + o) = r[3][i];
        }
        __syncthreads();
        if (t0 + kStateTile < cr.c1) load_tile(t0 + kStateTile);

        const uint16_t* T[4];
#pragma unroll
        for (int ts = 0; ts < 4; ++ts) T[ts] = reinterpret_cast<const uint16_t*>(lds + ts * kJTensor + hh * kJHead);
#pragma unroll
        for (int st = 0; st < kStateTile / 32; ++st) {
            // element e of lane (g, j) is token tb + 2e + g (row j of a, at; column j of v, vt)
            const int tb = (kStateTile / 2) * th + 16 * st;
            u32x4 op[4];
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const int r0 = (tb + 4 * t + g) * 32 + j;
                const int r1 = r0 + 2 * 32;
#pragma unroll
                for (int ts = 0; ts < 4; ++ts) op[ts][t] = (uint32_t)T[ts][r0] | ((uint32_t)T[ts][r1] << 16);
            }
            accV = mfma16<F16>(op[0], op[1], accV);
            accO = mfma16<F16>(op[0], ones, accO);
            accVt = mfma16<F16>(op[2], op[1], accVt);
            accVt = mfma16<F16>(op[0], op[3], accVt);
            accOt = mfma16<F16>(op[2], ones, accOt);
        }
    }

    __syncthreads();
    float* red = reinterpret_cast<float*>(lds);   // [head][4][16][64]
    const f32x16* accs[4] = {&accV, &accO, &accVt, &accOt};
    if (th == 1) {
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4)
#pragma unroll
            for (int rg = 0; rg < 16; ++rg) red[((hh * 4 + q4) * 16 + rg) * 64 + lane] = (*accs[q4])[rg];
    }
    __syncthreads();
    if (th == 0 && hh < nh) {
        const size_t bh = (size_t)b * H + h0 + hh;
        float* dS = part + ((bh * 2 + 0) * P + p) * kStateFloats;
        float* dT = part + ((bh * 2 + 1) * P + p) * kStateFloats;
#pragma unroll
        for (int rg = 0; rg < 16; ++rg) {
            const int row = 8 * (rg >> 2) + 4 * g + (rg & 3);
            dS[row * kW + j] = accV[rg] + red[((hh * 4 + 0) * 16 + rg) * 64 + lane];
            dT[row * kW + j] = accVt[rg] + red[((hh * 4 + 2) * 16 + rg) * 64 + lane];
            if (j == 0) {
                dS[row * kW + kD] = accO[rg] + red[((hh * 4 + 1) * 16 + rg) * 64 + lane];
                dT[row * kW + kD] = accOt[rg] + red[((hh * 4 + 3) * 16 + rg) * 64 + lane];
            }
        }
    }
}

// ------------------------------------------------------------------ output and tangent, MFMA
// grid.x = (b * HP + hp) * (NB * tpb) + beta * tpb + tile; wave w: head
// 2*hp + (w & 1), every other 32-token sub-tile (w >> 1).
template <bool F16, typename OutT>
__global__ __launch_bounds__(kThreads) void k_jvp_apply_mfma(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ qt, const float* __restrict__ state,
    OutT* __restrict__ out, OutT* __restrict__ outt, int N, int H, int HP, int L, int NB, int tile, int tpb,
    float eps) {
    __shared__ __attribute__((aligned(16))) float otile[4][32 * kPitch];

    const int per_unit = NB * tpb;
    const int tau = blockIdx.x % per_unit;
    const int bhp = blockIdx.x / per_unit;
    const int hp = bhp % HP, b = bhp / HP;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int h = 2 * hp + (wave & 1);
    if (h >= H) return;
    const int beta = tau / tpb, tib = tau - beta * tpb;
    const int blk0 = beta * L, blk1 = min(blk0 + L, N);
    const int t0 = blk0 + tib * tile, t1 = min(t0 + tile, blk1);
    if (t0 >= t1) return;
    const int g = lane >> 5, i = lane & 31;

    const size_t bh = (size_t)b * H + h;
    const float* S = state + ((bh * 2 + 0) * NB + beta) * kStateFloats;
    const float* St = state + ((bh * 2 + 1) * NB + beta) * kStateFloats;
    u32x4 sa[2][3], sat[2][3];
    state_operands(S, lane, true, sa);
    state_operands(St, lane, true, sat);
    float sz[16], szt[16];   // S[:, D] and St[:, D] at this lane's features 16 ks + 8 g + e
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            sz[8 * ks + e] = S[(16 * ks + 8 * g + e) * kW + kD];
            szt[8 * ks + e] = St[(16 * ks + 8 * g + e) * kW + kD];
        }

    const long long hstride = (long long)H * kD;
    float* ot = otile[wave];
    for (int tt = t0 + 32 * (wave >> 1); tt < t1; tt += 64) {
        const int row = min(tt + i, t1 - 1);   // clamped rows repeat the last row (see store_tile)
        const u32x4* srcq = reinterpret_cast<const u32x4*>(q + ((long long)b * N + row) * hstride + h * kD + 8 * g);
        const u32x4* srct = reinterpret_cast<const u32x4*>(qt + ((long long)b * N + row) * hstride + h * kD + 8 * g);
        const u32x4 f0 = relu_bf16x8(srcq[0]), f1 = relu_bf16x8(srcq[2]);
        const u32x4 ft0 = keep_where_nonzero(f0, srct[0]), ft1 = keep_where_nonzero(f1, srct[2]);
        const int n = min(32, t1 - tt);

        f32x16 acc = {}, acct = {};
        acc = mma_split<F16>(sa, f0, f1, acc);
        acct = mma_split<F16>(sat, f0, f1, acct);
        acct = mma_split<F16>(sa, ft0, ft1, acct);
        float dp = 0.f, dpt = 0.f;
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            const u32x4 fx = ks ? f1 : f0, fy = ks ? ft1 : ft0;
#pragma unroll
            for (int d = 0; d < 4; ++d) {
                float x0, x1, y0, y1;
                if constexpr (F16) {
                    x0 = f16_to_f32((uint16_t)(fx[d] & 0xffffu));
                    x1 = f16_to_f32((uint16_t)(fx[d] >> 16));
                    y0 = f16_to_f32((uint16_t)(fy[d] & 0xffffu));
                    y1 = f16_to_f32((uint16_t)(fy[d] >> 16));
                } else {
                    x0 = lo_bf16(fx[d]);
                    x1 = hi_bf16(fx[d]);
                    y0 = lo_bf16(fy[d]);
                    y1 = hi_bf16(fy[d]);
                }
                const int e = 8 * ks + 2 * d;
                dp = fmaf(x0, sz[e], dp);
                dp = fmaf(x1, sz[e + 1], dp);
                dpt = fmaf(x0, szt[e], dpt);
                dpt = fmaf(x1, szt[e + 1], dpt);
                dpt = fmaf(y0, sz[e], dpt);
                dpt = fmaf(y1, sz[e + 1], dpt);
            }
        }
        const float den = dp + __shfl_xor(dp, 32);
        const float dent = dpt + __shfl_xor(dpt, 32);
        const float rinv = 1.0f / (den + eps);
#pragma unroll
        for (int rg = 0; rg < 16; ++rg) {
            const float o = acc[rg] * rinv;
            acc[rg] = o;
            acct[rg] = (acct[rg] - o * dent) * rinv;
        }
        store_tile<OutT>(ot, acc, lane, n, [&](int t) { return out + ((long long)b * N + tt + t) * hstride + h * kD; });
        store_tile<OutT>(ot, acct, lane, n,
                         [&](int t) { return outt + ((long long)b * N + tt + t) * hstride + h * kD; });
    }
}

// ------------------------------------------------------------------ fp32 inputs, MFMA
// State and tangent state for fp32 k, v, kt, vt.  Tiles of 32 tokens of a
// head pair: each thread loads one 32-byte piece (8 features of one head of one
// token) of each tensor, forms a = ReLU(k), at = [k > 0] kt, v and vt, splits
// each value by truncation into three bf16 terms (exact) and stages them in
// LDS as term tiles [tensor][term][head][token][32 x 16 bit] (48 KB).  Wave w
// (head w & 1) then gathers tokens 16 (w >> 1) .. + 15 of the tile with
// transposing LDS reads and accumulates, over the term pairs i + j <= 2
// (0-based; the dropped products are below 2^-24 of the exact one):
//   S_v += a v,   St_v += at v + a vt,   S_z += a 1,   St_z += at 1 (exact)
constexpr int kJF32Tok = 32;
constexpr int kJF32Tile = kJF32Tok * kD;   // 16-bit elements of one term tile of one head

__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(3, 8))) void k_jvp_state_mfma_f32(
    const float* __restrict__ k, const float* __restrict__ v, const float* __restrict__ kt,
    const float* __restrict__ vt, float* __restrict__ part, int N, int H, int HP, int L, int cpb, int P, int chunk) {
    __shared__ __attribute__((aligned(16))) uint16_t lds[4][3][2][kJF32Tile];   // [a | v | at | vt][term][head]
    static_assert(sizeof(lds) >= 2 * 4 * 16 * 64 * sizeof(float), "reduction area exceeds the LDS tile");

    const int p = blockIdx.x % P;
    const int bhp = blockIdx.x / P;
    const int hp = bhp % HP, b = bhp / HP;
    const int h0 = 2 * hp;
    const int nh = min(2, H - h0);
    const ChunkRange cr = chunk_range(p, cpb, chunk, L, N);
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int hh = wave & 1, th = wave >> 1;
    const int g = lane >> 5, j = lane & 31;
    const long long hstride = (long long)H * kD;
    const float* src[4] = {k, v, kt, vt};

    // this thread's piece of a tile: part (tid & 3) = features 8 part .. + 7,
    // head (tid >> 2) & 1, token tid >> 3
    const int part_ = tid & 3, hd = (tid >> 2) & 1, tok = tid >> 3;
    f32x4 r[4][2];
    auto load_tile = [&](int t0) {
        const int n = t0 + tok;
        const bool ok = n < cr.c1 && hd < nh;
        const long long off = ((long long)b * N + (ok ? n : cr.c0)) * hstride + (h0 + (ok ? hd : 0)) * kD + part_ * 8;
#pragma unroll
        for (int ts = 0; ts < 4; ++ts) {
            const f32x4* s = reinterpret_cast<const f32x4*>(src[ts] + off);
            const f32x4 x0 = __builtin_nontemporal_load(s), x1 = __builtin_nontemporal_load(s + 1);
            r[ts][0] = ok ? x0 : (f32x4){0.f, 0.f, 0.f, 0.f};
            r[ts][1] = ok ? x1 : (f32x4){0.f, 0.f, 0.f, 0.f};
        }
    };

    f32x16 accV = {}, accO = {}, accVt = {}, accOt = {};
    const u32x4 ones = {0x3f803f80u, 0x3f803f80u, 0x3f803f80u, 0x3f803f80u};   // bf16 1.0 pairs

    if (cr.c0 < cr.c1) load_tile(cr.c0);
    for (int t0 = cr.c0; t0 < cr.c1; t0 += kJF32Tok) {
        __syncthreads();   // the previous tile has been consumed
        {
            float x[4][8];   // a, v, at, vt
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float kk = r[0][e >> 2][e & 3];
                x[0][e] = relu_f32(kk);
                x[1][e] = r[1][e >> 2][e & 3];
                x[2][e] = kk > 0.f ? r[2][e >> 2][e & 3] : 0.f;
                x[3][e] = r[3][e >> 2][e & 3];
            }
            const int o = tok * kD + part_ * 8;
#pragma unroll
            for (int ts = 0; ts < 4; ++ts) {
                u32x4 t[3];
                split3_trunc_f32x8(x[ts], t);
#pragma unroll
                for (int sp = 0; sp < 3; ++sp) *reinterpret_cast<u32x4*>(&lds[ts][sp][hd][o]) = t[sp];
            }
        }
        __syncthreads();
        if (t0 + kJF32Tok < cr.c1) load_tile(t0 + kJF32Tok);   // in flight during the MFMAs

        // lane (g, j): tokens 16 th + 8 g + e of feature (a, at) / channel (v, vt) j
        u32x4 ta[3], tv[3], tat[3], tvt[3];
#pragma unroll
        for (int sp = 0; sp < 3; ++sp) {
            ta[sp] = gather_tokens_t16(lds[0][sp][hh], kD, 16 * th, 0, lane);
            tv[sp] = gather_tokens_t16(lds[1][sp][hh], kD, 16 * th, 0, lane);
            tat[sp] = gather_tokens_t16(lds[2][sp][hh], kD, 16 * th, 0, lane);
            tvt[sp] = gather_tokens_t16(lds[3][sp][hh], kD, 16 * th, 0, lane);
        }
        // smallest products first
        accV = mma_terms(ta, tv, accV);
        accVt = mfma_bf16(tat[2], tv[0], accVt);
        accVt = mfma_bf16(tat[1], tv[1], accVt);
        accVt = mfma_bf16(tat[0], tv[2], accVt);
        accVt = mfma_bf16(ta[2], tvt[0], accVt);
        accVt = mfma_bf16(ta[1], tvt[1], accVt);
        accVt = mfma_bf16(ta[0], tvt[2], accVt);
        accVt = mfma_bf16(tat[1], tv[0], accVt);
        accVt = mfma_bf16(tat[0], tv[1], accVt);
        accVt = mfma_bf16(ta[1], tvt[0], accVt);
        accVt = mfma_bf16(ta[0], tvt[1], accVt);
        accVt = mfma_bf16(tat[0], tv[0], accVt);
        accVt = mfma_bf16(ta[0], tvt[0], accVt);
#pragma unroll
        for (int sp = 2; sp >= 0; --sp) {
            accO = mfma_bf16(ta[sp], ones, accO);
            accOt = mfma_bf16(tat[sp], ones, accOt);
        }
    }

    // the two token halves of each head in a fixed order, as the 16-bit kernel
    __syncthreads();
    float* red = reinterpret_cast<float*>(&lds[0][0][0][0]);   // [head][4][16][64]
    const f32x16* accs[4] = {&accV, &accO, &accVt, &accOt};
    if (th == 1) {
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4)
#pragma unroll
            for (int rg = 0; rg < 16; ++rg) red[((hh * 4 + q4) * 16 + rg) * 64 + lane] = (*accs[q4])[rg];
    }
    __syncthreads();
    if (th == 0 && hh < nh) {
        const size_t bh = (size_t)b * H + h0 + hh;
        float* dS = part + ((bh * 2 + 0) * P + p) * kStateFloats;
        float* dT = part + ((bh * 2 + 1) * P + p) * kStateFloats;
#pragma unroll
        for (int rg = 0; rg < 16; ++rg) {
            const int row = 8 * (rg >> 2) + 4 * g + (rg & 3);
            dS[row * kW + j] = accV[rg] + red[((hh * 4 + 0) * 16 + rg) * 64 + lane];
            dT[row * kW + j] = accVt[rg] + red[((hh * 4 + 2) * 16 + rg) * 64 + lane];
            if (j == 0) {
                dS[row * kW + kD] = accO[rg] + red[((hh * 4 + 1) * 16 + rg) * 64 + lane];
                dT[row * kW + kD] = accOt[rg] + red[((hh * 4 + 3) * 16 + rg) * 64 + lane];
            }
        }
    }
}

// Output and tangent for fp32 q and qt: the 16-bit kernel's waves and
// sub-tiles, q and qt read per wave in the operand layout (the next
// sub-tile's loads in flight during this one's work), f = ReLU(q) and
// ft = [q > 0] qt split into three bf16 terms each:
//   num = S_v^T f (6 term products per K-step), numt = St_v^T f + S_v^T ft (12);
// the normalisers are fp32 dot products of the unsplit values.
template <typename OutT>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 8))) void k_jvp_apply_mfma_f32(
    const float* __restrict__ q, const float* __restrict__ qt, const float* __restrict__ state,
    OutT* __restrict__ out, OutT* __restrict__ outt, int N, int H, int HP, int L, int NB, int tile, int tpb,
    float eps) {
    __shared__ __attribute__((aligned(16))) float otile[4][32 * kPitch];

    const int per_unit = NB * tpb;
    const int tau = blockIdx.x % per_unit;
    const int bhp = blockIdx.x / per_unit;
    const int hp = bhp % HP, b = bhp / HP;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int h = 2 * hp + (wave & 1);
    if (h >= H) return;
    const int beta = tau / tpb, tib = tau - beta * tpb;
    const int blk0 = beta * L, blk1 = min(blk0 + L, N);
    const int t0 = blk0 + tib * tile, t1 = min(t0 + tile, blk1);
    if (t0 >= t1 || t0 + 32 * (wave >> 1) >= t1) return;
    const int g = lane >> 5, i = lane & 31;

    const size_t bh = (size_t)b * H + h;
    const float* S = state + ((bh * 2 + 0) * NB + beta) * kStateFloats;
    const float* St = state + ((bh * 2 + 1) * NB + beta) * kStateFloats;
    u32x4 sa[2][3], sat[2][3];
    state_operands(S, lane, true, sa);
    state_operands(St, lane, true, sat);
    float sz[16], szt[16];   // S[:, D] and St[:, D] at this lane's features 16 ks + 8 g + e
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            sz[8 * ks + e] = S[(16 * ks + 8 * g + e) * kW + kD];
            szt[8 * ks + e] = St[(16 * ks + 8 * g + e) * kW + kD];
        }

    const long long hstride = (long long)H * kD;
    auto row_of = [&](const float* x, int tt) { return x + ((long long)b * N + min(tt + i, t1 - 1)) * hstride + h * kD; };
    float* ot = otile[wave];
    F32Operand qc, tc;
    qc.load(row_of(q, t0 + 32 * (wave >> 1)), g);
    tc.load(row_of(qt, t0 + 32 * (wave >> 1)), g);
    for (int tt = t0 + 32 * (wave >> 1); tt < t1; tt += 64) {
        const int n = min(32, t1 - tt);   // clamped rows repeat the last row (see store_tile)
        F32Operand qn, tn;
        const bool more = tt + 64 < t1;
        if (more) {
            qn.load(row_of(q, tt + 64), g);
            tn.load(row_of(qt, tt + 64), g);
        }
        f32x16 acc = {}, acct = {};
        float dp = 0.f, dpt = 0.f;
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            float f[8], ft[8];
            qc.half(ks, true, f);
            tc.half(ks, false, ft);
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                ft[e] = f[e] > 0.f ? ft[e] : 0.f;
                dp = fmaf(f[e], sz[8 * ks + e], dp);
                dpt = fmaf(f[e], szt[8 * ks + e], dpt);
                dpt = fmaf(ft[e], sz[8 * ks + e], dpt);
            }
            u32x4 tf[3], tft[3];
            split3_trunc_f32x8(f, tf);
            split3_trunc_f32x8(ft, tft);
            acc = mma_terms(sa[ks], tf, acc);
            acct = mma_terms(sat[ks], tf, acct);
            acct = mma_terms(sa[ks], tft, acct);
        }
        const float den = dp + __shfl_xor(dp, 32);
        const float dent = dpt + __shfl_xor(dpt, 32);
        const float rinv = 1.0f / (den + eps);
#pragma unroll
        for (int rg = 0; rg < 16; ++rg) {
            const float o = acc[rg] * rinv;
            acc[rg] = o;
            acct[rg] = (acct[rg] - o * dent) * rinv;
        }
        store_tile<OutT>(ot, acc, lane, n, [&](int t) { return out + ((long long)b * N + tt + t) * hstride + h * kD; });
        store_tile<OutT>(ot, acct, lane, n,
                         [&](int t) { return outt + ((long long)b * N + tt + t) * hstride + h * kD; });
        if (more) {
            qc = qn;
            tc = tn;
        }
    }
}

// ------------------------------------------------------------------ vector path (cross-check)
constexpr int kJTok = 64;

// grid.x = (b * H + h) * P + p; thread t owns state entries t, t + 256, ...
template <typename InT>
__global__ __launch_bounds__(kThreads) void k_jvp_state_valu(
    const InT* __restrict__ k, const InT* __restrict__ v, const InT* __restrict__ kt, const InT* __restrict__ vt,
    float* __restrict__ part, int N, int H, int L, int cpb, int P, int chunk) {
    __shared__ float sa[kJTok][kD + 1], sat[kJTok][kD + 1];   // a, at
    __shared__ float sv[kJTok][kW], svt[kJTok][kW];           // [v | 1], [vt | 0]
    const int p = blockIdx.x % P;
    const int bh = blockIdx.x / P;
    const int h = bh % H, b = bh / H;
    const ChunkRange cr = chunk_range(p, cpb, chunk, L, N);
    const int tid = threadIdx.x;
    float acc[5] = {}, acct[5] = {};
    for (int t0 = cr.c0; t0 < cr.c1; t0 += kJTok) {
        __syncthreads();
        for (int e = tid; e < kJTok * kD; e += kThreads) {
            const int tok = e >> 5, jj = e & 31;
            const int n = t0 + tok;
            float kk = 0.f, kkt = 0.f, vv = 0.f, vvt = 0.f;
            if (n < cr.c1) {
                const long long off = (((long long)b * N + n) * H + h) * kD + jj;
                kk = load_in(k, off);
                kkt = load_in(kt, off);
                vv = load_in(v, off);
                vvt = load_in(vt, off);
            }
            sa[tok][jj] = kk > 0.f ? kk : 0.f;
            sat[tok][jj] = kk > 0.f ? kkt : 0.f;
            sv[tok][jj] = vv;
            svt[tok][jj] = vvt;
        }
        if (tid < kJTok) {
            sv[tid][kD] = 1.f;
            svt[tid][kD] = 0.f;
        }
        __syncthreads();
#pragma unroll
        for (int m = 0; m < 5; ++m) {
            const int o = tid + kThreads * m;
            if (o < kStateFloats) {
                const int jj = o / kW, c = o - jj * kW;
                float s = acc[m], st = acct[m];
                for (int tok = 0; tok < kJTok; ++tok) {
                    s += sa[tok][jj] * sv[tok][c];
                    st += sat[tok][jj] * sv[tok][c] + sa[tok][jj] * svt[tok][c];
                }
                acc[m] = s;
                acct[m] = st;
            }
        }
    }
    float* dS = part + (((size_t)bh * 2 + 0) * P + p) * kStateFloats;
    float* dT = part + (((size_t)bh * 2 + 1) * P + p) * kStateFloats;
#pragma unroll
    for (int m = 0; m < 5; ++m) {
        const int o = tid + kThreads * m;
        if (o < kStateFloats) {
            dS[o] = acc[m];
            dT[o] = acct[m];
        }
    }
}

// grid.x = ((b * H + h) * NB + beta) * tpb + tile; one thread per token.
template <typename InT, typename OutT>
__global__ __launch_bounds__(kThreads) void k_jvp_apply_valu(
    const InT* __restrict__ q, const InT* __restrict__ qt, const float* __restrict__ state, OutT* __restrict__ out,
    OutT* __restrict__ outt, int N, int H, int L, int NB, int tpb, float eps) {
    __shared__ float sS[kStateFloats], sT[kStateFloats];
    const int tile = blockIdx.x % tpb;
    const size_t bhb = blockIdx.x / tpb;   // (b * H + h) * NB + beta
    const int beta = (int)(bhb % NB);
    const size_t bh = bhb / NB;
    const int h = (int)(bh % H), b = (int)(bh / H);
    for (int e = threadIdx.x; e < kStateFloats; e += kThreads) {
        sS[e] = state[((bh * 2 + 0) * NB + beta) * kStateFloats + e];
        sT[e] = state[((bh * 2 + 1) * NB + beta) * kStateFloats + e];
    }
    __syncthreads();
    const int blk0 = beta * L, blk1 = min(blk0 + L, N);
    const int row = blk0 + tile * kThreads + threadIdx.x;
    if (row >= blk1) return;
    const long long base = (((long long)b * N + row) * H + h) * kD;
    float f[kD], ft[kD];
#pragma unroll
    for (int jj = 0; jj < kD; ++jj) {
        const float x = load_in(q, base + jj);
        f[jj] = x > 0.f ? x : 0.f;
        ft[jj] = x > 0.f ? load_in(qt, base + jj) : 0.f;
    }
    float den = 0.f, dent = 0.f;
#pragma unroll
    for (int jj = 0; jj < kD; ++jj) {
        den += f[jj] * sS[jj * kW + kD];
        dent += sT[jj * kW + kD] * f[jj] + sS[jj * kW + kD] * ft[jj];
    }
    for (int c = 0; c < kD; ++c) {
        float num = 0.f, numt = 0.f;
#pragma unroll
        for (int jj = 0; jj < kD; ++jj) {
            num += f[jj] * sS[jj * kW + c];
            numt += sT[jj * kW + c] * f[jj] + sS[jj * kW + c] * ft[jj];
        }
        const float o = num / (den + eps);
        store_out(out, base + c, o);
        store_out(outt, base + c, (numt - o * dent) / (den + eps));
    }
}

template <typename T> struct Tag { using type = T; };
template <typename F> void by_dtype(int code, F&& f) {
    if (code == 1)
        f(Tag<uint16_t>{});
    else if (code == 2)
        f(Tag<_Float16>{});
    else
        f(Tag<float>{});
}

}  // namespace

hipError_t launch_jvp_state(const Plan& pl, const void* k, const void* v, const void* kt, const void* vt, float* part,
                            hipStream_t stream) {
    if (pl.mfma && pl.in_dtype == 0) {
        const unsigned grid = (unsigned)((size_t)pl.B * pl.HP * pl.P);
        hipLaunchKernelGGL(k_jvp_state_mfma_f32, dim3(grid), dim3(kThreads), 0, stream, static_cast<const float*>(k),
                           static_cast<const float*>(v), static_cast<const float*>(kt), static_cast<const float*>(vt),
                           part, pl.N, pl.H, pl.HP, pl.L, pl.cpb, pl.P, pl.chunk);
    } else if (pl.mfma16) {
        const unsigned grid = (unsigned)((size_t)pl.B * pl.HP * pl.P);
        const uint16_t *k16 = static_cast<const uint16_t*>(k), *v16 = static_cast<const uint16_t*>(v),
                       *kt16 = static_cast<const uint16_t*>(kt), *vt16 = static_cast<const uint16_t*>(vt);
        if (pl.in_dtype == 2)
            hipLaunchKernelGGL(k_jvp_state_mfma<true>, dim3(grid), dim3(kThreads), 0, stream, k16, v16, kt16, vt16,
                               part, pl.N, pl.H, pl.HP, pl.L, pl.cpb, pl.P, pl.chunk);
        else
            hipLaunchKernelGGL(k_jvp_state_mfma<false>, dim3(grid), dim3(kThreads), 0, stream, k16, v16, kt16, vt16,
                               part, pl.N, pl.H, pl.HP, pl.L, pl.cpb, pl.P, pl.chunk);
    } else {
        const unsigned grid = (unsigned)((size_t)pl.B * pl.H * pl.P);
        by_dtype(pl.in_dtype, [&](auto it) {
            using IT = typename decltype(it)::type;
            hipLaunchKernelGGL(k_jvp_state_valu<IT>, dim3(grid), dim3(kThreads), 0, stream, static_cast<const IT*>(k),
                               static_cast<const IT*>(v), static_cast<const IT*>(kt), static_cast<const IT*>(vt), part,
                               pl.N, pl.H, pl.L, pl.cpb, pl.P, pl.chunk);
        });
    }
    return hipGetLastError();
}

hipError_t launch_jvp_apply(const Plan& pl, const void* q, const void* qt, const float* state, void* out, void* outt,
                            float eps, hipStream_t stream) {
    if (pl.mfma && pl.in_dtype == 0) {
        const unsigned grid = (unsigned)((size_t)pl.B * pl.HP * pl.NB * pl.tpb);
        by_dtype(pl.out_dtype, [&](auto o) {
            using OT = typename decltype(o)::type;
            hipLaunchKernelGGL((k_jvp_apply_mfma_f32<OT>), dim3(grid), dim3(kThreads), 0, stream,
                               static_cast<const float*>(q), static_cast<const float*>(qt), state,
                               static_cast<OT*>(out), static_cast<OT*>(outt), pl.N, pl.H, pl.HP, pl.L, pl.NB, pl.tile,
                               pl.tpb, eps);
        });
    } else if (pl.mfma16) {
        const unsigned grid = (unsigned)((size_t)pl.B * pl.HP * pl.NB * pl.tpb);
        const uint16_t *q16 = static_cast<const uint16_t*>(q), *qt16 = static_cast<const uint16_t*>(qt);
        by_dtype(pl.out_dtype, [&](auto o) {
            using OT = typename decltype(o)::type;
            if (pl.in_dtype == 2)
                hipLaunchKernelGGL((k_jvp_apply_mfma<true, OT>), dim3(grid), dim3(kThreads), 0, stream, q16, qt16, state,
                                   static_cast<OT*>(out), static_cast<OT*>(outt), pl.N, pl.H, pl.HP, pl.L, pl.NB,
                                   pl.tile, pl.tpb, eps);
            else
                hipLaunchKernelGGL((k_jvp_apply_mfma<false, OT>), dim3(grid), dim3(kThreads), 0, stream, q16, qt16,
                                   state, static_cast<OT*>(out), static_cast<OT*>(outt), pl.N, pl.H, pl.HP, pl.L,
                                   pl.NB, pl.tile, pl.tpb, eps);
        });
    } else {
        const unsigned grid = (unsigned)((size_t)pl.B * pl.H * pl.NB * pl.tpb);
        by_dtype(pl.in_dtype, [&](auto in) {
            by_dtype(pl.out_dtype, [&](auto o) {
                using IT = typename decltype(in)::type;
                using OT = typename decltype(o)::type;
                hipLaunchKernelGGL((k_jvp_apply_valu<IT, OT>), dim3(grid), dim3(kThreads), 0, stream,
                                   static_cast<const IT*>(q), static_cast<const IT*>(qt), state, static_cast<OT*>(out),
                                   static_cast<OT*>(outt), pl.N, pl.H, pl.L, pl.NB, pl.tpb, eps);
            });
        });
    }
    return hipGetLastError();
}

}  // namespace sana
