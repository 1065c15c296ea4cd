// gfx950 kernels of the LiteLA backward (gradients of the ReLU-kernel linear
// self-attention of "Sana: the autoencoder does more of the work than the
// linear attention", section "What LiteLA actually computes").
//
// With f_i = ReLU(q_i), a_n = ReLU(k_n) and P the state a query's block uses
// (rebuilt by the forward's state and merge kernels):
//   r_i = 1 / (f_i . P[:, D] + eps),  num_i = P[:, :D]^T f_i,  out_i = r_i num_i
//   u_i = dout_i r_i,   w_i = -r_i (dout_i . out_i)           (dL/dnum_i, dL/dden_i)
//   dq_i = [q_i > 0] (P [u_i | w_i])
//   G^(beta) = sum over queries of block beta of f_i [u_i | w_i]^T    (D x (D+1))
//   Ghat^(beta) = sum_{beta' >= beta} G^(beta')   (a key of block beta feeds the
//                 states of every block >= beta; for the non-causal operator
//                 there is one block)
//   dk_n = [k_n > 0] (Ghat [v_n | 1]),   dv_n = Ghat[:, :D]^T a_n
// The derivative of ReLU at 0 is taken as 0.  Everything accumulates in fp32;
// reductions run in fixed orders, so results are bitwise repeatable.  Head dims
// 16 and 64 use the forward kernels' view of a token row as 32-feature groups
// (a group holds two heads of 16; a head of 64 is two groups).
#include "linattn_device.h"

#include <type_traits>

namespace sana {
namespace {

__device__ __forceinline__ float ld(const float* p, long long i) { return load_in(p, i); }
__device__ __forceinline__ float ld(const uint16_t* p, long long i) { return load_in(p, i); }
__device__ __forceinline__ float ld(const _Float16* p, long long i) { return load_in(p, i); }
__device__ __forceinline__ void st(float* p, long long i, float x) { store_out(p, i, x); }
__device__ __forceinline__ void st(uint16_t* p, long long i, float x) { store_out(p, i, x); }
__device__ __forceinline__ void st(_Float16* p, long long i, float x) { store_out(p, i, x); }

// Tokens per work-group of the vector query kernel (one per thread; 64 for
// head dim 64, whose per-token LDS rows are twice as long) and of the vector
// key kernel.
template <int DD> struct VTok { static constexpr int value = DD == 2 * kD ? 64 : 256; };
constexpr int kTok = 256;

// ------------------------------------------------------------------ query pass, vector unit
// grid.x = ((b * H + h) * NB + beta) * tpb + tile; thread t = token
// blk0 + tile * TOK + t of block beta.  Writes dq and the tile's partial
// gradient state gpart[(b * H + h) * (NB * tpb) + beta * tpb + tile].
// Head dim DD (16, 32 or 64): states are DD x (DD + 1).
template <typename InT, typename GT, typename OutT, int DD>
__global__ __launch_bounds__(kThreads) void k_bwd_query_valu(
    const InT* __restrict__ q, const GT* __restrict__ dout, const float* __restrict__ state,
    OutT* __restrict__ dq, float* __restrict__ gpart, int N, int H, int L, int NB, int tpb, float eps) {
    constexpr int WW = DD + 1, SF = DD * WW, TOK = VTok<DD>::value;
    __shared__ float sP[SF];
    __shared__ float sf[TOK][DD + 1];    // f of each token (padded row)
    __shared__ float suw[TOK][WW];       // [u | w] of each token

    const int tile = blockIdx.x % tpb;
    const size_t bhb = blockIdx.x / tpb;          // (b * H + h) * NB + beta
    const int beta = (int)(bhb % NB);
    const size_t bh = bhb / NB;
    const int h = (int)(bh % H), b = (int)(bh / H);
    for (int e = threadIdx.x; e < SF; e += kThreads) sP[e] = state[bhb * SF + e];
    __syncthreads();

    const int blk0 = beta * L, blk1 = min(blk0 + L, N);
    const int t = threadIdx.x;
    const int row = blk0 + tile * TOK + t;
    if (t < TOK && row < blk1) {
        const long long base = (((long long)b * N + row) * H + h) * DD;
        float f[DD], u[DD];
#pragma unroll
        for (int j = 0; j < DD; ++j) {
            const float x = ld(q, base + j);
            f[j] = x > 0.f ? x : 0.f;
            sf[t][j] = f[j];
        }
        float den = 0.f;
#pragma unroll
        for (int j = 0; j < DD; ++j) den += f[j] * sP[j * WW + DD];
        const float r = 1.0f / (den + eps);
        float go = 0.f;   // dout . num
        for (int c = 0; c < DD; ++c) {
            float num = 0.f;
#pragma unroll
            for (int j = 0; j < DD; ++j) num += f[j] * sP[j * WW + c];
            const float g = ld(dout, base + c);
            go += g * num;
            u[c] = g * r;
            suw[t][c] = u[c];
        }
        const float w = -(r * r) * go;
        suw[t][DD] = w;
        for (int j = 0; j < DD; ++j) {
            float s = sP[j * WW + DD] * w;
#pragma unroll
            for (int c = 0; c < DD; ++c) s += sP[j * WW + c] * u[c];
            st(dq, base + j, ld(q, base + j) > 0.f ? s : 0.f);
        }
    } else if (t < TOK) {
        for (int j = 0; j < DD; ++j) sf[t][j] = 0.f;
        for (int c = 0; c < WW; ++c) suw[t][c] = 0.f;
    }
    __syncthreads();
    // partial gradient state of this tile: thread t owns entries t, t + 256, ...
    float* dst = gpart + (bhb * tpb + tile) * SF;   // (bh * NB + beta) * tpb + tile
    for (int e = t; e < SF; e += kThreads) {
        const int j = e / WW, c = e - j * WW;
        float s = 0.f;
        for (int tok = 0; tok < TOK; ++tok) s += sf[tok][j] * suw[tok][c];
        dst[e] = s;
    }
}

// ------------------------------------------------------------------ suffix merge
// grid.x = (b * H + h) * groups + m, groups = ceil(SF / 256); thread t owns
// entry e = m * 256 + t of the SF-float states.
// For beta = NB-1 down to 0: the block's tile partials are summed (in groups
// of 8 added as a fixed pairwise tree, the groups in order) and added to the
// running suffix sum, which is written as Ghat of block beta.  The loads of up
// to 16 partials are issued together (the kernel is a few load round trips
// long).

__device__ __forceinline__ float tree8(const float* x) {
    return ((x[0] + x[1]) + (x[2] + x[3])) + ((x[4] + x[5]) + (x[6] + x[7]));
}

__global__ __launch_bounds__(kThreads) void k_bwd_merge_suffix(const float* __restrict__ gpart,
                                                                float* __restrict__ ghat, int NB, int tpb, int SF) {
    const int groups = (SF + kThreads - 1) / kThreads;
    const size_t bh = blockIdx.x / groups;
    const int e = (blockIdx.x % groups) * kThreads + threadIdx.x;
    if (e >= SF) return;
    const float* src = gpart + bh * NB * tpb * SF + e;
    float* dst = ghat + bh * NB * SF + e;
    float acc = 0.f;
    if (tpb == 1) {
        // one partial per block: 16 blocks' loads at once, last block first
        for (int b1 = NB; b1 > 0; b1 -= 16) {
            float x[16];
#pragma unroll
            for (int i = 0; i < 16; ++i) x[i] = (b1 - 1 - i >= 0) ? src[(size_t)(b1 - 1 - i) * SF] : 0.f;
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                if (b1 - 1 - i >= 0) {
                    acc += 0.f + x[i];   // the block sum of one partial, as the general path forms it
                    dst[(size_t)(b1 - 1 - i) * SF] = acc;
                }
            }
        }
    } else if (tpb <= 8) {
        // 4 blocks' partials in flight at once, last block first (loads take
        // clamped, always valid indices and are unconditional; entries past
        // tpb then read as zero): the block-causal shape has 16 blocks of 4
        for (int b1 = NB; b1 > 0; b1 -= 4) {
            float x[4][8];
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
                for (int c = 0; c < 8; ++c)
                    x[j][c] = src[((size_t)max(b1 - 1 - j, 0) * tpb + min(c, tpb - 1)) * SF];
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
                for (int c = 0; c < 8; ++c) asm volatile("" : "+v"(x[j][c]));   // all in flight first
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                if (b1 - 1 - j >= 0) {
#pragma unroll
                    for (int c = 0; c < 8; ++c) x[j][c] = c < tpb ? x[j][c] : 0.f;
                    acc += 0.f + tree8(x[j]);   // the block sum as the general path forms it
                    dst[(size_t)(b1 - 1 - j) * SF] = acc;
                }
            }
        }
    } else if (tpb <= 16) {
        for (int beta = NB - 1; beta >= 0; --beta) {
            const float* blk = src + (size_t)beta * tpb * SF;
            float x[16];
#pragma unroll
            for (int i = 0; i < 16; ++i) x[i] = blk[(size_t)min(i, tpb - 1) * SF];
#pragma unroll
            for (int i = 0; i < 16; ++i) asm volatile("" : "+v"(x[i]));   // all in flight first
#pragma unroll
            for (int i = 0; i < 16; ++i) x[i] = i < tpb ? x[i] : 0.f;
            float bs = 0.f;
            bs += tree8(x);
            if (tpb > 8) bs += tree8(x + 8);
            acc += bs;
            dst[(size_t)beta * SF] = acc;
        }
    } else {
        for (int beta = NB - 1; beta >= 0; --beta) {
            const float* blk = src + (size_t)beta * tpb * SF;
            float bs = 0.f;
            for (int s0 = 0; s0 < tpb; s0 += 8) {
                float x[8];
#pragma unroll
                for (int i = 0; i < 8; ++i) x[i] = (s0 + i < tpb) ? blk[(size_t)(s0 + i) * SF] : 0.f;
                bs += tree8(x);
            }
            acc += bs;
            dst[(size_t)beta * SF] = acc;
        }
    }
}

// ------------------------------------------------------------------ key pass, vector unit
// grid.x = ((b * H + h) * NB + beta) * tpb + tile; thread t = key token
// blk0 + tile * 256 + t of block beta.  Head dim DD (16, 32 or 64).
template <typename InT, typename OutT, int DD>
__global__ __launch_bounds__(kThreads) void k_bwd_key_valu(
    const InT* __restrict__ k, const InT* __restrict__ v, const float* __restrict__ ghat,
    OutT* __restrict__ dk, OutT* __restrict__ dv, int N, int H, int L, int NB, int tpb) {
    constexpr int WW = DD + 1, SF = DD * WW;
    __shared__ float sG[SF];
    const int tile = blockIdx.x % tpb;
    const size_t bhb = blockIdx.x / tpb;
    const int beta = (int)(bhb % NB);
    const size_t bh = bhb / NB;
    const int h = (int)(bh % H), b = (int)(bh / H);
    for (int e = threadIdx.x; e < SF; e += kThreads) sG[e] = ghat[bhb * SF + e];
    __syncthreads();
    const int blk0 = beta * L, blk1 = min(blk0 + L, N);
    const int row = blk0 + tile * kTok + threadIdx.x;
    if (row >= blk1) return;
    const long long base = (((long long)b * N + row) * H + h) * DD;
    float a[DD], x[DD];
#pragma unroll
    for (int j = 0; j < DD; ++j) {
        const float kk = ld(k, base + j);
        a[j] = kk > 0.f ? kk : 0.f;
        x[j] = ld(v, base + j);
    }
    for (int j = 0; j < DD; ++j) {
        float s = sG[j * WW + DD];
#pragma unroll
        for (int c = 0; c < DD; ++c) s += sG[j * WW + c] * x[c];
        st(dk, base + j, a[j] > 0.f ? s : 0.f);
    }
    for (int c = 0; c < DD; ++c) {
        float s = 0.f;
#pragma unroll
        for (int j = 0; j < DD; ++j) s += a[j] * sG[j * WW + c];
        st(dv, base + c, s);
    }
}

// Split-term operands of P (natural layout, state_operands) of the two heads
// of a work-group, kept in LDS (too many to keep in registers next to the
// streaming tiles): [head][ks][sp] of 64 lanes x 16 bytes.
struct OperandLds {
    u32x4 v[2][2][3][64];
};

// ------------------------------------------------------------------ input tiles through LDS
// Two [B][N][H][D] 16-bit tensors, 64 tokens x 2 heads per tile, staged
// through LDS by the whole work-group (the state kernel's scheme): the next
// tile's global loads are issued into registers before the current tile is
// worked on, so their latency is covered by a whole tile of work.  LDS layout
// [tensor][head][token][32 x 16 bit]; the second head's rows are shifted by 64
// bytes so that both heads' 16-byte writes of one token use different banks.
constexpr int kTileTok = 64;
constexpr int kTileRow = 80;                       // bytes per token row: 64 + 16 keeps 16-byte reads of
                                                   // 8 consecutive rows in distinct banks
constexpr int kTileHead = kTileTok * kTileRow + 64;   // bytes per head
constexpr int kTileTensor = 2 * kTileHead;            // bytes per tensor
constexpr int kUPitch = 40;   // 16-bit elements per row of a u term tile: 80 bytes, as the staged rows (8-byte aligned transposing reads)

struct TileLoader {
    const uint16_t* x[2];   // the two tensors (the second may be null: one tensor only)
    long long hstride;      // elements per token row
    int b, N, h0, row_elems, t1;   // row_elems: elements of a row that exist (pieces past them read as zero)
    u32x4 r[2][2];          // [tensor][piece]: this thread's 2 pieces of 16 bytes

    // piece p (0..511) of a tile: part (p & 3), head ((p >> 2) & 1), token p >> 3.
    // A missing head (or the missing half of a 32-feature group) reads as zero.  Tokens past t1 read as the row t1 - 1:
    // their per-token results equal that row's (store_tile relies on it), and
    // code that sums over tokens must skip them.
    __device__ __forceinline__ void load(int t0) {
#pragma unroll
        for (int pi = 0; pi < 2; ++pi) {
            const int pc = threadIdx.x + kThreads * pi;
            const int part = pc & 3, hd = (pc >> 2) & 1, tok = pc >> 3;
            const int n = min(t0 + tok, t1 - 1);
            const int col = (h0 + hd) * kD + part * 8;
            const bool ok = col < row_elems;
            const long long off = ((long long)b * N + n) * hstride + (ok ? col : 0);
#pragma unroll
            for (int ts = 0; ts < 2; ++ts) {
                if (ts == 1 && !x[1]) break;
                const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(x[ts] + off));
                r[ts][pi] = ok ? v : (u32x4){0u, 0u, 0u, 0u};
            }
        }
    }
    __device__ __forceinline__ void store(uint8_t* lds) const {
#pragma unroll
        for (int pi = 0; pi < 2; ++pi) {
            const int pc = threadIdx.x + kThreads * pi;
            const int part = pc & 3, hd = (pc >> 2) & 1, tok = pc >> 3;
            const int o = hd * kTileHead + tok * kTileRow + part * 16;
#pragma unroll
            for (int ts = 0; ts < 2; ++ts) {
                if (ts == 1 && !x[1]) break;
                *reinterpret_cast<u32x4*>(lds + ts * kTileTensor + o) = r[ts][pi];
            }
        }
    }
};

// Bit r (r = 0..15) set when feature 8 (r / 4) + 4 g + r % 4 of a staged
// 16-bit row is > 0: the accumulator rows of lane (g, i) for token i.
__device__ __forceinline__ uint32_t positive_rows(const uint8_t* row, int g) {
    uint32_t m = 0;
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
        const u32x2 x = *reinterpret_cast<const u32x2*>(row + 16 * rr + 8 * g);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const short hv = (short)((e & 1) ? (x[e >> 1] >> 16) : (x[e >> 1] & 0xffffu));
            m |= (uint32_t)(hv > 0) << (4 * rr + e);
        }
    }
    return m;
}

// B operand of token `tok` of a staged tile: lane (g, i) gets features 8g..8g+7
// and 16+8g..16+8g+7 of tensor ts, head hh.
__device__ __forceinline__ void tile_operand(const uint8_t* lds, int ts, int hh, int tok, int g, u32x4& x0,
                                             u32x4& x1) {
    const uint8_t* row = lds + ts * kTileTensor + hh * kTileHead + tok * kTileRow + 16 * g;
    x0 = *reinterpret_cast<const u32x4*>(row);
    x1 = *reinterpret_cast<const u32x4*>(row + 32);
}

// ------------------------------------------------------------------ key pass, matrix cores
// grid.x = (b * HP + hp) * (NB * tpb) + beta * tpb + tile.  The work-group
// stages 64-key tiles of k and v (both heads) through LDS; wave w then handles
// head 2*hp + (w & 1) and keys 32 (w >> 1) .. + 31 of the tile.  With
// a = ReLU(k):
//   dv^T = Ghat_v^T a^T          (A = Ghat transposed, B = a)
//   da^T = Ghat_v v^T + Ghat_z   (A = Ghat natural,    B = v)
//   dk   = da masked by k > 0
// Head dims 16 and 64 take the forward's 32-feature groups ("heads" here: H of
// them, HP pairs; HR real heads): HD = 64, wave w computes the rows of group
// w & 1 of its head against all 64 features (four K-steps, the B operand from
// both groups' staged rows); HD = 16, the group's two heads as one
// block-diagonal state (state_operands).
template <bool F16, typename OutT, int HD>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(HD == 2 * kD ? 2 : 3, 8))) void k_bwd_key_mfma(
    const uint16_t* __restrict__ k, const uint16_t* __restrict__ v, const float* __restrict__ ghat,
    OutT* __restrict__ dk, OutT* __restrict__ dv, int N, int H, int HP, int HR, int L, int NB, int tile, int tpb) {
    constexpr int KS = KSteps<HD>::value, SW = HD + 1, SF = HD * SW;
    constexpr bool D64 = HD == 2 * kD, D16 = HD == kD / 2;
    __shared__ __attribute__((aligned(16))) uint8_t lds[2 * kTileTensor];
    __shared__ __attribute__((aligned(16))) float otile[4][32 * kPitch];                // fp32 out
    __shared__ __attribute__((aligned(16))) uint16_t ctile[2][2][32 * kPairRow];        // 16-bit out: [half][dv, dk]

    const int per_unit = NB * tpb;
    const int tau = blockIdx.x % per_unit;
    const int bhp = blockIdx.x / per_unit;
    const int hp = bhp % HP, b = bhp / HP;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int hh = wave & 1, th = wave >> 1, h = 2 * hp + hh;
    const int beta = tau / tpb, tib = tau - beta * tpb;
    const int blk0 = beta * L, blk1 = min(blk0 + L, N);
    const int t0 = blk0 + tib * tile, t1 = min(t0 + tile, blk1);
    const int g = lane >> 5, i = lane & 31;
    if (t0 >= t1) return;   // uniform over the work-group

    // this wave's group: Ghat as split-term operands in both layouts, Ghat[:, D]
    const int hs = min(h, H - 1);   // a missing second group computes on the first (never stored)
    auto head_G = [&](int hr) { return ghat + (((size_t)b * HR + hr) * NB + beta) * SF; };
    const int grp = D64 ? hp : hs;
    u32x4 gt[KS][3], gn[KS][3];
    state_operands<HD>(head_G, grp, hh, HR, lane, true, gt);
    state_operands<HD>(head_G, grp, hh, HR, lane, false, gn);
    float gz[16];   // Ghat[row][HD] at this lane's accumulator rows 8 (r / 4) + 4 g + r % 4
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        const int row = 8 * (r >> 2) + 4 * g + (r & 3);
        if constexpr (D16) {
            const int hr = 2 * hs + (row >> 4);
            gz[r] = hr < HR ? head_G(hr)[(row & 15) * SW + HD] : 0.f;
        } else {
            gz[r] = head_G(grp)[((D64 ? kD * hh : 0) + row) * SW + HD];
        }
    }

    const long long hstride = (long long)HR * HD;
    const int ncols = min(32, HR * HD - h * kD);                 // fp32 out: columns of this group that exist
    const int nchunk = min(8, (HR * HD - 2 * hp * kD) / 8);      // 16-bit out: 16-byte chunks of the line
    TileLoader ld = {{k, v}, hstride, b, N, 2 * hp, HR * HD, t1, {}};
    float* ot = otile[wave];
    ld.load(t0);
    for (int tt0 = t0; tt0 < t1; tt0 += kTileTok) {
        __syncthreads();   // the previous tile has been consumed
        ld.store(lds);
        __syncthreads();
        if (tt0 + kTileTok < t1) ld.load(tt0 + kTileTok);   // in flight during this tile's work

        const int tt = tt0 + 32 * th;   // first key of this wave's half
        const int n = min(32, t1 - tt);
        if constexpr (sizeof(OutT) == 4) {
            if (n <= 0 || h >= H) continue;
        }
        // (16-bit out: every wave computes, so that the work-group barrier
        // below is reached by all; rows past the range hold the clamped last
        // row and a missing head computes on zeros, never stored)
        // B operands: features 16 ks + 8 g .. of the key (HD = 64: K-steps 0, 1
        // from group 0's staged row, 2, 3 from group 1's)
        u32x4 a[KS], vb[KS];
#pragma unroll
        for (int gi = 0; gi < KS / 2; ++gi) {
            const int gr = D64 ? gi : hh;
            tile_operand(lds, 0, gr, 32 * th + i, g, a[2 * gi], a[2 * gi + 1]);
            tile_operand(lds, 1, gr, 32 * th + i, g, vb[2 * gi], vb[2 * gi + 1]);
        }
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) a[ks] = relu_bf16x8(a[ks]);
        const uint32_t mask = positive_rows(lds + hh * kTileHead + (32 * th + i) * kTileRow, g);

        f32x16 accv = {};
        accv = mma_split_ks<F16, KS>(gt, a, accv);
        f32x16 acck = {};
        acck = mma_split_ks<F16, KS>(gn, vb, acck);
#pragma unroll
        for (int r = 0; r < 16; ++r) acck[r] = ((mask >> r) & 1u) ? acck[r] + gz[r] : 0.f;
        if constexpr (sizeof(OutT) == 4) {
            store_tile<OutT>(ot, accv, lane, n, [&](int t) { return dv + ((long long)b * N + tt + t) * hstride + h * kD; },
                             ncols);
            store_tile<OutT>(ot, acck, lane, n, [&](int t) { return dk + ((long long)b * N + tt + t) * hstride + h * kD; },
                             ncols);
        } else {
            // both heads of a key share a 128-byte line of dk and of dv
            put_pair_tile<OutT>(ctile[th][0], accv, lane, hh);
            put_pair_tile<OutT>(ctile[th][1], acck, lane, hh);
            __syncthreads();
            // wave (th, hh) stores rows 16 hh .. 16 hh + 15 of its half; rows
            // past the range repeat the last row (same bits)
            auto row = [&](OutT* base) {
                return [=](int r) {
                    return reinterpret_cast<uint16_t*>(base + ((long long)b * N + min(tt + r, t1 - 1)) * hstride + 2 * hp * kD);
                };
            };
            store_pair_rows<OutT>(ctile[th][0], lane, 16 * hh, nchunk, row(dv));
            store_pair_rows<OutT>(ctile[th][1], lane, 16 * hh, nchunk, row(dk));
            // the next tile's first barrier keeps the pair tiles until these reads are done
        }
    }
}

// The key pass for fp32 k and v: the work-group, waves and sub-tiles of the
// 16-bit kernel, but each wave reads its own 32 keys straight from global
// memory in the operand layout (the next sub-tile's loads issued before this
// one's work), and k, a = ReLU(k) and v enter the MFMAs as three bf16 terms.
// Head dim 16 as in the 16-bit kernel (groups of two heads, block-diagonal
// Ghat; a lone head's other half is neither read nor stored).
template <typename OutT, int HD>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 8))) void k_bwd_key_mfma_f32(
    const float* __restrict__ k, const float* __restrict__ v, const float* __restrict__ ghat,
    OutT* __restrict__ dk, OutT* __restrict__ dv, int N, int H, int HP, int HR, int L, int NB, int tile, int tpb) {
    static_assert(HD == kD || HD == kD / 2, "head dims 32 and 16");
    constexpr bool D16 = HD == kD / 2;
    constexpr int SW = HD + 1, SF = HD * SW;
    __shared__ __attribute__((aligned(16))) float otile[4][32 * kPitch];                // fp32 out
    __shared__ __attribute__((aligned(16))) uint16_t ctile[2][2][32 * kPairRow];        // 16-bit out: [half][dv, dk]

    const int per_unit = NB * tpb;
    const int tau = blockIdx.x % per_unit;
    const int bhp = blockIdx.x / per_unit;
    const int hp = bhp % HP, b = bhp / HP;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int hh = wave & 1, th = wave >> 1, h = 2 * hp + hh;
    const int beta = tau / tpb, tib = tau - beta * tpb;
    const int blk0 = beta * L, blk1 = min(blk0 + L, N);
    const int t0 = blk0 + tib * tile, t1 = min(t0 + tile, blk1);
    const int g = lane >> 5, i = lane & 31;
    if (t0 >= t1) return;   // uniform over the work-group

    const int hs = min(h, H - 1);   // a missing second group computes on the first (never stored)
    auto head_G = [&](int hr) { return ghat + (((size_t)b * HR + hr) * NB + beta) * SF; };
    u32x4 gt[2][3], gn[2][3];
    state_operands<HD>(head_G, hs, 0, HR, lane, true, gt);
    state_operands<HD>(head_G, hs, 0, HR, lane, false, gn);
    float gz[16];   // Ghat[row][HD] at this lane's accumulator rows
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        const int row = 8 * (r >> 2) + 4 * g + (r & 3);
        if constexpr (D16) {
            const int hr = 2 * hs + (row >> 4);
            gz[r] = hr < HR ? head_G(hr)[(row & 15) * SW + HD] : 0.f;
        } else {
            gz[r] = head_G(hs)[row * SW + HD];
        }
    }

    const long long hstride = (long long)HR * HD;
    const bool upper = HR * HD - hs * kD > kD / 2;                 // the group's second half exists
    const int ncols = min(32, HR * HD - h * kD);                   // fp32 out: columns of this group that exist
    const int nchunk = min(8, (HR * HD - 2 * hp * kD) / 8);        // 16-bit out: 16-byte chunks of the line
    auto row_of = [&](const float* x, int tt) { return x + ((long long)b * N + min(tt + i, t1 - 1)) * hstride + hs * kD; };
    float* ot = otile[wave];
    F32Operand kc, vc;
    kc.load(row_of(k, t0 + 32 * th), g, upper);
    vc.load(row_of(v, t0 + 32 * th), g, upper);
    for (int tt0 = t0; tt0 < t1; tt0 += kTileTok) {
        const int tt = tt0 + 32 * th;   // first key of this wave's half
        const int n = min(32, t1 - tt);
        F32Operand kn, vn;
        const bool more = tt0 + kTileTok < t1;
        if (more) {   // in flight during this sub-tile's work
            kn.load(row_of(k, tt + kTileTok), g, upper);
            vn.load(row_of(v, tt + kTileTok), g, upper);
        }
        // (rows past the range hold the clamped last row: with 16-bit outputs
        // every wave computes, so that the work-group barrier below is reached
        // by all)
        if (sizeof(OutT) == 2 || (n > 0 && h < H)) {
            const uint32_t mask = kc.positive(g);
            f32x16 accv = {};
            accv = mma_split3(gt, kc, true, accv);
            f32x16 acck = {};
            acck = mma_split3(gn, vc, false, acck);
#pragma unroll
            for (int r = 0; r < 16; ++r)
                acck[r] = ((mask >> (8 * (r >> 2) + 4 * g + (r & 3))) & 1u) ? acck[r] + gz[r] : 0.f;
            if constexpr (sizeof(OutT) == 4) {
                store_tile<OutT>(ot, accv, lane, n,
                                 [&](int t) { return dv + ((long long)b * N + tt + t) * hstride + h * kD; }, ncols);
                store_tile<OutT>(ot, acck, lane, n,
                                 [&](int t) { return dk + ((long long)b * N + tt + t) * hstride + h * kD; }, ncols);
            } else {
                __syncthreads();   // the previous sub-tile's pair tiles have been stored
                put_pair_tile<OutT>(ctile[th][0], accv, lane, hh);
                put_pair_tile<OutT>(ctile[th][1], acck, lane, hh);
                __syncthreads();
                auto row = [&](OutT* base) {
                    return [=](int r) {
                        return reinterpret_cast<uint16_t*>(base + ((long long)b * N + min(tt + r, t1 - 1)) * hstride + 2 * hp * kD);
                    };
                };
                store_pair_rows<OutT>(ctile[th][0], lane, 16 * hh, nchunk, row(dv));
                store_pair_rows<OutT>(ctile[th][1], lane, 16 * hh, nchunk, row(dk));
            }
        }
        if (more) {
            kc = kn;
            vc = vn;
        }
    }
}

// The key pass for fp32 k and v at head dim 64: the 16-bit dim-64 kernel's
// work-groups and waves (wave w: the rows of group w & 1 of the head, keys
// 32 (w >> 1) .. of each 64-key step), each wave reading both groups' k and v
// rows straight from global memory in the operand layout (no loads ahead: the
// four K-steps' operands of both layouts take the registers), k, a = ReLU(k)
// and v split into three bf16 terms.
template <typename OutT>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 8))) void k_bwd_key_mfma_f32_64(
    const float* __restrict__ k, const float* __restrict__ v, const float* __restrict__ ghat,
    OutT* __restrict__ dk, OutT* __restrict__ dv, int N, int HR, int L, int NB, int tile, int tpb) {
    constexpr int HD = 2 * kD, KS = KSteps<HD>::value, SW = HD + 1, SF = HD * SW;
    __shared__ __attribute__((aligned(16))) float otile[4][32 * kPitch];                // fp32 out
    __shared__ __attribute__((aligned(16))) uint16_t ctile[2][2][32 * kPairRow];        // 16-bit out: [half][dv, dk]

    const int per_unit = NB * tpb;
    const int tau = blockIdx.x % per_unit;
    const int bh = blockIdx.x / per_unit;
    const int hq = bh % HR, b = bh / HR;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int a = wave & 1, th = wave >> 1;
    const int beta = tau / tpb, tib = tau - beta * tpb;
    const int blk0 = beta * L, blk1 = min(blk0 + L, N);
    const int t0 = blk0 + tib * tile, t1 = min(t0 + tile, blk1);
    const int g = lane >> 5, i = lane & 31;
    if (t0 >= t1) return;   // uniform over the work-group

    const float* G = ghat + (((size_t)b * HR + hq) * NB + beta) * SF;
    auto head_G = [&](int) { return G; };
    u32x4 gt[KS][3], gn[KS][3];
    state_operands<HD>(head_G, hq, a, HR, lane, true, gt);
    state_operands<HD>(head_G, hq, a, HR, lane, false, gn);
    float gz[16];   // Ghat[32 a + row][64] at this lane's accumulator rows
#pragma unroll
    for (int r = 0; r < 16; ++r) gz[r] = G[(kD * a + 8 * (r >> 2) + 4 * g + (r & 3)) * SW + HD];

    const long long hstride = (long long)HR * HD;
    auto row_of = [&](const float* x, int tt) { return x + ((long long)b * N + min(tt + i, t1 - 1)) * hstride + hq * HD; };
    float* ot = otile[wave];
    for (int tt0 = t0; tt0 < t1; tt0 += kTileTok) {
        const int tt = tt0 + 32 * th;   // first key of this wave's half
        const int n = min(32, t1 - tt);
        // (rows past the range hold the clamped last row: with 16-bit outputs
        // every wave computes, so that the work-group barriers are reached by all)
        if (sizeof(OutT) == 2 || n > 0) {
            F32Operand kx[2], vx[2];   // features 0..31 and 32..63 of the key
#pragma unroll
            for (int gi = 0; gi < 2; ++gi) {
                kx[gi].load(row_of(k, tt) + kD * gi, g);
                vx[gi].load(row_of(v, tt) + kD * gi, g);
            }
            const uint32_t m0 = kx[0].positive(g), m1 = kx[1].positive(g);
            const uint32_t mask = a ? m1 : m0;   // bit j: feature 32 a + j of the key > 0
            f32x16 accv = {}, acck = {};
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                u32x4 t[3];
                split_half(kx[ks >> 1], ks & 1, true, t);
                accv = mma_terms(gt[ks], t, accv);
                split_half(vx[ks >> 1], ks & 1, false, t);
                acck = mma_terms(gn[ks], t, acck);
            }
#pragma unroll
            for (int r = 0; r < 16; ++r)
                acck[r] = ((mask >> (8 * (r >> 2) + 4 * g + (r & 3))) & 1u) ? acck[r] + gz[r] : 0.f;
            const int col = (2 * hq + a) * kD;
            if constexpr (sizeof(OutT) == 4) {
                store_tile<OutT>(ot, accv, lane, n, [&](int t) { return dv + ((long long)b * N + tt + t) * hstride + col; });
                store_tile<OutT>(ot, acck, lane, n, [&](int t) { return dk + ((long long)b * N + tt + t) * hstride + col; });
            } else {
                __syncthreads();   // the previous step's pair tiles have been stored
                put_pair_tile<OutT>(ctile[th][0], accv, lane, a);
                put_pair_tile<OutT>(ctile[th][1], acck, lane, a);
                __syncthreads();
                auto row = [&](OutT* base) {
                    return [=](int r) {
                        return reinterpret_cast<uint16_t*>(base + ((long long)b * N + min(tt + r, t1 - 1)) * hstride + hq * HD);
                    };
                };
                store_pair_rows<OutT>(ctile[th][0], lane, 16 * a, 8, row(dv));
                store_pair_rows<OutT>(ctile[th][1], lane, 16 * a, 8, row(dk));
            }
        }
    }
}

// ------------------------------------------------------------------ query pass, matrix cores
// Upstream gradient of one token in the accumulator layout: lane (g, i) gets
// features 8 rr + 4 g .. + 3 (rr = 0..3) of its token.
template <typename GT> struct GradRow;
template <> struct GradRow<float> {
    f32x4 x[4];
    __device__ __forceinline__ void load_lds(const uint8_t*, int) {}   // fp32 rows are not staged
    // rows rr >= nrr (features 16.. of a group that is a lone head of dim 16) read as zero
    __device__ __forceinline__ void load(const float* row, int g, int nrr = 4) {
#pragma unroll
        for (int rr = 0; rr < 4; ++rr)
            x[rr] = rr < nrr ? *reinterpret_cast<const f32x4*>(row + 8 * rr + 4 * g)
                             : (f32x4){0.f, 0.f, 0.f, 0.f};
    }
    __device__ __forceinline__ float at(int rr, int e) const { return x[rr][e]; }
};
template <> struct GradRow<uint16_t> {
    u32x2 x[4];
    // from a staged LDS row of 32 x 16 bit
    __device__ __forceinline__ void load_lds(const uint8_t* row, int g) {
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) x[rr] = *reinterpret_cast<const u32x2*>(row + 16 * rr + 8 * g);
    }
    __device__ __forceinline__ void load(const uint16_t* row, int g, int nrr = 4) {
#pragma unroll
        for (int rr = 0; rr < 4; ++rr)
            x[rr] = rr < nrr ? *reinterpret_cast<const u32x2*>(row + 8 * rr + 4 * g)
                             : (u32x2){0u, 0u};
    }
    __device__ __forceinline__ float at(int rr, int e) const {
        const uint32_t w = x[rr][e >> 1];
        return (e & 1) ? hi_bf16(w) : lo_bf16(w);
    }
};
template <> struct GradRow<_Float16> {
    u32x2 x[4];
    __device__ __forceinline__ void load_lds(const uint8_t* row, int g) {
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) x[rr] = *reinterpret_cast<const u32x2*>(row + 16 * rr + 8 * g);
    }
    __device__ __forceinline__ void load(const _Float16* row, int g, int nrr = 4) {
#pragma unroll
        for (int rr = 0; rr < 4; ++rr)
            x[rr] = rr < nrr ? *reinterpret_cast<const u32x2*>(row + 8 * rr + 4 * g)
                             : (u32x2){0u, 0u};
    }
    __device__ __forceinline__ float at(int rr, int e) const {
        const uint32_t w = x[rr][e >> 1];
        return f16_to_f32((uint16_t)((e & 1) ? (w >> 16) : (w & 0xffffu)));
    }
};

// grid.x = (b * HP + hp) * (NB * tpb) + beta * tpb + tile.  Wave w handles head
// 2*hp + (w & 1) and every other 32-query sub-tile (w >> 1).  Per sub-tile,
// with f = ReLU(q), P the block's state, P_v = P[:, :D] and z = P[:, D]:
//   den = f . z in fp32; r = 1 / (den + eps); u = dout r
//   m^T = P_v dout^T on MFMA (A = P natural; B = the 16-bit dout, exact, or
//   for fp32 dout u as three bf16 terms, products below 2^-24 dropped, which
//   gives m = P_v u = r P_v dout directly)
//   dout . num = f . (P_v dout) (no numerator product is needed), so
//   w = -r^2 (f . P_v dout); dq = [q > 0] (r P_v dout + w z)
//   G_v += f^T u  (fp32 MFMA 32x32x2, tokens as the reduction dimension, two
//   per instruction: u and w from the wave's LDS tiles, f from the staged q)
//   G_z += f^T w  (an fp32 dot product per lane on the vector unit)
// f, the mask and dout are read in the accumulator layout (lane (g, i): token
// i, features 8 rr + 4 g + e), the layout of the MFMA result.
// The two waves of a head then add their G in a fixed order and write the
// tile's partial gradient state.
//
// Head dim 16 (HD = 16, 16-bit q): a 32-feature group holds two heads (H
// counts the groups, HR the heads).  P is the group's block-diagonal state
// (state_operands), so m = P_v dout keeps the heads apart; every per-token
// scalar (r, w) exists per head (rows 0..15 the first, 16..31 the second),
// and of the group's G only the diagonal 16 x 16 blocks are written.
template <typename QT, typename GT, typename OutT, int HD>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(sizeof(QT) == 2 ? 3 : 2, 8))) void k_bwd_query_mfma(
    const QT* __restrict__ q, const GT* __restrict__ dout, const float* __restrict__ state,
    OutT* __restrict__ dq, float* __restrict__ gpart, int N, int H, int HP, int HR, int L, int NB, int tile, int tpb,
    float eps) {
    constexpr bool D16 = HD == kD / 2;
    static_assert(HD == kD || D16, "head dims 32 and 16");
    constexpr int SW = HD + 1, SF = HD * SW;
    // 16-bit q (and 16-bit dout) are staged through LDS by the work-group;
    // fp32 q is read by each wave straight from global memory, its f = ReLU(q)
    // kept in an fp32 LDS tile per wave (in the staging area) for the G sums
    constexpr bool kStage = sizeof(QT) == 2;
    __shared__ OperandLds opnd;                                     // P natural split terms, both heads
    __shared__ __attribute__((aligned(16))) float pzs[2][32];       // P[:, D] of each head
    __shared__ __attribute__((aligned(16))) float ut[4][32 * kPitch];   // u tile, then the dq tile
    __shared__ __attribute__((aligned(16))) float wv[4][2][32];     // w of each token (head dim 16: of each head)
    __shared__ __attribute__((aligned(16))) uint8_t lds_in[2 * kTileTensor];   // staged q (and 16-bit dout)
    static_assert(sizeof(lds_in) >= 4 * 32 * kPitch * sizeof(float), "f tiles exceed the staging area");

    const int per_unit = NB * tpb;
    const int tau = blockIdx.x % per_unit;
    const int bhp = blockIdx.x / per_unit;
    const int hp = bhp % HP, b = bhp / HP;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int hh = wave & 1, h = 2 * hp + hh;
    const int beta = tau / tpb, tib = tau - beta * tpb;
    const int blk0 = beta * L, blk1 = min(blk0 + L, N);
    const int t0 = blk0 + tib * tile, t1 = min(t0 + tile, blk1);
    const int g = lane >> 5, i = lane & 31;

    auto head_P = [&](int hr) { return state + (((size_t)b * HR + hr) * NB + beta) * SF; };
    if (wave < 2 && h < H) {
        u32x4 t[2][3];
        state_operands<HD>(head_P, h, 0, HR, lane, false, t);
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
#pragma unroll
            for (int sp = 0; sp < 3; ++sp) opnd.v[hh][ks][sp][lane] = t[ks][sp];
        if (lane < 32) {
            if constexpr (D16) {
                const int hr = 2 * h + (lane >> 4);
                pzs[hh][lane] = hr < HR ? head_P(hr)[(lane & 15) * SW + HD] : 0.f;
            } else {
                pzs[hh][lane] = head_P(h)[lane * SW + HD];
            }
        }
    }
    __syncthreads();

    const long long hstride = (long long)HR * HD;
    const int ncols = min(32, HR * HD - h * kD);   // columns of this group that exist (16: a lone head of dim 16)
    const bool active = h < H && t0 < t1;
    float* ot = ut[wave];
    float* wl = wv[wave][0];
    f32x16 accG = {};
    float gz_acc = 0.f;   // lane (g, j): sum over this lane's tokens of f_j w

    struct Tile {
        GradRow<QT> qa;    // q of this lane's token in the accumulator layout
        u32x4 g0, g1;      // 16-bit dout in the operand layout
        GradRow<GT> gr;    // dout in the accumulator layout
    };
    constexpr bool kDoutOperand = sizeof(GT) == 2;   // 16-bit dout is the B operand as it is
    float* ft = reinterpret_cast<float*>(lds_in) + wave * 32 * kPitch;   // fp32 q: f tile of this wave
    auto body = [&](int tt, const Tile& x) {
        asm volatile("" ::: "memory");   // keep the LDS operands in LDS (see the key kernel)
        const int n = min(32, t1 - tt);
        // f at this lane's accumulator rows (decoded where used, to keep few
        // registers live; f > 0 is the mask q > 0); z = P[:, D] at the same rows
        auto fa = [&](int rr, int e) { return relu_f32(x.qa.at(rr, e)); };
        auto zrow = [&](int rr) { return *reinterpret_cast<const f32x4*>(&pzs[hh][8 * rr + 4 * g]); };
        float dp[2] = {0.f, 0.f};   // head dim 16: per head (rows rr < 2, rr >= 2)
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
            const f32x4 z = zrow(rr);
            float& d = dp[D16 && rr >= 2];
#pragma unroll
            for (int e = 0; e < 4; ++e) d = fmaf(fa(rr, e), z[e], d);
        }
        float rh[2];
#pragma unroll
        for (int s2 = 0; s2 < (D16 ? 2 : 1); ++s2) rh[s2] = 1.0f / (dp[s2] + __shfl_xor(dp[s2], 32) + eps);
        if constexpr (!D16) rh[1] = rh[0];
        auto rrow = [&](int rr) { return rh[D16 && rr >= 2]; };   // r of the head of rows 8 rr ..

        // u to the LDS tile (token-major); for fp32 q also f
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
            f32x4 u4;
#pragma unroll
            for (int e = 0; e < 4; ++e) u4[e] = x.gr.at(rr, e) * rrow(rr);
            *reinterpret_cast<f32x4*>(ot + i * kPitch + 8 * rr + 4 * g) = u4;
            if constexpr (!kStage) {
                f32x4 f4;
#pragma unroll
                for (int e = 0; e < 4; ++e) f4[e] = fa(rr, e);
                *reinterpret_cast<f32x4*>(ft + i * kPitch + 8 * rr + 4 * g) = f4;
            }
        }

        f32x16 acc = {};
        float rs[2];   // per-token (per-head) factor of the MFMA result: acc * rs = r P_v dout
        {
            u32x4 A[2][3];
#pragma unroll
            for (int ks = 0; ks < 2; ++ks)
#pragma unroll
                for (int sp = 0; sp < 3; ++sp) A[ks][sp] = opnd.v[hh][ks][sp][lane];
            if constexpr (kDoutOperand) {
                const u32x4 gb[2] = {x.g0, x.g1};
                acc = mma_split_ks<std::is_same<GT, _Float16>::value, 2>(A, gb, acc);
                rs[0] = rh[0];
                rs[1] = rh[1];
            } else {
                // u read back in the operand layout (channels 16 ks + 8 g ..)
                // and split into three bf16 terms
                __builtin_amdgcn_wave_barrier();
                asm volatile("" ::: "memory");
                u32x4 ub[2][3];
#pragma unroll
                for (int ks = 0; ks < 2; ++ks) {
                    float uu[8];
                    const f32x4 a4 = *reinterpret_cast<const f32x4*>(ot + i * kPitch + 16 * ks + 8 * g);
                    const f32x4 b4 = *reinterpret_cast<const f32x4*>(ot + i * kPitch + 16 * ks + 8 * g + 4);
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        uu[e] = a4[e];
                        uu[4 + e] = b4[e];
                    }
                    split3_trunc_f32x8(uu, ub[ks]);
                }
#pragma unroll
                for (int ks = 0; ks < 2; ++ks) {
                    // products of split terms in increasing size; those below 2^-24 are dropped
                    acc = mfma_bf16(A[ks][0], ub[ks][2], acc);
                    acc = mfma_bf16(A[ks][1], ub[ks][1], acc);
                    acc = mfma_bf16(A[ks][2], ub[ks][0], acc);
                    acc = mfma_bf16(A[ks][0], ub[ks][1], acc);
                    acc = mfma_bf16(A[ks][1], ub[ks][0], acc);
                    acc = mfma_bf16(A[ks][0], ub[ks][0], acc);
                }
                rs[0] = rs[1] = 1.f;
            }
        }
        // w = -r (dout . out) = -r (f . acc rs), per head for head dim 16
        float go[2] = {0.f, 0.f};
#pragma unroll
        for (int rr = 0; rr < 4; ++rr)
#pragma unroll
            for (int e = 0; e < 4; ++e) go[D16 && rr >= 2] = fmaf(fa(rr, e), acc[4 * rr + e], go[D16 && rr >= 2]);
        float wh[2];
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) {
            const float gs = go[s2] + __shfl_xor(go[s2], 32);
            wh[s2] = -rh[s2] * (gs * rs[s2]);
        }
        if constexpr (!D16) wh[1] = wh[0];
        if (g == 0) {   // 0 past the range: the G_z sum skips those tokens
            wl[i] = i < n ? wh[0] : 0.f;
            if constexpr (D16) wl[32 + i] = i < n ? wh[1] : 0.f;
        }
        __builtin_amdgcn_wave_barrier();
        asm volatile("" ::: "memory");   // phase boundary: keeps each phase's LDS reads in its phase

        // G_v += f^T u on fp32 MFMA (32 x 32 x 2: token pair m, lane (g, x)
        // supplies f and u of token 2 m + g at feature x), G_z += f^T w on
        // the vector unit; tokens past the range are skipped
        const uint8_t* qrows = lds_in + hh * kTileHead + 32 * (wave >> 1) * kTileRow;   // this sub-tile's q rows
        auto gather = [&](int tok, float& fv, float& uv, float& wv_) {
            if constexpr (kStage) {
                const uint16_t fb = *reinterpret_cast<const uint16_t*>(qrows + tok * kTileRow + 2 * i);
                const uint16_t fr = relu_16(fb);
                fv = std::is_same<QT, _Float16>::value ? f16_to_f32(fr) : bf16_to_f32(fr);
            } else {
                fv = ft[tok * kPitch + i];
            }
            uv = ot[tok * kPitch + i];
            wv_ = wl[(D16 && i >= 16 ? 32 : 0) + tok];   // w of the head of feature i
        };
        if (n == 32) {   // a whole sub-tile (every one but a range's last)
#pragma unroll
            for (int m = 0; m < 16; ++m) {
                float fv, uv, wv_;
                gather(2 * m + g, fv, uv, wv_);
                accG = __builtin_amdgcn_mfma_f32_32x32x2f32(fv, uv, accG, 0, 0, 0);
                gz_acc = fmaf(fv, wv_, gz_acc);
            }
        } else {
#pragma unroll
            for (int m = 0; m < 16; ++m) {
                const int tok = 2 * m + g;
                const bool ok = tok < n;
                float fv, uv, wv_;
                gather(tok, fv, uv, wv_);
                const float fa_ = ok ? fv : 0.f;
                accG = __builtin_amdgcn_mfma_f32_32x32x2f32(fa_, ok ? uv : 0.f, accG, 0, 0, 0);
                gz_acc = fmaf(fa_, ok ? wv_ : 0.f, gz_acc);
            }
        }

#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
            const f32x4 z = zrow(rr);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int rg = 4 * rr + e;
                const int s2 = D16 && rr >= 2;
                acc[rg] = fa(rr, e) > 0.f ? fmaf(z[e], wh[s2], acc[rg] * rs[s2]) : 0.f;
            }
        }
        __builtin_amdgcn_wave_barrier();
        asm volatile("" ::: "memory");   // every read of the u tile precedes the dq tile's writes
        store_tile<OutT>(ot, acc, lane, n, [&](int t) { return dq + ((long long)b * N + tt + t) * hstride + h * kD; },
                         ncols);
    };

    if constexpr (!kStage) {
        // fp32 q: each wave reads its sub-tiles' rows itself, the next
        // sub-tile's loads in flight during this one's work
        // (a group that is a lone head of dim 16 reads only its first 16 features)
        auto load = [&](int tt, Tile& x) {
            const long long row = ((long long)b * N + min(tt + i, t1 - 1)) * hstride + h * kD;
            x.qa.load(reinterpret_cast<const float*>(q) + row, g, ncols / 8);
            if constexpr (kDoutOperand) {
                x.g0 = *reinterpret_cast<const u32x4*>(dout + row + 8 * g);
                x.g1 = ncols > 16 ? *reinterpret_cast<const u32x4*>(dout + row + 16 + 8 * g)
                                  : (u32x4){0u, 0u, 0u, 0u};
            }
            x.gr.load(dout + row, g, ncols / 8);
        };
        if (active && t0 + 32 * (wave >> 1) < t1) {
            Tile cur;
            load(t0 + 32 * (wave >> 1), cur);
            for (int tt = t0 + 32 * (wave >> 1); tt < t1; tt += kTileTok) {
                Tile nxt;
                const bool more = tt + kTileTok < t1;
                if (more) load(tt + kTileTok, nxt);
                body(tt, cur);
                if (more) cur = nxt;
            }
        }
    } else if (t0 < t1) {   // uniform over the work-group
        const uint16_t* dsrc = kDoutOperand ? reinterpret_cast<const uint16_t*>(dout) : nullptr;
        TileLoader ld = {{reinterpret_cast<const uint16_t*>(q), dsrc}, hstride, b, N, 2 * hp, HR * HD, t1, {}};
        ld.load(t0);
        for (int tt0 = t0; tt0 < t1; tt0 += kTileTok) {
            __syncthreads();   // the previous tile has been consumed
            ld.store(lds_in);
            __syncthreads();
            if (tt0 + kTileTok < t1) ld.load(tt0 + kTileTok);   // in flight during this tile's work
            const int tt = tt0 + 32 * (wave >> 1);
            if (!active || tt >= t1) continue;
            Tile x;
            const uint8_t* qrow = lds_in + hh * kTileHead + (32 * (wave >> 1) + i) * kTileRow;
            x.qa.load_lds(qrow, g);
            if constexpr (kDoutOperand) {
                tile_operand(lds_in, 1, hh, 32 * (wave >> 1) + i, g, x.g0, x.g1);
                x.gr.load_lds(lds_in + kTileTensor + hh * kTileHead + (32 * (wave >> 1) + i) * kTileRow, g);
            } else {
                const int row = min(tt + i, t1 - 1);
                x.gr.load(dout + ((long long)b * N + row) * hstride + h * kD, g, ncols / 8);
            }
            body(tt, x);
        }
    }

    // the two waves of a head add their G in a fixed order; the LDS operands
    // are no longer needed, so their space holds the second wave's G
    __syncthreads();
    // G_z of lane j: the sum of its two token halves (the same in both lanes:
    // fp32 addition commutes)
    const float gz = gz_acc + __shfl_xor(gz_acc, 32);
    float* red = reinterpret_cast<float*>(&opnd);   // [head][16][64] G, then [head][32] G_z
    if (wave >= 2) {
#pragma unroll
        for (int rg = 0; rg < 16; ++rg) red[(hh * 16 + rg) * 64 + lane] = accG[rg];
        if (lane < 32) red[2 * 16 * 64 + hh * 32 + lane] = gz;
    }
    __syncthreads();
    if (wave < 2 && h < H) {
        auto part_of = [&](int hr) { return gpart + ((((size_t)b * HR + hr) * NB + beta) * tpb + tib) * SF; };
        if constexpr (D16) {
            // the diagonal 16 x 16 blocks: rows 0..15 (rg < 8) and the lanes of
            // columns 0..15 are the first head's, the rest the second's
#pragma unroll
            for (int rg = 0; rg < 16; ++rg) {
                const int j = 8 * (rg >> 2) + 4 * g + (rg & 3), hr = 2 * h + (rg >> 3);
                if ((i >> 4) == (rg >> 3) && hr < HR)
                    part_of(hr)[(j & 15) * SW + (i & 15)] = accG[rg] + red[(hh * 16 + rg) * 64 + lane];
            }
            if (lane < 32 && 2 * h + (lane >> 4) < HR)
                part_of(2 * h + (lane >> 4))[(lane & 15) * SW + HD] = gz + red[2 * 16 * 64 + hh * 32 + lane];
        } else {
            float* dst = part_of(h);
#pragma unroll
            for (int rg = 0; rg < 16; ++rg) {
                const int j = 8 * (rg >> 2) + 4 * g + (rg & 3);
                dst[j * SW + i] = accG[rg] + red[(hh * 16 + rg) * 64 + lane];
            }
            if (lane < 32) dst[lane * SW + HD] = gz + red[2 * 16 * 64 + hh * 32 + lane];
        }
    }
}

static_assert(sizeof(OperandLds) >= (2 * 16 * 64 + 2 * 32) * sizeof(float), "G reduction area exceeds the operand space");

// ------------------------------------------------------------------ query pass, matrix cores, head dim 64
// grid.x = (b * HR + hq) * (NB * tpb) + beta * tpb + tile: one head hq (its two
// 32-feature groups as the pair of the dim-32 kernel); wave w works on group
// a = w & 1 (features 32 a .. 32 a + 31) and every other 32-query sub-tile
// (w >> 1), next to the wave of the other group on the same queries.  Per
// sub-tile, as the dim-32 kernel with the 64 x 65 state P:
//   den = f . z over both groups (each wave reads both groups' q), r
//   u_a = dout_a r to the wave's LDS tile
//   m_a = P[32 a .., :64] dout (four K-steps; a 16-bit dout of both groups is
//   the B operand as it is, an fp32 one goes in as both waves' u split into
//   three bf16 terms)
//   dout . num = f_0 . m_0 + f_1 . m_1: the two waves exchange their halves
//   through LDS (a work-group barrier), w = -r^2 (dout . num)
//   dq_a = [q_a > 0] (r m_a + w z_a)
//   G[32 a .., 32 b ..] += f_a^T u_b for b = 0, 1 (u_b from the wave of
//   group b), G_z[32 a ..] += f_a^T w; with bf16 q on the bf16 matrix
//   instructions (tokens as the reduction dimension, both operands gathered
//   transposed from LDS: f exact, u as the three bf16 terms of its truncation
//   split, which sum to u exactly), with fp32 or fp16 q on the fp32 ones
// A last barrier keeps each u tile until the other wave has read it.  Every
// wave takes every step (a sub-tile past the range computes on the clamped
// last row and stores nothing), so the barriers are reached by all.  16-bit q
// (and 16-bit dout) are staged through LDS by the work-group; fp32 q is read
// by each wave, its f kept in an fp32 LDS tile (in the staging area).
template <typename QT, typename GT, typename OutT>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 8))) void k_bwd_query_mfma64(
    const QT* __restrict__ q, const GT* __restrict__ dout, const float* __restrict__ state, OutT* __restrict__ dq,
    float* __restrict__ gpart, int N, int HR, int L, int NB, int tile, int tpb, float eps) {
    constexpr int HD = 2 * kD, KS = KSteps<HD>::value, SW = HD + 1, SF = HD * SW;
    constexpr bool kStageQ = sizeof(QT) == 2, kDout16 = sizeof(GT) == 2;
    constexpr bool GF16 = std::is_same<GT, _Float16>::value, QF16 = std::is_same<QT, _Float16>::value;
    __shared__ u32x4 opnd[2][KS][3][64];                              // P natural split terms, rows of group a
    __shared__ __attribute__((aligned(16))) float pzs[2][32];          // P[:, 64] at the rows of each group
    __shared__ __attribute__((aligned(16))) uint16_t ush[4][3][32 * kUPitch];   // u as three bf16 terms, then the dq tile
    __shared__ __attribute__((aligned(16))) float wv[4][32];           // w of each token
    __shared__ __attribute__((aligned(16))) float gop[4][32];          // f_a . m_a of each token
    __shared__ __attribute__((aligned(16))) uint8_t lds_in[2 * kTileTensor];   // staged q (and 16-bit dout) / f tiles
    static_assert(sizeof(opnd) >= (2 * 2 * 16 * 64 + 2 * 32) * sizeof(float), "G reduction area exceeds the operand space");
    static_assert(sizeof(lds_in) >= 4 * 32 * kPitch * sizeof(float), "f tiles exceed the staging area");
    static_assert(sizeof(ush[0]) >= 32 * kPitch * sizeof(float), "dq tile exceeds the u area");

    const int per_unit = NB * tpb;
    const int tau = blockIdx.x % per_unit;
    const int bh = blockIdx.x / per_unit;
    const int hq = bh % HR, b = bh / HR;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int a = wave & 1, sub = wave >> 1;
    const int beta = tau / tpb, tib = tau - beta * tpb;
    const int blk0 = beta * L, blk1 = min(blk0 + L, N);
    const int t0 = blk0 + tib * tile, t1 = min(t0 + tile, blk1);
    const int g = lane >> 5, i = lane & 31;
    if (t0 >= t1) {
        // a tile past the end of a short last block: its partial gradient
        // state is zero (the suffix merge adds every tile slot of a block)
        float* dst = gpart + ((((size_t)b * HR + hq) * NB + beta) * tpb + tib) * SF;
        for (int e = threadIdx.x; e < SF; e += kThreads) dst[e] = 0.f;
        return;   // uniform over the work-group
    }

    const float* P = state + (((size_t)b * HR + hq) * NB + beta) * SF;
    if (wave < 2) {
        u32x4 t[KS][3];
        state_operands<HD>([&](int) { return P; }, hq, a, HR, lane, false, t);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
#pragma unroll
            for (int sp = 0; sp < 3; ++sp) opnd[a][ks][sp][lane] = t[ks][sp];
        if (lane < 32) pzs[a][lane] = P[(kD * a + lane) * SW + HD];
    }
    __syncthreads();

    const long long hstride = (long long)HR * HD;
    float* ot = reinterpret_cast<float*>(&ush[wave][0][0]);   // dq tile (after the u terms are read)
    float* ft = reinterpret_cast<float*>(lds_in) + wave * 32 * kPitch;   // fp32 q: f tile of this wave
    f32x16 accG[2] = {};   // G[32 a .., 32 b ..] for b = 0, 1
    float gz_acc = 0.f;    // lane (g, j): sum over this lane's tokens of f_j w (feature 32 a + j)
    auto zrow = [&](int gi, int rr) { return *reinterpret_cast<const f32x4*>(&pzs[gi][8 * rr + 4 * g]); };

    const uint16_t* dstage = kDout16 ? reinterpret_cast<const uint16_t*>(dout) : nullptr;
    TileLoader ld = {{reinterpret_cast<const uint16_t*>(q), dstage}, hstride, b, N, 2 * hq, HR * HD, t1, {}};
    if constexpr (kStageQ) ld.load(t0);
    for (int tt0 = t0; tt0 < t1; tt0 += kTileTok) {
        if constexpr (kStageQ) {
            __syncthreads();   // the previous tile has been consumed
            ld.store(lds_in);
            __syncthreads();
            if (tt0 + kTileTok < t1) ld.load(tt0 + kTileTok);   // in flight during this tile's work
        }
        __builtin_amdgcn_wave_barrier();
        asm volatile("" ::: "memory");   // the last step's dq tile is read before the u terms overwrite it
        const int tt = tt0 + 32 * sub;
        const int n = min(32, t1 - tt);   // <= 0: a step past the range (computes, stores nothing)
        const int tok = 32 * sub + i;     // this lane's token in the tile
        const long long grow = ((long long)b * N + min(tt + i, t1 - 1)) * hstride + hq * HD;   // its global row

        // q of both groups for the normaliser (the same order in both waves of
        // the pair), and of this wave's group (a separate read: an index by the
        // wave's group would put the rows in memory)
        auto load_q = [&](GradRow<QT>& r, int gi) {
            if constexpr (kStageQ)
                r.load_lds(lds_in + gi * kTileHead + tok * kTileRow, g);
            else
                r.load(q + grow + kD * gi, g);
        };
        float den = 0.f;
#pragma unroll
        for (int gi = 0; gi < 2; ++gi) {
            GradRow<QT> qg;
            load_q(qg, gi);
            float dp = 0.f;
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) {
                const f32x4 z = zrow(gi, rr);
#pragma unroll
                for (int e = 0; e < 4; ++e) dp = fmaf(relu_f32(qg.at(rr, e)), z[e], dp);
            }
            den += dp + __shfl_xor(dp, 32);
        }
        GradRow<QT> qo;
        load_q(qo, a);
        auto fa = [&](int rr, int e) { return relu_f32(qo.at(rr, e)); };
        const float r = 1.0f / (den + eps);

        // u of this group's channels to the LDS tiles as three bf16 truncation
        // terms (token-major); for fp32 q also f.  Tokens past the range keep
        // the clamped row's values (store_tile relies on it): the G products
        // mask them through f.
        GradRow<GT> gr;
        if constexpr (kStageQ && kDout16)
            gr.load_lds(lds_in + kTileTensor + a * kTileHead + tok * kTileRow, g);
        else
            gr.load(dout + grow + kD * a, g);
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
            f32x4 u4;
#pragma unroll
            for (int e = 0; e < 4; ++e) u4[e] = gr.at(rr, e) * r;
            const float x8[8] = {u4[0], u4[1], u4[2], u4[3], 0.f, 0.f, 0.f, 0.f};
            u32x4 ts[3];
            split3_trunc_f32x8(x8, ts);
#pragma unroll
            for (int sp = 0; sp < 3; ++sp)
                *reinterpret_cast<u32x2*>(&ush[wave][sp][i * kUPitch + 8 * rr + 4 * g]) = (u32x2){ts[sp][0], ts[sp][1]};
            if constexpr (!kStageQ) {
                f32x4 f4;
#pragma unroll
                for (int e = 0; e < 4; ++e) f4[e] = fa(rr, e);
                *reinterpret_cast<f32x4*>(ft + i * kPitch + 8 * rr + 4 * g) = f4;
            }
        }

        // m_a^T = P[32 a .., :64] dout^T (acc rs = r m_a)
        f32x16 acc = {};
        float rs;
        {
            u32x4 A[KS][3];
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
#pragma unroll
                for (int sp = 0; sp < 3; ++sp) A[ks][sp] = opnd[a][ks][sp][lane];
            if constexpr (kDout16) {
                u32x4 db[KS];   // dout of both groups, features 16 ks + 8 g ..
                if constexpr (kStageQ) {
                    tile_operand(lds_in, 1, 0, tok, g, db[0], db[1]);
                    tile_operand(lds_in, 1, 1, tok, g, db[2], db[3]);
                } else {
#pragma unroll
                    for (int ks = 0; ks < KS; ++ks)
                        db[ks] = *reinterpret_cast<const u32x4*>(dout + grow + 16 * ks + 8 * g);
                }
                acc = mma_split_ks<GF16, KS>(A, db, acc);
                rs = r;
            } else {
                // both waves' u terms (channels 16 ks + 8 g .. of group ks / 2);
                // products below 2^-24 dropped
                __syncthreads();   // both u tiles written
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) {
                    u32x4 ub[3];
#pragma unroll
                    for (int sp = 0; sp < 3; ++sp)
                        ub[sp] = *reinterpret_cast<const u32x4*>(
                            &ush[2 * sub + (ks >> 1)][sp][i * kUPitch + 16 * (ks & 1) + 8 * g]);
                    acc = mma_terms(A[ks], ub, acc);
                }
                rs = 1.f;
            }
        }
        float go = 0.f;
#pragma unroll
        for (int rr = 0; rr < 4; ++rr)
#pragma unroll
            for (int e = 0; e < 4; ++e) go = fmaf(fa(rr, e), acc[4 * rr + e], go);
        go += __shfl_xor(go, 32);
        if (g == 0) gop[wave][i] = go;
        __syncthreads();   // both groups' halves of dout . num, both u tiles written
        const float gsum = gop[2 * sub][i] + gop[2 * sub + 1][i];
        const float w = -r * (gsum * rs);
        if (g == 0) wv[wave][i] = i < n ? w : 0.f;   // 0 past the range: the G_z sum skips those tokens
        __builtin_amdgcn_wave_barrier();
        asm volatile("" ::: "memory");

        // G[32 a .., 32 b ..] += f_a^T u_b; G_z from the same f (lane (g, j):
        // feature j of its tokens)
        if constexpr (kStageQ && !QF16) {
            const uint16_t* qg = reinterpret_cast<const uint16_t*>(lds_in + a * kTileHead);
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                // f of tokens 32 sub + 16 ks + 8 g + e, feature i
                u32x4 fa4 = gather_tokens_t16(qg, kTileRow / 2, 32 * sub + 16 * ks, 0, lane);
                const f32x4 w0 = *reinterpret_cast<const f32x4*>(&wv[wave][16 * ks + 8 * g]);
                const f32x4 w1 = *reinterpret_cast<const f32x4*>(&wv[wave][16 * ks + 8 * g + 4]);
#pragma unroll
                for (int d = 0; d < 4; ++d) {
                    const int tb = 16 * ks + 8 * g + 2 * d;   // the tokens of the two halves: tb, tb + 1
                    const uint32_t keep = (tb < n ? 0xffffu : 0u) | (tb + 1 < n ? 0xffff0000u : 0u);
                    const uint32_t x = fa4[d] & ~(((fa4[d] & 0x80008000u) >> 15) * 0xffffu) & keep;   // ReLU, range
                    const float wl = d < 2 ? w0[2 * d] : w1[2 * d - 4], wh = d < 2 ? w0[2 * d + 1] : w1[2 * d - 3];
                    fa4[d] = x;
                    gz_acc = fmaf(hi_bf16(x), wh, fmaf(lo_bf16(x), wl, gz_acc));
                }
#pragma unroll
                for (int bg = 0; bg < 2; ++bg)
#pragma unroll
                    for (int sp = 2; sp >= 0; --sp) {
                        const u32x4 ub = gather_tokens_t16(ush[2 * sub + bg][sp], kUPitch, 16 * ks, 0, lane);
                        accG[bg] = mfma_bf16(fa4, ub, accG[bg]);
                    }
            }
        } else {
            // fp32 (or fp16) f on fp32 MFMA (32 x 32 x 2, token pairs); u is the sum of its terms
#pragma unroll
            for (int bg = 0; bg < 2; ++bg) {
#pragma unroll
                for (int m = 0; m < 16; ++m) {
                    const int tk = 2 * m + g;
                    const bool ok = tk < n;
                    float f_;
                    if constexpr (kStageQ)
                        f_ = ok ? f16_to_f32(relu_16(*reinterpret_cast<const uint16_t*>(
                                      lds_in + a * kTileHead + (32 * sub + tk) * kTileRow + 2 * i)))
                                : 0.f;
                    else
                        f_ = ok ? ft[tk * kPitch + i] : 0.f;
                    const int o = tk * kUPitch + i;
                    const uint16_t* ub = &ush[2 * sub + bg][0][0];
                    const float uv = (bf16_to_f32(ub[o]) + bf16_to_f32(ub[32 * kUPitch + o])) +
                                     bf16_to_f32(ub[2 * 32 * kUPitch + o]);
                    accG[bg] = __builtin_amdgcn_mfma_f32_32x32x2f32(f_, uv, accG[bg], 0, 0, 0);
                    if (bg == 0) gz_acc = fmaf(f_, ok ? wv[wave][tk] : 0.f, gz_acc);
                }
            }
        }

#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
            const f32x4 z = zrow(a, rr);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int rg = 4 * rr + e;
                acc[rg] = fa(rr, e) > 0.f ? fmaf(z[e], w, acc[rg] * rs) : 0.f;
            }
        }
        __syncthreads();   // the other wave has read this wave's u tile
        if (n > 0)
            store_tile<OutT>(ot, acc, lane, n,
                             [&](int t) { return dq + ((long long)b * N + tt + t) * hstride + (2 * hq + a) * kD; });
    }

    // the two sub-tile waves of a group add their G in a fixed order
    __syncthreads();
    const float gz = gz_acc + __shfl_xor(gz_acc, 32);
    float* red = reinterpret_cast<float*>(&opnd[0][0][0][0]);   // [group][block][16][64] G, then [group][32] G_z
    if (sub == 1) {
#pragma unroll
        for (int bg = 0; bg < 2; ++bg)
#pragma unroll
            for (int rg = 0; rg < 16; ++rg) red[((a * 2 + bg) * 16 + rg) * 64 + lane] = accG[bg][rg];
        if (lane < 32) red[2 * 2 * 16 * 64 + a * 32 + lane] = gz;
    }
    __syncthreads();
    if (sub == 0) {
        float* dst = gpart + ((((size_t)b * HR + hq) * NB + beta) * tpb + tib) * SF;
#pragma unroll
        for (int bg = 0; bg < 2; ++bg)
#pragma unroll
            for (int rg = 0; rg < 16; ++rg) {
                const int j = 8 * (rg >> 2) + 4 * g + (rg & 3);
                dst[(kD * a + j) * SW + kD * bg + i] = accG[bg][rg] + red[((a * 2 + bg) * 16 + rg) * 64 + lane];
            }
        if (lane < 32) dst[(kD * a + lane) * SW + HD] = gz + red[2 * 2 * 16 * 64 + a * 32 + lane];
    }
}

// ------------------------------------------------------------------ query pass, head dim 32, 16-bit q and dout
// The direct query kernel reads each wave's 32 rows straight from global
// memory in the MFMA operand layout (lane (g, i): token i, features 8 g .. + 7
// and 16 + 8 g .. + 7, two 16-byte loads per tensor), with the next sub-tile's
// loads in flight, as the forward's apply kernel does; nothing is staged in
// LDS.  The state operand's rows are permuted so that a product lands on the
// features the lane has loaded: output row r of a 32 x 32 MFMA tile (register
// 4 rr + e of lane (g, .), r = 8 rr + 4 g + e) is made feature perm_row(r),
// which swaps bits 2 and 3 of r, and register rg of lane (g, .) then holds
// feature 16 (rg >> 3) + 8 g + (rg & 7): element rg & 7 of the lane's operand
// half rg >> 3.  Masks and per-feature terms then use the lane's own
// registers.
__device__ __forceinline__ int perm_row(int r) { return (r & ~12) | ((r & 4) << 1) | ((r & 8) >> 1); }
__device__ __forceinline__ int perm_feature(int g, int rg) { return 16 * (rg >> 3) + 8 * g + (rg & 7); }

// Split-term operands (state_operands' three bf16 terms) of a head's 32 x 33
// state S with permuted rows: lane (g, i) gets A[i][16 ks + 8 g + e] =
// S[perm_row(i)][16 ks + 8 g + e].
__device__ __forceinline__ void perm_operands(const float* S, int lane, u32x4 (&out)[2][3]) {
    constexpr int SW = kD + 1;
    const int g = lane >> 5, ri = perm_row(lane & 31);
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
        float x[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] = S[ri * SW + 16 * ks + 8 * g + e];
        split3_f32x8(x, out[ks]);
    }
}

// The same for head dim 16: the 32-feature group grp holds heads 2 grp and
// 2 grp + 1 (the second may not exist: zero), whose states form one
// block-diagonal 32 x 32 matrix; row i is feature perm_row(i) of head
// 2 grp + (perm_row(i) >> 4), nonzero in that head's 16 columns only.
template <typename HeadState>
__device__ __forceinline__ void perm_operands16(HeadState head, int grp, int HR, int lane, u32x4 (&out)[2][3]) {
    constexpr int SW = kD / 2 + 1;
    const int g = lane >> 5, f = perm_row(lane & 31), hr = 2 * grp + (f >> 4);
    const float* S = head(min(hr, HR - 1));
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
        float x[8];
        const bool on = hr < HR && ks == (f >> 4);
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] = on ? S[(f & 15) * SW + 8 * g + e] : 0.f;
        split3_f32x8(x, out[ks]);
    }
}

// Element rg & 7 of operand half rg >> 3 (a packed 16-bit operand) as fp32.
template <bool F16>
__device__ __forceinline__ float operand_elem(const u32x4 (&x)[2], int rg) {
    const uint32_t w = x[rg >> 3][(rg & 7) >> 1];
    if constexpr (F16)
        return f16_to_f32((uint16_t)((rg & 1) ? (w >> 16) : (w & 0xffffu)));
    else
        return (rg & 1) ? hi_bf16(w) : lo_bf16(w);
}

// Two fp32 values rounded (nearest-even) to OutT and packed (one
// v_cvt_pk_bf16_f32 / v_cvt_pk_f16_f32).
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
template <typename OutT>
__device__ __forceinline__ uint32_t pack2(float a, float b) {
    if constexpr (std::is_same<OutT, _Float16>::value) {
        // pin the fp32 values (see put_pair_tile)
        asm volatile("" : "+v"(a));
        asm volatile("" : "+v"(b));
        return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){a, b}, f16x2));
    } else {
        return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){a, b}, bf16x2));
    }
}

// A permuted-layout tile (lane (g, i): token i, register rg = feature
// perm_feature(g, rg)) rounded to OutT into head hh's half of a pair tile.
template <typename OutT>
__device__ __forceinline__ void put_pair_tile_perm(uint16_t* ct, const f32x16& acc, int lane, int hh) {
    const int g = lane >> 5, i = lane & 31;
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
        u32x4 p;
#pragma unroll
        for (int d = 0; d < 4; ++d) p[d] = pack2<OutT>(acc[8 * hf + 2 * d], acc[8 * hf + 2 * d + 1]);
        *reinterpret_cast<u32x4*>(ct + i * kPairRow + hh * 32 + 16 * hf + 8 * g) = p;
    }
}

// store_tile for a permuted-layout fp32 tile: through the wave's LDS tile,
// then whole 128-byte rows; rows t >= n repeat row n - 1 (same values).
template <typename RowPtr>
__device__ __forceinline__ void store_tile_perm(float* ot, const f32x16& acc, int lane, int n, RowPtr dst,
                                                int ncols = 32) {
    const int g = lane >> 5, i = lane & 31;
#pragma unroll
    for (int p = 0; p < 4; ++p)
        *reinterpret_cast<f32x4*>(ot + i * kPitch + 16 * (p >> 1) + 8 * g + 4 * (p & 1)) =
            (f32x4){acc[4 * p], acc[4 * p + 1], acc[4 * p + 2], acc[4 * p + 3]};
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int s4 = 0; s4 < 4; ++s4) {
        const int r = 8 * s4 + (lane >> 3), cc = (lane & 7) * 4;
        if (cc < ncols) store4(dst(min(r, n - 1)) + cc, *reinterpret_cast<const f32x4*>(ot + r * kPitch + cc));
    }
    __builtin_amdgcn_wave_barrier();
}

// 16-bit rows of q and dout for the 32 tokens of a sub-tile (operand layout).
struct Rows16 {
    u32x4 x[2], y[2];
};
__device__ __forceinline__ void load_rows16(const uint16_t* x, const uint16_t* y, long long off, Rows16& r) {
    const u32x4* px = reinterpret_cast<const u32x4*>(x + off);
    const u32x4* py = reinterpret_cast<const u32x4*>(y + off);
    r.x[0] = px[0];
    r.x[1] = px[2];
    r.y[0] = py[0];
    r.y[1] = py[2];
}

// grid.x = (b * HP + hp) * (NB * tpb) + beta * tpb + tile; wave w handles head
// 2 hp + (w & 1) and the 32-query sub-tiles 32 (w >> 1) + 64 s of the tile.
// Per sub-tile, with f = ReLU(q), P the block's state (rows permuted), z =
// P[:, D]:
//   den = f . z (fp32, the lane's 16 features and its partner's), r = 1/(den + eps)
//   m = P_v dout^T on MFMA (six products: P's split terms, the 16-bit dout
//   exact; fp16 dout as two exact bf16 terms)
//   w = -r (r (f . m)) (dout . num = f . m), dq = [q > 0] (r m + w z)
// then the gradient state, tokens as the reduction dimension: f^T and dout^T
// come out of MFMAs against identity operands (exact: one product 1 * x per
// output), which leave lane (g, j) with feature j of the tokens 8 rr + 4 g + e
// in register 4 rr + e; r and w of those tokens are read back from the wave's
// LDS row (zero for tokens past the range), u = r dout^T, and
//   G_v += f^T u, bf16 q: on the bf16 matrix instructions, 16 tokens per
//                 K-step, f^T exact and u as the three terms of its
//                 truncation split (which sum to u exactly): three MFMAs per
//                 K-step instead of eight fp32 ones;
//                 fp16 q: 16 fp32 MFMAs 32 x 32 x 2 (f is not a bf16 value)
//   G_z += f^T w (vector FMAs).
// 16-bit dq: the two waves of a sub-tile fill a pair tile and store whole
// 128-byte lines (two work-group barriers per step; every wave takes the same
// number of steps, a step past the range working on the clamped last row);
// fp32 dq: each wave stores its own rows through its LDS tile.  At the end the
// two waves of a head add their G in a fixed order and write the tile's
// partial gradient state (zero for a tile with no tokens).
template <bool QF16, bool GF16, typename OutT, int HD>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(sizeof(OutT) == 4 || HD == kD / 2 ? 2 : 3, 8))) void k_bwd_query_direct(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ dout, const float* __restrict__ state,
    OutT* __restrict__ dq, float* __restrict__ gpart, int N, int H, int HP, int HR, int L, int NB, int tile,
    int tpb, float eps) {
    constexpr bool D16 = HD == kD / 2;
    static_assert(HD == kD || D16, "head dims 32 and 16");
    constexpr int NS = D16 ? 2 : 1;   // heads per 32-feature group
    constexpr int SW = HD + 1, SF = HD * SW;
    constexpr bool kPair = sizeof(OutT) == 2;
    __shared__ __attribute__((aligned(16))) uint16_t ct[kPair ? 2 : 1][kPair ? 2 : 1][kPair ? 32 * kPairRow : 8];   // [step & 1][sub]
    __shared__ __attribute__((aligned(16))) float otile[kPair ? 1 : 4][kPair ? 4 : 32 * kPitch];
    __shared__ __attribute__((aligned(16))) float rw[4][NS][2][32];   // r and w of each wave's tokens (per head)
    __shared__ __attribute__((aligned(16))) float red[2][16 * 64 + 32];   // the second waves' G

    const int per_unit = NB * tpb;
    const int tau = blockIdx.x % per_unit;
    const int bhp = blockIdx.x / per_unit;
    const int hp = bhp % HP, b = bhp / HP;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int hh = wave & 1, sub = wave >> 1, h = 2 * hp + hh;
    const int hs = min(h, H - 1);   // a missing second head computes on the first (never stored)
    const int beta = tau / tpb, tib = tau - beta * tpb;
    const int blk0 = beta * L, blk1 = min(blk0 + L, N);
    const int t0 = blk0 + tib * tile, t1 = min(t0 + tile, blk1);
    const int g = lane >> 5, i = lane & 31;

    auto head_P = [&](int hr) { return state + (((size_t)b * HR + hr) * NB + beta) * SF; };
    const bool second = !D16 || 2 * hs + 1 < HR;   // head dim 16: group hs has a second head
    f32x16 accG = {};
    float gzacc = 0.f;   // lane (g, j): sum over this lane's tokens of f_j w
    if (t0 < t1) {       // uniform over the work-group
        u32x4 pa[2][3];
        float zr[16];
        if constexpr (D16) {
            perm_operands16(head_P, hs, HR, lane, pa);
#pragma unroll
            for (int rg = 0; rg < 16; ++rg) {
                const int f = perm_feature(g, rg), hr = 2 * hs + (f >> 4);
                zr[rg] = hr < HR ? head_P(hr)[(f & 15) * SW + HD] : 0.f;
            }
        } else {
            const float* P = head_P(hs);
            perm_operands(P, lane, pa);
#pragma unroll
            for (int rg = 0; rg < 16; ++rg) zr[rg] = P[perm_feature(g, rg) * SW + HD];
        }
        // identity operands: element e of K-step ks is one where 16 ks + 8 g + e = i
        u32x4 iq[2], ig[2];
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
#pragma unroll
            for (int d = 0; d < 4; ++d) {
                const int e0 = 16 * ks + 8 * g + 2 * d;
                const uint32_t oq = QF16 ? 0x3c00u : 0x3f80u, og = GF16 ? 0x3c00u : 0x3f80u;
                iq[ks][d] = (e0 == i ? oq : 0u) | (e0 + 1 == i ? oq << 16 : 0u);
                ig[ks][d] = (e0 == i ? og : 0u) | (e0 + 1 == i ? og << 16 : 0u);
            }

        const long long hstride = (long long)HR * HD;
        auto row_off = [&](int tt) { return ((long long)b * N + min(tt + i, t1 - 1)) * hstride + hs * kD + 8 * g; };
        // a lone head of dim 16 has no features 16.. (they are read as zero)
        auto load = [&](int tt, Rows16& r) {
            if (second) {
                load_rows16(q, dout, row_off(tt), r);
            } else {
                const long long o = row_off(tt);
                r.x[0] = *reinterpret_cast<const u32x4*>(q + o);
                r.y[0] = *reinterpret_cast<const u32x4*>(dout + o);
                r.x[1] = r.y[1] = (u32x4){0u, 0u, 0u, 0u};
            }
        };
        const int steps = (t1 - t0 + 63) / 64;
        int tt = t0 + 32 * sub;
        Rows16 cur;   // x: q, y: dout
        load(tt, cur);
        for (int st = 0; st < steps; ++st, tt += 64) {
            Rows16 nxt;
            load(tt + 64, nxt);   // in flight during this sub-tile's work
            const int n = min(32, t1 - tt);
            const u32x4 fq[2] = {relu_bf16x8(cur.x[0]), relu_bf16x8(cur.x[1])};
            // per head of the group (head dim 16: registers rg >> 3 = head)
            float dp[NS] = {};
#pragma unroll
            for (int rg = 0; rg < 16; ++rg) {
                float& d = dp[D16 ? rg >> 3 : 0];
                d = fmaf(operand_elem<QF16>(fq, rg), zr[rg], d);
            }
            float r[NS], w[NS];
#pragma unroll
            for (int s2 = 0; s2 < NS; ++s2) r[s2] = 1.0f / (dp[s2] + __shfl_xor(dp[s2], 32) + eps);
            f32x16 acc = {};
            acc = mma_split_ks<GF16, 2>(pa, cur.y, acc);
            float go[NS] = {};
#pragma unroll
            for (int rg = 0; rg < 16; ++rg) {
                float& o = go[D16 ? rg >> 3 : 0];
                o = fmaf(operand_elem<QF16>(fq, rg), acc[rg], o);
            }
#pragma unroll
            for (int s2 = 0; s2 < NS; ++s2) w[s2] = -r[s2] * ((go[s2] + __shfl_xor(go[s2], 32)) * r[s2]);
#pragma unroll
            for (int rg = 0; rg < 16; ++rg) {
                const int s2 = D16 ? rg >> 3 : 0;
                acc[rg] = operand_elem<QF16>(fq, rg) > 0.f ? fmaf(zr[rg], w[s2], acc[rg] * r[s2]) : 0.f;
            }
            if (g == 0) {   // zero past the range: the G sums skip those tokens
#pragma unroll
                for (int s2 = 0; s2 < NS; ++s2) {
                    rw[wave][s2][0][i] = i < n ? r[s2] : 0.f;
                    rw[wave][s2][1][i] = i < n ? w[s2] : 0.f;
                }
            }
            // f^T and dout^T: lane (g, j) gets feature j of tokens 8 rr + 4 g + e
            f32x16 fT = {}, gT = {};
            fT = mfma16<QF16>(fq[0], iq[0], fT);
            fT = mfma16<QF16>(fq[1], iq[1], fT);
            gT = mfma16<GF16>(cur.y[0], ig[0], gT);
            gT = mfma16<GF16>(cur.y[1], ig[1], gT);
            if constexpr (kPair) {
                put_pair_tile_perm<OutT>(ct[st & 1][sub], acc, lane, hh);
            } else if (n > 0 && h < H) {
                store_tile_perm(otile[wave], acc, lane, n, [&](int t) {
                    return reinterpret_cast<float*>(dq + ((long long)b * N + tt + t) * hstride + h * kD);
                }, min(32, HR * HD - h * kD));
            }
            __builtin_amdgcn_wave_barrier();
            asm volatile("" ::: "memory");   // the r, w rows are written before they are read
            if constexpr (!QF16) {
#pragma unroll
                for (int ks = 0; ks < 2; ++ks) {
                    float uu[8];
                    u32x4 fp;
#pragma unroll
                    for (int h2 = 0; h2 < 2; ++h2) {
                        const int rr = 2 * ks + h2;
                        const f32x4 r4 = *reinterpret_cast<const f32x4*>(&rw[wave][D16 ? i >> 4 : 0][0][8 * rr + 4 * g]);
                        const f32x4 w4 = *reinterpret_cast<const f32x4*>(&rw[wave][D16 ? i >> 4 : 0][1][8 * rr + 4 * g]);
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            const int s = 4 * rr + e;
                            uu[4 * h2 + e] = gT[s] * r4[e];
                            gzacc = fmaf(fT[s], w4[e], gzacc);
                        }
#pragma unroll
                        for (int d = 0; d < 2; ++d) {
                            // through scalars: bit_cast of a vector element
                            // expression reads the vector's first element with
                            // this compiler
                            const float f0 = fT[4 * rr + 2 * d], f1 = fT[4 * rr + 2 * d + 1];
                            fp[2 * h2 + d] = (__builtin_bit_cast(uint32_t, f0) >> 16) |
                                             (__builtin_bit_cast(uint32_t, f1) & 0xffff0000u);
                        }
                    }
                    u32x4 ut[3];
                    split3_trunc_f32x8(uu, ut);
                    accG = mfma_bf16(fp, ut[2], accG);
                    accG = mfma_bf16(fp, ut[1], accG);
                    accG = mfma_bf16(fp, ut[0], accG);
                }
            } else {
#pragma unroll
                for (int rr = 0; rr < 4; ++rr) {
                    const f32x4 r4 = *reinterpret_cast<const f32x4*>(&rw[wave][D16 ? i >> 4 : 0][0][8 * rr + 4 * g]);
                    const f32x4 w4 = *reinterpret_cast<const f32x4*>(&rw[wave][D16 ? i >> 4 : 0][1][8 * rr + 4 * g]);
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int s = 4 * rr + e;
                        accG = __builtin_amdgcn_mfma_f32_32x32x2f32(fT[s], gT[s] * r4[e], accG, 0, 0, 0);
                        gzacc = fmaf(fT[s], w4[e], gzacc);
                    }
                }
            }
            if constexpr (kPair) {
                // double-buffered pair tiles: this step's barrier also orders
                // the previous step's reads of the other buffer before its
                // next writes
                __syncthreads();
                const int nchunk = min(8, (HR * HD - 2 * hp * kD) / 8);
                store_pair_rows<OutT>(ct[st & 1][sub], lane, 16 * hh, nchunk, [&](int rrow) {
                    return reinterpret_cast<uint16_t*>(dq + ((long long)b * N + min(tt + rrow, t1 - 1)) * hstride + 2 * hp * kD);
                });
            }
            __builtin_amdgcn_wave_barrier();
            asm volatile("" ::: "memory");   // every read of the r, w rows precedes the next writes
            cur = nxt;
        }
    }

    // the two waves of a head add their G in a fixed order
    const float gz = gzacc + __shfl_xor(gzacc, 32);
    if (sub == 1) {
#pragma unroll
        for (int rg = 0; rg < 16; ++rg) red[hh][rg * 64 + lane] = accG[rg];
        if (lane < 32) red[hh][16 * 64 + lane] = gz;
    }
    __syncthreads();
    if (sub == 0 && h < H) {
        auto part_of = [&](int hr) { return gpart + ((((size_t)b * HR + hr) * NB + beta) * tpb + tib) * SF; };
        if constexpr (D16) {
            // the diagonal 16 x 16 blocks: rows 0..15 and the lanes of columns
            // 0..15 are the first head's, the rest the second's
#pragma unroll
            for (int rg = 0; rg < 16; ++rg) {
                const int j = 8 * (rg >> 2) + 4 * g + (rg & 3), hr = 2 * h + (j >> 4);
                if ((i >> 4) == (j >> 4) && hr < HR)
                    part_of(hr)[(j & 15) * SW + (i & 15)] = accG[rg] + red[hh][rg * 64 + lane];
            }
            if (lane < 32 && 2 * h + (lane >> 4) < HR)
                part_of(2 * h + (lane >> 4))[(lane & 15) * SW + HD] = gz + red[hh][16 * 64 + lane];
        } else {
            float* dst = part_of(h);
#pragma unroll
            for (int rg = 0; rg < 16; ++rg) {
                const int j = 8 * (rg >> 2) + 4 * g + (rg & 3);
                dst[j * SW + i] = accG[rg] + red[hh][rg * 64 + lane];
            }
            if (lane < 32) dst[lane * SW + HD] = gz + red[hh][16 * 64 + lane];
        }
    }
}

// ------------------------------------------------------------------ query pass, head dim 64, 16-bit q and dout
// The per-wave scheme of k_bwd_query_direct for a head of 64 features, seen
// as two 32-feature groups.  grid.x = (b * HR + hq) * (NB * tpb) + beta * tpb
// + tile; wave w works on group a = w & 1 of head hq and the 32-query
// sub-tiles 32 (w >> 1) + 64 s, next to the wave of the other group on the
// same queries.  Per sub-tile, with P the head's 64 x 65 state (rows 32 a ..
// of group a, permuted as perm_row does):
//   den_a = f_a . z_a, m_a = P[32 a .., :64] dout^T (four K-steps: dout of
//   both groups is loaded by each wave), f_a . m_a;
//   the two waves exchange den_a and f_a . m_a through LDS (a work-group
//   barrier) and both form den = den_0 + den_1, dout . num = f_0 . m_0 +
//   f_1 . m_1 in that order, r and w;
//   dq_a = [q_a > 0] (r m_a + w z_a) into the head's pair tile (group a in
//   its half of each 128-byte line);
//   G[32 a .., 32 b ..] += f_a^T u_b for b = 0, 1 (f_a^T and dout_b^T from
//   identity MFMAs, u_b = r dout_b^T split into three bf16 terms; bf16 q;
//   fp32 products 32 x 32 x 2 for fp16 q), G_z[32 a ..] += f_a^T w.
// Every wave takes every step (a step past the range works on the clamped
// last row), so the barriers are reached by all.  At the end the two waves of
// a group add their G in a fixed order and write rows 32 a .. of the tile's
// partial gradient state (zero for a tile with no tokens).
template <bool QF16, bool GF16, typename OutT>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 8))) void k_bwd_query_direct64(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ dout, const float* __restrict__ state,
    OutT* __restrict__ dq, float* __restrict__ gpart, int N, int HR, int L, int NB, int tile, int tpb, float eps) {
    constexpr int HD = 2 * kD, SW = HD + 1, SF = HD * SW;
    constexpr bool kPair = sizeof(OutT) == 2;
    __shared__ __attribute__((aligned(16))) uint16_t ct[kPair ? 2 : 1][kPair ? 2 : 1][kPair ? 32 * kPairRow : 8];   // [step & 1][sub]
    __shared__ __attribute__((aligned(16))) float otile[kPair ? 1 : 4][kPair ? 4 : 32 * kPitch];
    __shared__ __attribute__((aligned(16))) float rw[4][2][32];        // r and w of each wave's tokens
    __shared__ __attribute__((aligned(16))) float xch[2][2][2][32];    // [sub][group][den, f . m] partial sums
    __shared__ __attribute__((aligned(16))) float red[2][2 * 16 * 64 + 32];   // the second waves' G

    const int per_unit = NB * tpb;
    const int tau = blockIdx.x % per_unit;
    const int bh = blockIdx.x / per_unit;
    const int hq = bh % HR, b = bh / HR;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int a = wave & 1, sub = wave >> 1;
    const int beta = tau / tpb, tib = tau - beta * tpb;
    const int blk0 = beta * L, blk1 = min(blk0 + L, N);
    const int t0 = blk0 + tib * tile, t1 = min(t0 + tile, blk1);
    const int g = lane >> 5, i = lane & 31;

    const float* P = state + (((size_t)b * HR + hq) * NB + beta) * SF;
    f32x16 accG[2] = {};
    float gzacc = 0.f;   // lane (g, j): sum over this lane's tokens of f_(32 a + j) w
    if (t0 < t1) {       // uniform over the work-group
        // P rows 32 a + perm_row(i), all 64 columns (four K-steps)
        u32x4 pa[4][3];
        {
            const int ri = kD * a + perm_row(i);
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                float x[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) x[e] = P[ri * SW + 16 * ks + 8 * g + e];
                split3_f32x8(x, pa[ks]);
            }
        }
        float zr[16];
#pragma unroll
        for (int rg = 0; rg < 16; ++rg) zr[rg] = P[(kD * a + perm_feature(g, rg)) * SW + HD];
        // identity operands: element e of K-step ks is one where 16 ks + 8 g + e = i
        u32x4 iq[2], ig[2];
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
#pragma unroll
            for (int d = 0; d < 4; ++d) {
                const int e0 = 16 * ks + 8 * g + 2 * d;
                const uint32_t oq = QF16 ? 0x3c00u : 0x3f80u, og = GF16 ? 0x3c00u : 0x3f80u;
                iq[ks][d] = (e0 == i ? oq : 0u) | (e0 + 1 == i ? oq << 16 : 0u);
                ig[ks][d] = (e0 == i ? og : 0u) | (e0 + 1 == i ? og << 16 : 0u);
            }

        const long long hstride = (long long)HR * HD;
        struct Rows {
            u32x4 x[2], y[4];   // q of group a; dout of both groups
        };
        auto load = [&](int tt, Rows& r) {
            const long long row = ((long long)b * N + min(tt + i, t1 - 1)) * hstride + hq * HD + 8 * g;
            const u32x4* px = reinterpret_cast<const u32x4*>(q + row + kD * a);
            const u32x4* py = reinterpret_cast<const u32x4*>(dout + row);
            r.x[0] = px[0];
            r.x[1] = px[2];
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) r.y[ks] = py[2 * ks];
        };
        const int steps = (t1 - t0 + 63) / 64;
        int tt = t0 + 32 * sub;
        Rows cur;
        load(tt, cur);
        for (int st = 0; st < steps; ++st, tt += 64) {
            Rows nxt;
            load(tt + 64, nxt);   // in flight during this sub-tile's work
            const int n = min(32, t1 - tt);
            const u32x4 fq[2] = {relu_bf16x8(cur.x[0]), relu_bf16x8(cur.x[1])};
            float dp = 0.f;
#pragma unroll
            for (int rg = 0; rg < 16; ++rg) dp = fmaf(operand_elem<QF16>(fq, rg), zr[rg], dp);
            f32x16 acc = {};
            acc = mma_split_ks<GF16, 4>(pa, cur.y, acc);
            float go = 0.f;
#pragma unroll
            for (int rg = 0; rg < 16; ++rg) go = fmaf(operand_elem<QF16>(fq, rg), acc[rg], go);
            dp += __shfl_xor(dp, 32);
            go += __shfl_xor(go, 32);
            if (g == 0) {
                xch[sub][a][0][i] = dp;
                xch[sub][a][1][i] = go;
            }
            __syncthreads();   // both groups' partial sums are in xch
            const float r = 1.0f / (xch[sub][0][0][i] + xch[sub][1][0][i] + eps);
            const float w = -r * ((xch[sub][0][1][i] + xch[sub][1][1][i]) * r);
#pragma unroll
            for (int rg = 0; rg < 16; ++rg)
                acc[rg] = operand_elem<QF16>(fq, rg) > 0.f ? fmaf(zr[rg], w, acc[rg] * r) : 0.f;
            if (g == 0) {   // zero past the range: the G sums skip those tokens
                rw[wave][0][i] = i < n ? r : 0.f;
                rw[wave][1][i] = i < n ? w : 0.f;
            }
            f32x16 fT = {};
            fT = mfma16<QF16>(fq[0], iq[0], fT);
            fT = mfma16<QF16>(fq[1], iq[1], fT);
            if constexpr (kPair) {
                put_pair_tile_perm<OutT>(ct[st & 1][sub], acc, lane, a);
            } else if (n > 0) {
                store_tile_perm(otile[wave], acc, lane, n, [&](int t) {
                    return reinterpret_cast<float*>(dq + ((long long)b * N + tt + t) * hstride + hq * HD + kD * a);
                });
            }
            __builtin_amdgcn_wave_barrier();
            asm volatile("" ::: "memory");   // the r, w rows are written before they are read
#pragma unroll
            for (int bg = 0; bg < 2; ++bg) {
                f32x16 gT = {};
                gT = mfma16<GF16>(cur.y[2 * bg], ig[0], gT);
                gT = mfma16<GF16>(cur.y[2 * bg + 1], ig[1], gT);
                if constexpr (!QF16) {
#pragma unroll
                    for (int ks = 0; ks < 2; ++ks) {
                        float uu[8];
                        u32x4 fp;
#pragma unroll
                        for (int h2 = 0; h2 < 2; ++h2) {
                            const int rr = 2 * ks + h2;
                            const f32x4 r4 = *reinterpret_cast<const f32x4*>(&rw[wave][0][8 * rr + 4 * g]);
#pragma unroll
                            for (int e = 0; e < 4; ++e) uu[4 * h2 + e] = gT[4 * rr + e] * r4[e];
#pragma unroll
                            for (int d = 0; d < 2; ++d) {
                                // through scalars: bit_cast of a vector element
                                // expression reads the vector's first element
                                // with this compiler
                                const float f0 = fT[4 * rr + 2 * d], f1 = fT[4 * rr + 2 * d + 1];
                                fp[2 * h2 + d] = (__builtin_bit_cast(uint32_t, f0) >> 16) |
                                                 (__builtin_bit_cast(uint32_t, f1) & 0xffff0000u);
                            }
                        }
                        u32x4 ut[3];
                        split3_trunc_f32x8(uu, ut);
                        accG[bg] = mfma_bf16(fp, ut[2], accG[bg]);
                        accG[bg] = mfma_bf16(fp, ut[1], accG[bg]);
                        accG[bg] = mfma_bf16(fp, ut[0], accG[bg]);
                    }
                } else {
#pragma unroll
                    for (int rr = 0; rr < 4; ++rr) {
                        const f32x4 r4 = *reinterpret_cast<const f32x4*>(&rw[wave][0][8 * rr + 4 * g]);
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            const int s = 4 * rr + e;
                            accG[bg] = __builtin_amdgcn_mfma_f32_32x32x2f32(fT[s], gT[s] * r4[e], accG[bg], 0, 0, 0);
                        }
                    }
                }
            }
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) {
                const f32x4 w4 = *reinterpret_cast<const f32x4*>(&rw[wave][1][8 * rr + 4 * g]);
#pragma unroll
                for (int e = 0; e < 4; ++e) gzacc = fmaf(fT[4 * rr + e], w4[e], gzacc);
            }
            if constexpr (kPair) {
                // double-buffered pair tiles (the head's 128-byte rows): this
                // step's barrier also orders the previous step's reads of the
                // other buffer before its next writes
                __syncthreads();
                store_pair_rows<OutT>(ct[st & 1][sub], lane, 16 * a, 8, [&](int rrow) {
                    return reinterpret_cast<uint16_t*>(dq + ((long long)b * N + min(tt + rrow, t1 - 1)) * hstride + hq * HD);
                });
            } else {
                __syncthreads();   // every read of xch precedes the next step's writes
            }
            __builtin_amdgcn_wave_barrier();
            asm volatile("" ::: "memory");   // every read of the r, w rows precedes the next writes
            cur = nxt;
        }
    }

    // the two waves of a group add their G in a fixed order
    const float gz = gzacc + __shfl_xor(gzacc, 32);
    if (sub == 1) {
#pragma unroll
        for (int bg = 0; bg < 2; ++bg)
#pragma unroll
            for (int rg = 0; rg < 16; ++rg) red[a][(bg * 16 + rg) * 64 + lane] = accG[bg][rg];
        if (lane < 32) red[a][2 * 16 * 64 + lane] = gz;
    }
    __syncthreads();
    if (sub == 0) {
        float* dst = gpart + ((((size_t)b * HR + hq) * NB + beta) * tpb + tib) * SF;
#pragma unroll
        for (int bg = 0; bg < 2; ++bg)
#pragma unroll
            for (int rg = 0; rg < 16; ++rg) {
                const int j = 8 * (rg >> 2) + 4 * g + (rg & 3);
                dst[(kD * a + j) * SW + kD * bg + i] = accG[bg][rg] + red[a][(bg * 16 + rg) * 64 + lane];
            }
        if (lane < 32) dst[(kD * a + lane) * SW + HD] = gz + red[a][2 * 16 * 64 + lane];
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

hipError_t launch_bwd_query(const BwdPlan& bp, const void* q, const void* dout, const float* state, void* dq,
                            float* gpart, float eps, hipStream_t stream) {
    const Plan& pl = bp.fw;
    if (bp.query_direct) {
        const unsigned grid = (unsigned)((size_t)pl.B * pl.HP * pl.NB * bp.tpbq);
        by_dtype(bp.grad_dtype, [&](auto ot) {
            using OT = typename decltype(ot)::type;
            const bool qf16 = pl.in_dtype == 2, gf16 = bp.dout_dtype == 2;
            auto pick = [&](auto dd) {
                constexpr int DD = decltype(dd)::value;
                return qf16 ? (gf16 ? k_bwd_query_direct<true, true, OT, DD> : k_bwd_query_direct<true, false, OT, DD>)
                            : (gf16 ? k_bwd_query_direct<false, true, OT, DD> : k_bwd_query_direct<false, false, OT, DD>);
            };
            if (pl.D == 2 * kD) {
                auto kern64 = qf16 ? (gf16 ? k_bwd_query_direct64<true, true, OT> : k_bwd_query_direct64<true, false, OT>)
                                   : (gf16 ? k_bwd_query_direct64<false, true, OT> : k_bwd_query_direct64<false, false, OT>);
                hipLaunchKernelGGL(kern64, dim3(grid), dim3(kThreads), 0, stream, static_cast<const uint16_t*>(q),
                                   static_cast<const uint16_t*>(dout), state, static_cast<OT*>(dq), gpart, pl.N, pl.H,
                                   pl.L, pl.NB, bp.tq, bp.tpbq, eps);
                return;
            }
            auto kern = pl.D == kD / 2 ? pick(std::integral_constant<int, kD / 2>{}) : pick(std::integral_constant<int, kD>{});
            hipLaunchKernelGGL(kern, dim3(grid), dim3(kThreads), 0, stream, static_cast<const uint16_t*>(q),
                               static_cast<const uint16_t*>(dout), state, static_cast<OT*>(dq), gpart, pl.N,
                               groups32(pl), pl.HP, pl.H, pl.L, pl.NB, bp.tq, bp.tpbq, eps);
        });
        return hipGetLastError();
    }
    if (bp.query_mfma) {
        const unsigned grid = (unsigned)((size_t)pl.B * pl.HP * pl.NB * bp.tpbq);
        bool routed = true;
        by_dtype(bp.dout_dtype, [&](auto gt) {
            by_dtype(bp.grad_dtype, [&](auto ot) {
                using GT = typename decltype(gt)::type;
                using OT = typename decltype(ot)::type;
                by_dtype(pl.in_dtype, [&](auto it) {
                    using QT = typename decltype(it)::type;
                    // 16-bit q with a 16-bit dout takes the per-wave kernels
                    // above: only combinations with an fp32 q or dout come here
                    if constexpr (std::is_same<QT, float>::value || std::is_same<GT, float>::value) {
                        if (pl.D == 2 * kD) {
                            hipLaunchKernelGGL((k_bwd_query_mfma64<QT, GT, OT>), dim3(grid), dim3(kThreads), 0, stream,
                                               static_cast<const QT*>(q), static_cast<const GT*>(dout), state,
                                               static_cast<OT*>(dq), gpart, pl.N, pl.H, pl.L, pl.NB, bp.tq, bp.tpbq,
                                               eps);
                        } else if (pl.D == kD / 2) {
                            hipLaunchKernelGGL((k_bwd_query_mfma<QT, GT, OT, kD / 2>), dim3(grid), dim3(kThreads), 0,
                                               stream, static_cast<const QT*>(q), static_cast<const GT*>(dout), state,
                                               static_cast<OT*>(dq), gpart, pl.N, groups32(pl), pl.HP, pl.H, pl.L,
                                               pl.NB, bp.tq, bp.tpbq, eps);
                        } else {
                            hipLaunchKernelGGL((k_bwd_query_mfma<QT, GT, OT, kD>), dim3(grid), dim3(kThreads), 0, stream,
                                               static_cast<const QT*>(q), static_cast<const GT*>(dout), state,
                                               static_cast<OT*>(dq), gpart, pl.N, pl.H, pl.HP, pl.H, pl.L, pl.NB,
                                               bp.tq, bp.tpbq, eps);
                        }
                    } else {
                        routed = false;   // the plan sends these to the per-wave kernels
                    }
                });
            });
        });
        return routed ? hipGetLastError() : hipErrorInvalidConfiguration;
    }
    const unsigned grid = (unsigned)((size_t)pl.B * pl.H * pl.NB * bp.tpbq);
    by_dtype(pl.in_dtype, [&](auto it) {
        by_dtype(bp.dout_dtype, [&](auto gt) {
            by_dtype(bp.grad_dtype, [&](auto ot) {
                by_head_dim(pl.D, [&](auto dd) {
                    using IT = typename decltype(it)::type;
                    using GT = typename decltype(gt)::type;
                    using OT = typename decltype(ot)::type;
                    constexpr int DD = decltype(dd)::value;
                    hipLaunchKernelGGL((k_bwd_query_valu<IT, GT, OT, DD>), dim3(grid), dim3(kThreads), 0, stream,
                                       static_cast<const IT*>(q), static_cast<const GT*>(dout), state,
                                       static_cast<OT*>(dq), gpart, pl.N, pl.H, pl.L, pl.NB, bp.tpbq, eps);
                });
            });
        });
    });
    return hipGetLastError();
}

hipError_t launch_bwd_merge(const BwdPlan& bp, const float* gpart, float* ghat, hipStream_t stream) {
    const Plan& pl = bp.fw;
    const int SF = pl.D * (pl.D + 1);
    const unsigned grid = (unsigned)((size_t)pl.B * pl.H * ((SF + kThreads - 1) / kThreads));
    hipLaunchKernelGGL(k_bwd_merge_suffix, dim3(grid), dim3(kThreads), 0, stream, gpart, ghat, pl.NB, bp.tpbq, SF);
    return hipGetLastError();
}

hipError_t launch_bwd_key(const BwdPlan& bp, const void* k, const void* v, const float* ghat, void* dk, void* dv,
                          hipStream_t stream) {
    const Plan& pl = bp.fw;
    if (bp.key_mfma) {
        const unsigned grid = (unsigned)((size_t)pl.B * pl.HP * pl.NB * bp.tpbk);
        const uint16_t* k16 = static_cast<const uint16_t*>(k);
        const uint16_t* v16 = static_cast<const uint16_t*>(v);
        by_dtype(bp.grad_dtype, [&](auto ot) {
            using OT = typename decltype(ot)::type;
            if (pl.in_dtype == 0 && pl.D == 2 * kD)
                hipLaunchKernelGGL((k_bwd_key_mfma_f32_64<OT>), dim3(grid), dim3(kThreads), 0, stream,
                                   static_cast<const float*>(k), static_cast<const float*>(v), ghat,
                                   static_cast<OT*>(dk), static_cast<OT*>(dv), pl.N, pl.H, pl.L, pl.NB, bp.tk,
                                   bp.tpbk);
            else if (pl.in_dtype == 0)
                hipLaunchKernelGGL((pl.D == kD / 2 ? k_bwd_key_mfma_f32<OT, kD / 2> : k_bwd_key_mfma_f32<OT, kD>),
                                   dim3(grid), dim3(kThreads), 0, stream, static_cast<const float*>(k),
                                   static_cast<const float*>(v), ghat, static_cast<OT*>(dk), static_cast<OT*>(dv),
                                   pl.N, groups32(pl), pl.HP, pl.H, pl.L, pl.NB, bp.tk, bp.tpbk);
            else
                by_head_dim(pl.D, [&](auto dd) {
                    constexpr int DD = decltype(dd)::value;
                    hipLaunchKernelGGL((pl.in_dtype == 2 ? k_bwd_key_mfma<true, OT, DD> : k_bwd_key_mfma<false, OT, DD>),
                                       dim3(grid), dim3(kThreads), 0, stream, k16, v16, ghat, static_cast<OT*>(dk),
                                       static_cast<OT*>(dv), pl.N, groups32(pl), pl.HP, pl.H, pl.L, pl.NB, bp.tk,
                                       bp.tpbk);
                });
        });
        return hipGetLastError();
    }
    const unsigned grid = (unsigned)((size_t)pl.B * pl.H * pl.NB * bp.tpbk);
    by_dtype(pl.in_dtype, [&](auto it) {
        by_dtype(bp.grad_dtype, [&](auto ot) {
            by_head_dim(pl.D, [&](auto dd) {
                using IT = typename decltype(it)::type;
                using OT = typename decltype(ot)::type;
                constexpr int DD = decltype(dd)::value;
                hipLaunchKernelGGL((k_bwd_key_valu<IT, OT, DD>), dim3(grid), dim3(kThreads), 0, stream,
                                   static_cast<const IT*>(k), static_cast<const IT*>(v), ghat, static_cast<OT*>(dk),
                                   static_cast<OT*>(dv), pl.N, pl.H, pl.L, pl.NB, bp.tpbk);
            });
        });
    });
    return hipGetLastError();
}

}  // namespace sana
