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
// Everything accumulates in fp32; products of 16-bit inputs are exact.  Head
// dims 16 and 64 run the matrix-core kernels on 32-feature groups of the token
// row, as the forward's kernels do.
#include "linattn_device.h"

#include <type_traits>

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

// Writes a chunk's state and tangent-state partials, part[((b * HR + head) * 2
// + s) * P + p] (s = 0 the state, 1 the tangent state), from each wave's four
// accumulators acc = {S_v, S_z, St_v, St_z} (row 8 (r / 4) + 4 g + r % 4 of
// column j in register r of lane (g, j)).  Must be reached by the whole
// work-group.
//  - HD = 32 and 16: wave (hh, th) holds token half th of group h0 + hh's
//    sums; the halves are added in a fixed order through red (LDS, [head][4]
//    [16][64] floats).  HD = 16 keeps each group's diagonal 16 x 16 blocks, the
//    states of heads 2 (h0 + hh) and 2 (h0 + hh) + 1.
//  - HD = 64: wave (hh, th) holds the whole sums of block (K group hh, V group
//    th) of head h0 / 2 and writes them itself (V group 0 also the z column).
template <int HD>
__device__ __forceinline__ void jvp_write_partials(float* part, float* red, const f32x16 (&acc)[4], int b, int HR,
                                                   int h0, int nh, int P, int p, int hh, int th, int lane) {
    constexpr int SW = HD + 1, SF = HD * SW;
    const int g = lane >> 5, j = lane & 31;
    if constexpr (HD == 2 * kD) {
        const size_t bh = (size_t)b * HR + h0 / 2;
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            float* dst = part + ((bh * 2 + s) * P + p) * SF;
#pragma unroll
            for (int rg = 0; rg < 16; ++rg) {
                const int row = kD * hh + 8 * (rg >> 2) + 4 * g + (rg & 3);
                dst[row * SW + kD * th + j] = acc[2 * s][rg];
                if (th == 0 && j == 0) dst[row * SW + HD] = acc[2 * s + 1][rg];
            }
        }
        return;
    }
    __syncthreads();   // the tiles in red's space have been consumed
    if (th == 1) {
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4)
#pragma unroll
            for (int rg = 0; rg < 16; ++rg) red[((hh * 4 + q4) * 16 + rg) * 64 + lane] = acc[q4][rg];
    }
    __syncthreads();
    if (th != 0 || hh >= nh) return;
    auto sum = [&](int q4, int rg) { return acc[q4][rg] + red[((hh * 4 + q4) * 16 + rg) * 64 + lane]; };
#pragma unroll
    for (int rg = 0; rg < 16; ++rg) {
        int head, row, col;
        if constexpr (HD == kD / 2) {
            // rows 0..15 (rg < 8) are the group's first head, 16..31 its second;
            // the lanes of columns of the same half hold that head's state
            const int half = rg >> 3;
            head = 2 * (h0 + hh) + half;
            if ((j >> 4) != half || head >= HR) continue;
            row = 8 * ((rg >> 2) & 1) + 4 * g + (rg & 3);
            col = j & 15;
        } else {
            head = h0 + hh;
            row = 8 * (rg >> 2) + 4 * g + (rg & 3);
            col = j;
        }
        const size_t bh = (size_t)b * HR + head;
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            float* dst = part + ((bh * 2 + s) * P + p) * SF;
            dst[row * SW + col] = sum(2 * s, rg);
            if (col == 0) dst[row * SW + HD] = sum(2 * s + 1, rg);
        }
    }
}

// ------------------------------------------------------------------ state and tangent state, MFMA
// As the forward's state kernel, with four tensors in the LDS tile:
// [a | v | at | vt][head 0|1][token][32 x 16 bit].
constexpr int kJHead = kStateTile * 64 + 64;   // bytes per head (second head shifted by 64 bytes)
constexpr int kJTensor = 2 * kJHead;
constexpr int kJPieces = kStateTile / 32;
static_assert(4 * kJTensor >= 2 * 4 * 16 * 64 * (int)sizeof(float), "reduction area exceeds the LDS tile");

// grid.x = (b * HP + hp) * P + p.  Partials as jvp_write_partials.  Head dims
// 16 and 64 as in the forward's state kernel: H counts the 32-feature groups
// of a token row, HP their pairs, HR the real heads (rows of HR * HD elements;
// pieces past the row read as zero); HD = 64: wave w accumulates block (K
// group w & 1, V group w >> 1) over all tokens of each tile.
template <bool F16, int HD>
__global__ __launch_bounds__(kThreads) void k_jvp_state_mfma(
    const uint16_t* __restrict__ k, const uint16_t* __restrict__ v, const uint16_t* __restrict__ kt,
    const uint16_t* __restrict__ vt, float* __restrict__ part, int N, int H, int HP, int HR, int L, int cpb, int P,
    int chunk) {
    constexpr bool D64 = HD == 2 * kD;
    __shared__ __attribute__((aligned(16))) uint8_t lds[4 * kJTensor];

    const int p = blockIdx.x % P;
    const int bhp = blockIdx.x / P;
    const int hp = bhp % HP, b = bhp / HP;
    const int h0 = 2 * hp;
    const int nh = min(2, H - h0);
    const ChunkRange cr = chunk_range(p, cpb, chunk, L, N);
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int hh = wave & 1, th = wave >> 1;
    const long long hstride = (long long)HR * HD;
    const uint16_t* src[4] = {k, v, kt, vt};

    u32x4 r[4][kJPieces];
    auto load_tile = [&](int t0) {
#pragma unroll
        for (int i = 0; i < kJPieces; ++i) {
            const int pc = tid + kThreads * i;
            const int part_ = pc & 3, hd = (pc >> 2) & 1, tok = pc >> 3;
            const int n = t0 + tok;
            const int col = (h0 + hd) * kD + part_ * 8;
            const bool ok = n < cr.c1 && col < HR * HD;
            // a piece outside the range reads the range's first row, column 0 (in bounds)
            const long long off = ((long long)b * N + (ok ? n : cr.c0)) * hstride + (ok ? col : 0);
#pragma unroll
            for (int ts = 0; ts < 4; ++ts) {
                const u32x4 x = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(src[ts] + off));
                r[ts][i] = ok ? x : (u32x4){0u, 0u, 0u, 0u};
            }
        }
    };

    f32x16 acc[4] = {};   // S_v, S_z, St_v, St_z
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

        // K group hh (a, at); V group hh, or th for HD = 64 (v, vt)
        const uint16_t* T[4];
#pragma unroll
        for (int ts = 0; ts < 4; ++ts)
            T[ts] = reinterpret_cast<const uint16_t*>(lds + ts * kJTensor + ((D64 && (ts & 1)) ? th : hh) * kJHead);
#pragma unroll
        for (int st = 0; st < (D64 ? kStateTile / 16 : kStateTile / 32); ++st) {
            // element e of lane (g, j) is token tb + 2e + g (row j of a, at; column j of v, vt)
            const int tb = D64 ? 16 * st : (kStateTile / 2) * th + 16 * st;
            u32x4 op[4];
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const int r0 = (tb + 4 * t + g) * 32 + j;
                const int r1 = r0 + 2 * 32;
#pragma unroll
                for (int ts = 0; ts < 4; ++ts) op[ts][t] = (uint32_t)T[ts][r0] | ((uint32_t)T[ts][r1] << 16);
            }
            acc[0] = mfma16<F16>(op[0], op[1], acc[0]);
            if (!D64 || th == 0) acc[1] = mfma16<F16>(op[0], ones, acc[1]);
            acc[2] = mfma16<F16>(op[2], op[1], acc[2]);
            acc[2] = mfma16<F16>(op[0], op[3], acc[2]);
            if (!D64 || th == 0) acc[3] = mfma16<F16>(op[2], ones, acc[3]);
        }
    }
    jvp_write_partials<HD>(part, reinterpret_cast<float*>(lds), acc, b, HR, h0, nh, P, p, hh, th, lane);
}

// out = num r and out_t = (num_t - out den_t) r, r = 1 / (den + eps), from
// this lane's partial normaliser dot products (its half of the features; the
// partner lane i + 32 holds the other).  Head dim 16 (D16): rows 0..15 (r < 8)
// are the group's first head (dp, dpt), 16..31 its second (dp1, dpt1).
template <bool D16>
__device__ __forceinline__ void finish_tangent(f32x16& acc, f32x16& acct, float dp, float dpt, float dp1, float dpt1,
                                               float eps) {
    const float den = dp + __shfl_xor(dp, 32);
    const float dent = dpt + __shfl_xor(dpt, 32);
    const float rinv = 1.0f / (den + eps);
    float rinv1 = rinv, dent1 = dent;
    if constexpr (D16) {
        const float den1 = dp1 + __shfl_xor(dp1, 32);
        dent1 = dpt1 + __shfl_xor(dpt1, 32);
        rinv1 = 1.0f / (den1 + eps);
    }
#pragma unroll
    for (int rg = 0; rg < 16; ++rg) {
        const float r = (D16 && rg >= 8) ? rinv1 : rinv;
        const float dt = (D16 && rg >= 8) ? dent1 : dent;
        const float o = acc[rg] * r;
        acc[rg] = o;
        acct[rg] = (acct[rg] - o * dt) * r;
    }
}

// ------------------------------------------------------------------ output and tangent, MFMA
// grid.x = (b * HP + hp) * (NB * tpb) + beta * tpb + tile; wave w: 32-feature
// group 2*hp + (w & 1) of the token row, every other 32-token sub-tile
// (w >> 1).  H counts the groups, HR the real heads.  Head dim 32: the group
// is head 2 hp + (w & 1); 64: output half w & 1 of head hp, reducing over all
// 64 features of q; 16: heads 2 h and 2 h + 1 of group h against their
// block-diagonal states, each with its own normalisers (see apply_operands).
// Occupancy target of the 16-bit apply kernel: 3 waves per SIMD for bf16 q at
// head dims 16 and 32 with 16-bit outputs (166-168 VGPRs, no spills; the JVP
// with bf16 out 141-143 against 150 us, same box); with fp32 outputs that
// was slower (153-155 against 151 us), and fp16 q (the split of f and f_t)
// and head dim 64 would spill, so those are left to the compiler (2).
template <bool F16, int HD, typename OutT>
constexpr int jvp_apply_waves() { return !F16 && HD != 2 * kD && sizeof(OutT) == 2 ? 3 : 1; }

template <bool F16, typename OutT, int HD>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(jvp_apply_waves<F16, HD, OutT>(), 8))) void k_jvp_apply_mfma(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ qt, const float* __restrict__ state,
    OutT* __restrict__ out, OutT* __restrict__ outt, int N, int H, int HP, int HR, int L, int NB, int tile, int tpb,
    float eps) {
    constexpr int KS = KSteps<HD>::value, SF = HD * (HD + 1);
    constexpr bool D64 = HD == 2 * kD, D16 = HD == kD / 2;
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

    const size_t bhr = (size_t)b * HR;
    auto head_S = [&](int hr) { return state + (((bhr + hr) * 2 + 0) * NB + beta) * SF; };
    auto head_St = [&](int hr) { return state + (((bhr + hr) * 2 + 1) * NB + beta) * SF; };
    u32x4 sa[KS][3], sat[KS][3];
    // S[:, D] and St[:, D] at this lane's features 16 ks + 8 g + e, kept in
    // the wave's LDS (the same for all lanes of a half): registers go to the
    // operands
    __shared__ __attribute__((aligned(16))) float zlds[4][2][2][8 * KS];   // [wave][S | St][g]
    {
        float sz[8 * KS], szt[8 * KS];
        apply_operands<HD>(head_S, D64 ? hp : h, wave & 1, HR, lane, sa, sz);
        apply_operands<HD>(head_St, D64 ? hp : h, wave & 1, HR, lane, sat, szt);
        if (i == 0) {
#pragma unroll
            for (int e = 0; e < 8 * KS; ++e) {
                zlds[wave][0][g][e] = sz[e];
                zlds[wave][1][g][e] = szt[e];
            }
        }
        __builtin_amdgcn_wave_barrier();
        asm volatile("" ::: "memory");
    }
    const float* sz = zlds[wave][0][g];
    const float* szt = zlds[wave][1][g];

    const long long hstride = (long long)HR * HD;
    const int qcol = (D64 ? 2 * hp : h) * kD + 8 * g;   // this lane's first q feature in the row
    const bool second = !D16 || 2 * h + 1 < HR;       // head dim 16: the group has a second head
    const int ncols = second ? 32 : 16;
    float* ot = otile[wave];
    // One sub-tile's products, normalisers and stores from its prepared rows
    // f = ReLU(q) and f_t (zero where q <= 0); NC: the group's columns stored.
    auto body = [&](int tt, const u32x4 (&f)[KS], const u32x4 (&ft)[KS], auto ncols_c) {
        const int NC = ncols_c;   // an int, or a constant that folds the stores' column test
        const int n = min(32, t1 - tt);
        f32x16 acc = {}, acct = {};
        acc = mma_split_ks<F16, KS>(sa, f, acc);
        acct = mma_split_ks<F16, KS>(sat, f, acct);
        acct = mma_split_ks<F16, KS>(sa, ft, acct);
        float dp = 0.f, dpt = 0.f, dp1 = 0.f, dpt1 = 0.f;   // dp1, dpt1: head dim 16, the second head
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            float& a = (D16 && ks == 1) ? dp1 : dp;
            float& at = (D16 && ks == 1) ? dpt1 : dpt;
#pragma unroll
            for (int d = 0; d < 4; ++d) {
                float x0, x1, y0, y1;
                if constexpr (F16) {
                    x0 = f16_to_f32((uint16_t)(f[ks][d] & 0xffffu));
                    x1 = f16_to_f32((uint16_t)(f[ks][d] >> 16));
                    y0 = f16_to_f32((uint16_t)(ft[ks][d] & 0xffffu));
                    y1 = f16_to_f32((uint16_t)(ft[ks][d] >> 16));
                } else {
                    x0 = lo_bf16(f[ks][d]);
                    x1 = hi_bf16(f[ks][d]);
                    y0 = lo_bf16(ft[ks][d]);
                    y1 = hi_bf16(ft[ks][d]);
                }
                const int e = 8 * ks + 2 * d;
                a = fmaf(x0, sz[e], a);
                a = fmaf(x1, sz[e + 1], a);
                at = fmaf(x0, szt[e], at);
                at = fmaf(x1, szt[e + 1], at);
                at = fmaf(y0, sz[e], at);
                at = fmaf(y1, sz[e + 1], at);
            }
        }
        finish_tangent<D16>(acc, acct, dp, dpt, dp1, dpt1, eps);
        store_tile<OutT>(ot, acc, lane, n,
                         [&](int t) { return out + ((long long)b * N + tt + t) * hstride + h * kD; }, NC);
        store_tile<OutT>(ot, acct, lane, n,
                         [&](int t) { return outt + ((long long)b * N + tt + t) * hstride + h * kD; }, NC);
    };
    if constexpr (jvp_apply_waves<F16, HD, OutT>() != 3) {
        // The next sub-tile's rows are requested before this one's products
        // and prepared after its stores have been issued, so that the wait for
        // them leaves the stores in flight.  Loads are unconditional: rows past
        // the range are clamped to its last row (see store_tile), and a missing
        // second head of a group of dim 16 reads the first head's piece, zeroed
        // when prepared.  The stores are unconditional when the group's 32
        // columns all exist (a loop of its own for a lone head of dim 16).
        // (At 3 waves per SIMD the extra rows would spill: the loop below.)
        struct Rows {
            u32x4 x[KS], t[KS];
        };
        auto load = [&](int tt, Rows& r) {
            const int row = min(tt + i, t1 - 1);
            const u32x4* srcq = reinterpret_cast<const u32x4*>(q + ((long long)b * N + row) * hstride + qcol);
            const u32x4* srct = reinterpret_cast<const u32x4*>(qt + ((long long)b * N + row) * hstride + qcol);
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                const int c = ks == 0 || second ? 2 * ks : 0;   // features 16 ks + 8 g .. + 7 = src[2 ks]
                r.x[ks] = srcq[c];
                r.t[ks] = srct[c];
            }
        };
        u32x4 f[KS], ft[KS];
        auto prepare = [&](const Rows& r) {
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                const bool on = ks == 0 || second;
                f[ks] = relu_bf16x8(on ? r.x[ks] : (u32x4){0u, 0u, 0u, 0u});
                ft[ks] = keep_where_nonzero(f[ks], on ? r.t[ks] : (u32x4){0u, 0u, 0u, 0u});
            }
        };
        auto run = [&](auto ncols_c) {
            int tt = t0 + 32 * (wave >> 1);
            if (tt >= t1) return;
            Rows nx;
            load(tt, nx);
            prepare(nx);
            for (; tt < t1; tt += 64) {
                load(tt + 64, nx);
                body(tt, f, ft, ncols_c);
                prepare(nx);   // the next sub-tile's rows (past the end: the last row again, unused)
            }
        };
        if (ncols == 32)
            run(std::integral_constant<int, 32>{});
        else
            run(std::integral_constant<int, 16>{});
    } else {
        for (int tt = t0 + 32 * (wave >> 1); tt < t1; tt += 64) {
            const int row = min(tt + i, t1 - 1);   // clamped rows repeat the last row (see store_tile)
            const u32x4* srcq = reinterpret_cast<const u32x4*>(q + ((long long)b * N + row) * hstride + qcol);
            const u32x4* srct = reinterpret_cast<const u32x4*>(qt + ((long long)b * N + row) * hstride + qcol);
            u32x4 f[KS], ft[KS];
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                const bool on = ks == 0 || second;   // features 16 ks + 8 g .. + 7 = src[2 ks]
                f[ks] = relu_bf16x8(on ? srcq[2 * ks] : (u32x4){0u, 0u, 0u, 0u});
                ft[ks] = keep_where_nonzero(f[ks], on ? srct[2 * ks] : (u32x4){0u, 0u, 0u, 0u});
            }
            const int n = min(32, t1 - tt);

            f32x16 acc = {}, acct = {};
            acc = mma_split_ks<F16, KS>(sa, f, acc);
            acct = mma_split_ks<F16, KS>(sat, f, acct);
            acct = mma_split_ks<F16, KS>(sa, ft, acct);
            float dp = 0.f, dpt = 0.f, dp1 = 0.f, dpt1 = 0.f;   // dp1, dpt1: head dim 16, the second head
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                float& a = (D16 && ks == 1) ? dp1 : dp;
                float& at = (D16 && ks == 1) ? dpt1 : dpt;
#pragma unroll
                for (int d = 0; d < 4; ++d) {
                    float x0, x1, y0, y1;
                    if constexpr (F16) {
                        x0 = f16_to_f32((uint16_t)(f[ks][d] & 0xffffu));
                        x1 = f16_to_f32((uint16_t)(f[ks][d] >> 16));
                        y0 = f16_to_f32((uint16_t)(ft[ks][d] & 0xffffu));
                        y1 = f16_to_f32((uint16_t)(ft[ks][d] >> 16));
                    } else {
                        x0 = lo_bf16(f[ks][d]);
                        x1 = hi_bf16(f[ks][d]);
                        y0 = lo_bf16(ft[ks][d]);
                        y1 = hi_bf16(ft[ks][d]);
                    }
                    const int e = 8 * ks + 2 * d;
                    a = fmaf(x0, sz[e], a);
                    a = fmaf(x1, sz[e + 1], a);
                    at = fmaf(x0, szt[e], at);
                    at = fmaf(x1, szt[e + 1], at);
                    at = fmaf(y0, sz[e], at);
                    at = fmaf(y1, sz[e + 1], at);
                }
            }
            finish_tangent<D16>(acc, acct, dp, dpt, dp1, dpt1, eps);
            store_tile<OutT>(ot, acc, lane, n, [&](int t) { return out + ((long long)b * N + tt + t) * hstride + h * kD; },
                             ncols);
            store_tile<OutT>(ot, acct, lane, n,
                             [&](int t) { return outt + ((long long)b * N + tt + t) * hstride + h * kD; }, ncols);
        }
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
// Head dims 16 and 64 as in the 16-bit kernel ("heads" are 32-feature groups;
// HD = 64: wave w takes all 32 tokens of K group w & 1 against V group w >> 1).
constexpr int kJF32Tok = 32;
constexpr int kJF32Tile = kJF32Tok * kD;   // 16-bit elements of one term tile of one head

template <int HD>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(3, 8))) void k_jvp_state_mfma_f32(
    const float* __restrict__ k, const float* __restrict__ v, const float* __restrict__ kt,
    const float* __restrict__ vt, float* __restrict__ part, int N, int H, int HP, int HR, int L, int cpb, int P,
    int chunk) {
    constexpr bool D64 = HD == 2 * kD;
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
    const long long hstride = (long long)HR * HD;
    const float* src[4] = {k, v, kt, vt};

    // this thread's piece of a tile: part (tid & 3) = features 8 part .. + 7,
    // head (tid >> 2) & 1, token tid >> 3
    const int part_ = tid & 3, hd = (tid >> 2) & 1, tok = tid >> 3;
    f32x4 r[4][2];
    auto load_tile = [&](int t0) {
        const int n = t0 + tok;
        const int col = (h0 + hd) * kD + part_ * 8;
        const bool ok = n < cr.c1 && col < HR * HD;
        // a piece outside the range reads the range's first row, column 0 (in bounds)
        const long long off = ((long long)b * N + (ok ? n : cr.c0)) * hstride + (ok ? col : 0);
#pragma unroll
        for (int ts = 0; ts < 4; ++ts) {
            const f32x4* s = reinterpret_cast<const f32x4*>(src[ts] + off);
            const f32x4 x0 = s[0], x1 = s[1];   // plain loads: each reads half of a line
            r[ts][0] = ok ? x0 : (f32x4){0.f, 0.f, 0.f, 0.f};
            r[ts][1] = ok ? x1 : (f32x4){0.f, 0.f, 0.f, 0.f};
        }
    };

    f32x16 acc[4] = {};   // S_v, S_z, St_v, St_z
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

        // lane (g, j): tokens tb + 8 g + e of feature (a, at) / channel (v, vt)
        // j: wave (hh, th) takes token half th of group hh; for HD = 64 all
        // 32 tokens of K group hh against V group th
        const int vg = D64 ? th : hh;
#pragma unroll
        for (int st = 0; st < (D64 ? 2 : 1); ++st) {
            const int tb = D64 ? 16 * st : 16 * th;
            u32x4 ta[3], tv[3], tat[3], tvt[3];
#pragma unroll
            for (int sp = 0; sp < 3; ++sp) {
                ta[sp] = gather_tokens_t16(lds[0][sp][hh], kD, tb, 0, lane);
                tv[sp] = gather_tokens_t16(lds[1][sp][vg], kD, tb, 0, lane);
                tat[sp] = gather_tokens_t16(lds[2][sp][hh], kD, tb, 0, lane);
                tvt[sp] = gather_tokens_t16(lds[3][sp][vg], kD, tb, 0, lane);
            }
            // smallest products first
            acc[0] = mma_terms(ta, tv, acc[0]);
            acc[2] = mfma_bf16(tat[2], tv[0], acc[2]);
            acc[2] = mfma_bf16(tat[1], tv[1], acc[2]);
            acc[2] = mfma_bf16(tat[0], tv[2], acc[2]);
            acc[2] = mfma_bf16(ta[2], tvt[0], acc[2]);
            acc[2] = mfma_bf16(ta[1], tvt[1], acc[2]);
            acc[2] = mfma_bf16(ta[0], tvt[2], acc[2]);
            acc[2] = mfma_bf16(tat[1], tv[0], acc[2]);
            acc[2] = mfma_bf16(tat[0], tv[1], acc[2]);
            acc[2] = mfma_bf16(ta[1], tvt[0], acc[2]);
            acc[2] = mfma_bf16(ta[0], tvt[1], acc[2]);
            acc[2] = mfma_bf16(tat[0], tv[0], acc[2]);
            acc[2] = mfma_bf16(ta[0], tvt[0], acc[2]);
            if (!D64 || th == 0) {
#pragma unroll
                for (int sp = 2; sp >= 0; --sp) {
                    acc[1] = mfma_bf16(ta[sp], ones, acc[1]);
                    acc[3] = mfma_bf16(tat[sp], ones, acc[3]);
                }
            }
        }
    }
    jvp_write_partials<HD>(part, reinterpret_cast<float*>(&lds[0][0][0][0]), acc, b, HR, h0, nh, P, p, hh, th,
                           lane);
}

// Output and tangent for fp32 q and qt: the 16-bit kernel's waves, groups and
// sub-tiles, q and qt read per wave in the operand layout (the next
// sub-tile's loads in flight during this one's work), f = ReLU(q) and
// ft = [q > 0] qt split into three bf16 terms each:
//   num = S_v^T f (6 term products per K-step), numt = St_v^T f + S_v^T ft (12);
// the normalisers are fp32 dot products of the unsplit values.
template <typename OutT, int HD>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 8))) void k_jvp_apply_mfma_f32(
    const float* __restrict__ q, const float* __restrict__ qt, const float* __restrict__ state,
    OutT* __restrict__ out, OutT* __restrict__ outt, int N, int H, int HP, int HR, int L, int NB, int tile, int tpb,
    float eps) {
    constexpr int KS = KSteps<HD>::value, SF = HD * (HD + 1);
    constexpr bool D64 = HD == 2 * kD, D16 = HD == kD / 2;
    constexpr int G = KS / 2;   // 32-feature groups of q a wave reads
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

    const size_t bhr = (size_t)b * HR;
    auto head_S = [&](int hr) { return state + (((bhr + hr) * 2 + 0) * NB + beta) * SF; };
    auto head_St = [&](int hr) { return state + (((bhr + hr) * 2 + 1) * NB + beta) * SF; };
    u32x4 sa[KS][3], sat[KS][3];
    // S[:, D] and St[:, D] at this lane's features 16 ks + 8 g + e, kept in
    // the wave's LDS (the same for all lanes of a half): registers go to the
    // operands
    __shared__ __attribute__((aligned(16))) float zlds[4][2][2][8 * KS];   // [wave][S | St][g]
    {
        float sz[8 * KS], szt[8 * KS];
        apply_operands<HD>(head_S, D64 ? hp : h, wave & 1, HR, lane, sa, sz);
        apply_operands<HD>(head_St, D64 ? hp : h, wave & 1, HR, lane, sat, szt);
        if (i == 0) {
#pragma unroll
            for (int e = 0; e < 8 * KS; ++e) {
                zlds[wave][0][g][e] = sz[e];
                zlds[wave][1][g][e] = szt[e];
            }
        }
        __builtin_amdgcn_wave_barrier();
        asm volatile("" ::: "memory");
    }
    const float* sz = zlds[wave][0][g];
    const float* szt = zlds[wave][1][g];

    const long long hstride = (long long)HR * HD;
    const int qcol = (D64 ? 2 * hp : h) * kD;     // first q feature of the wave's groups in the row
    const bool second = !D16 || 2 * h + 1 < HR;   // head dim 16: the group has a second head
    const int ncols = second ? 32 : 16;
    auto row_of = [&](const float* x, int tt) { return x + ((long long)b * N + min(tt + i, t1 - 1)) * hstride + qcol; };
    auto load = [&](F32Operand (&o)[G], const float* x, int tt) {
#pragma unroll
        for (int gi = 0; gi < G; ++gi) o[gi].load(row_of(x, tt) + kD * gi, g, second);
    };
    float* ot = otile[wave];
    F32Operand qc[G], tc[G];
    load(qc, q, t0 + 32 * (wave >> 1));
    load(tc, qt, t0 + 32 * (wave >> 1));
    for (int tt = t0 + 32 * (wave >> 1); tt < t1; tt += 64) {
        const int n = min(32, t1 - tt);   // clamped rows repeat the last row (see store_tile)
        // the next sub-tile's rows in flight during this one's work (head dim
        // 64 reads them after it: two groups of q and qt would not fit)
        F32Operand qn[G], tn[G];
        const bool more = tt + 64 < t1;
        if (more && G == 1) {
            load(qn, q, tt + 64);
            load(tn, qt, tt + 64);
        }
        f32x16 acc = {}, acct = {};
        float dp = 0.f, dpt = 0.f, dp1 = 0.f, dpt1 = 0.f;   // dp1, dpt1: head dim 16, the second head
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            float& a = (D16 && ks == 1) ? dp1 : dp;
            float& at = (D16 && ks == 1) ? dpt1 : dpt;
            float f[8], ft[8];
            qc[ks >> 1].half(ks & 1, true, f);
            tc[ks >> 1].half(ks & 1, false, ft);
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                ft[e] = f[e] > 0.f ? ft[e] : 0.f;
                a = fmaf(f[e], sz[8 * ks + e], a);
                at = fmaf(f[e], szt[8 * ks + e], at);
                at = fmaf(ft[e], sz[8 * ks + e], at);
            }
            u32x4 tf[3], tft[3];
            split3_trunc_f32x8(f, tf);
            split3_trunc_f32x8(ft, tft);
            acc = mma_terms(sa[ks], tf, acc);
            acct = mma_terms(sat[ks], tf, acct);
            acct = mma_terms(sa[ks], tft, acct);
        }
        finish_tangent<D16>(acc, acct, dp, dpt, dp1, dpt1, eps);
        store_tile<OutT>(ot, acc, lane, n, [&](int t) { return out + ((long long)b * N + tt + t) * hstride + h * kD; },
                         ncols);
        store_tile<OutT>(ot, acct, lane, n,
                         [&](int t) { return outt + ((long long)b * N + tt + t) * hstride + h * kD; }, ncols);
        if (more && G == 1) {
            qc[0] = qn[0];
            tc[0] = tn[0];
        } else if (more) {
            load(qc, q, tt + 64);
            load(tc, qt, tt + 64);
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
    if (pl.mfma) {
        const unsigned grid = (unsigned)((size_t)pl.B * pl.HP * pl.P);
        const uint16_t *k16 = static_cast<const uint16_t*>(k), *v16 = static_cast<const uint16_t*>(v),
                       *kt16 = static_cast<const uint16_t*>(kt), *vt16 = static_cast<const uint16_t*>(vt);
        by_head_dim(pl.D, [&](auto dd) {
            constexpr int DD = decltype(dd)::value;
            if (pl.in_dtype == 0)
                hipLaunchKernelGGL(k_jvp_state_mfma_f32<DD>, dim3(grid), dim3(kThreads), 0, stream,
                                   static_cast<const float*>(k), static_cast<const float*>(v),
                                   static_cast<const float*>(kt), static_cast<const float*>(vt), part, pl.N,
                                   groups32(pl), pl.HP, pl.H, pl.L, pl.cpb, pl.P, pl.chunk);
            else
                hipLaunchKernelGGL((pl.in_dtype == 2 ? k_jvp_state_mfma<true, DD> : k_jvp_state_mfma<false, DD>),
                                   dim3(grid), dim3(kThreads), 0, stream, k16, v16, kt16, vt16, part, pl.N,
                                   groups32(pl), pl.HP, pl.H, pl.L, pl.cpb, pl.P, pl.chunk);
        });
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
    if (pl.mfma) {
        const unsigned grid = (unsigned)((size_t)pl.B * pl.HP * pl.NB * pl.tpb);
        const uint16_t *q16 = static_cast<const uint16_t*>(q), *qt16 = static_cast<const uint16_t*>(qt);
        by_dtype(pl.out_dtype, [&](auto o) {
            by_head_dim(pl.D, [&](auto dd) {
                using OT = typename decltype(o)::type;
                constexpr int DD = decltype(dd)::value;
                if (pl.in_dtype == 0)
                    hipLaunchKernelGGL((k_jvp_apply_mfma_f32<OT, DD>), dim3(grid), dim3(kThreads), 0, stream,
                                       static_cast<const float*>(q), static_cast<const float*>(qt), state,
                                       static_cast<OT*>(out), static_cast<OT*>(outt), pl.N, groups32(pl), pl.HP,
                                       pl.H, pl.L, pl.NB, pl.tile, pl.tpb, eps);
                else
                    hipLaunchKernelGGL((pl.in_dtype == 2 ? k_jvp_apply_mfma<true, OT, DD> : k_jvp_apply_mfma<false, OT, DD>),
                                       dim3(grid), dim3(kThreads), 0, stream, q16, qt16, state, static_cast<OT*>(out),
                                       static_cast<OT*>(outt), pl.N, groups32(pl), pl.HP, pl.H, pl.L, pl.NB, pl.tile,
                                       pl.tpb, eps);
            });
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
