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
// reductions run in fixed orders, so results are bitwise repeatable.
#include "linattn_internal.h"

namespace sana {
namespace {

__device__ __forceinline__ float ld(const float* p, long long i) { return p[i]; }
__device__ __forceinline__ float ld(const uint16_t* p, long long i) {
    return __builtin_bit_cast(float, (uint32_t)p[i] << 16);
}
__device__ __forceinline__ float ld(const _Float16* p, long long i) { return (float)p[i]; }

// Round to nearest, ties to even (finite inputs; NaN is kept a quiet NaN).
__device__ __forceinline__ uint16_t to_bf16(float f) {
    uint32_t u = __builtin_bit_cast(uint32_t, f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}
__device__ __forceinline__ void st(float* p, long long i, float x) { p[i] = x; }
__device__ __forceinline__ void st(uint16_t* p, long long i, float x) { p[i] = to_bf16(x); }
__device__ __forceinline__ void st(_Float16* p, long long i, float x) { p[i] = (_Float16)x; }

constexpr int kTok = 256;   // tokens per work-group of the vector kernels (one per thread)

// ------------------------------------------------------------------ query pass, vector unit
// grid.x = ((b * H + h) * NB + beta) * tpb + tile; thread t = token
// blk0 + tile * 256 + t of block beta.  Writes dq and the tile's partial
// gradient state gpart[(b * H + h) * (NB * tpb) + beta * tpb + tile].
template <typename InT, typename GT, typename OutT>
__global__ __launch_bounds__(kThreads) void k_bwd_query_valu(
    const InT* __restrict__ q, const GT* __restrict__ dout, const float* __restrict__ state,
    OutT* __restrict__ dq, float* __restrict__ gpart, int N, int H, int L, int NB, int tpb, float eps) {
    __shared__ float sP[kStateFloats];
    __shared__ float sf[kTok][kD + 1];    // f of each token (padded row)
    __shared__ float suw[kTok][kW];       // [u | w] of each token

    const int tile = blockIdx.x % tpb;
    const size_t bhb = blockIdx.x / tpb;          // (b * H + h) * NB + beta
    const int beta = (int)(bhb % NB);
    const size_t bh = bhb / NB;
    const int h = (int)(bh % H), b = (int)(bh / H);
    for (int e = threadIdx.x; e < kStateFloats; e += kThreads) sP[e] = state[bhb * kStateFloats + e];
    __syncthreads();

    const int blk0 = beta * L, blk1 = min(blk0 + L, N);
    const int t = threadIdx.x;
    const int row = blk0 + tile * kTok + t;
    if (row < blk1) {
        const long long base = (((long long)b * N + row) * H + h) * kD;
        float f[kD], u[kD];
#pragma unroll
        for (int j = 0; j < kD; ++j) {
            const float x = ld(q, base + j);
            f[j] = x > 0.f ? x : 0.f;
            sf[t][j] = f[j];
        }
        float den = 0.f;
#pragma unroll
        for (int j = 0; j < kD; ++j) den += f[j] * sP[j * kW + kD];
        const float r = 1.0f / (den + eps);
        float go = 0.f;   // dout . num
        for (int c = 0; c < kD; ++c) {
            float num = 0.f;
#pragma unroll
            for (int j = 0; j < kD; ++j) num += f[j] * sP[j * kW + c];
            const float g = ld(dout, base + c);
            go += g * num;
            u[c] = g * r;
            suw[t][c] = u[c];
        }
        const float w = -(r * r) * go;
        suw[t][kD] = w;
        for (int j = 0; j < kD; ++j) {
            float s = sP[j * kW + kD] * w;
#pragma unroll
            for (int c = 0; c < kD; ++c) s += sP[j * kW + c] * u[c];
            st(dq, base + j, ld(q, base + j) > 0.f ? s : 0.f);
        }
    } else {
        for (int j = 0; j < kD; ++j) sf[t][j] = 0.f;
        for (int c = 0; c < kW; ++c) suw[t][c] = 0.f;
    }
    __syncthreads();
    // partial gradient state of this tile: thread t owns entries t, t + 256, ...
    float* dst = gpart + (bhb * tpb + tile) * kStateFloats;   // (bh * NB + beta) * tpb + tile
    for (int e = t; e < kStateFloats; e += kThreads) {
        const int j = e / kW, c = e - j * kW;
        float s = 0.f;
        for (int tok = 0; tok < kTok; ++tok) s += sf[tok][j] * suw[tok][c];
        dst[e] = s;
    }
}

// ------------------------------------------------------------------ suffix merge
// grid.x = (b * H + h) * kGroups + m; thread t owns entry e = m * 256 + t.
// For beta = NB-1 down to 0: the block's tile partials are summed (groups of 8
// loads in flight, a fixed pairwise tree) and added to the running suffix sum,
// which is written as Ghat of block beta.
constexpr int kGroups = (kStateFloats + kThreads - 1) / kThreads;

__global__ __launch_bounds__(kThreads) void k_bwd_merge_suffix(const float* __restrict__ gpart,
                                                                float* __restrict__ ghat, int NB, int tpb) {
    const size_t bh = blockIdx.x / kGroups;
    const int e = (blockIdx.x % kGroups) * kThreads + threadIdx.x;
    if (e >= kStateFloats) return;
    const float* src = gpart + bh * NB * tpb * kStateFloats + e;
    float* dst = ghat + bh * NB * kStateFloats + e;
    float acc = 0.f;
    for (int beta = NB - 1; beta >= 0; --beta) {
        const float* blk = src + (size_t)beta * tpb * kStateFloats;
        float bs = 0.f;
        for (int s0 = 0; s0 < tpb; s0 += 8) {
            float x[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) x[i] = (s0 + i < tpb) ? blk[(size_t)(s0 + i) * kStateFloats] : 0.f;
            bs += ((x[0] + x[1]) + (x[2] + x[3])) + ((x[4] + x[5]) + (x[6] + x[7]));
        }
        acc += bs;
        dst[(size_t)beta * kStateFloats] = acc;
    }
}

// ------------------------------------------------------------------ key pass, vector unit
// grid.x = ((b * H + h) * NB + beta) * tpb + tile; thread t = key token
// blk0 + tile * 256 + t of block beta.
template <typename InT, typename OutT>
__global__ __launch_bounds__(kThreads) void k_bwd_key_valu(
    const InT* __restrict__ k, const InT* __restrict__ v, const float* __restrict__ ghat,
    OutT* __restrict__ dk, OutT* __restrict__ dv, int N, int H, int L, int NB, int tpb) {
    __shared__ float sG[kStateFloats];
    const int tile = blockIdx.x % tpb;
    const size_t bhb = blockIdx.x / tpb;
    const int beta = (int)(bhb % NB);
    const size_t bh = bhb / NB;
    const int h = (int)(bh % H), b = (int)(bh / H);
    for (int e = threadIdx.x; e < kStateFloats; e += kThreads) sG[e] = ghat[bhb * kStateFloats + e];
    __syncthreads();
    const int blk0 = beta * L, blk1 = min(blk0 + L, N);
    const int row = blk0 + tile * kTok + threadIdx.x;
    if (row >= blk1) return;
    const long long base = (((long long)b * N + row) * H + h) * kD;
    float a[kD], x[kD];
#pragma unroll
    for (int j = 0; j < kD; ++j) {
        const float kk = ld(k, base + j);
        a[j] = kk > 0.f ? kk : 0.f;
        x[j] = ld(v, base + j);
    }
    for (int j = 0; j < kD; ++j) {
        float s = sG[j * kW + kD];
#pragma unroll
        for (int c = 0; c < kD; ++c) s += sG[j * kW + c] * x[c];
        st(dk, base + j, a[j] > 0.f ? s : 0.f);
    }
    for (int c = 0; c < kD; ++c) {
        float s = 0.f;
#pragma unroll
        for (int j = 0; j < kD; ++j) s += a[j] * sG[j * kW + c];
        st(dv, base + c, s);
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
    const unsigned grid = (unsigned)((size_t)pl.B * pl.H * pl.NB * bp.tpbq);
    by_dtype(pl.in_dtype, [&](auto it) {
        by_dtype(bp.dout_dtype, [&](auto gt) {
            by_dtype(bp.grad_dtype, [&](auto ot) {
                using IT = typename decltype(it)::type;
                using GT = typename decltype(gt)::type;
                using OT = typename decltype(ot)::type;
                hipLaunchKernelGGL((k_bwd_query_valu<IT, GT, OT>), dim3(grid), dim3(kThreads), 0, stream,
                                   static_cast<const IT*>(q), static_cast<const GT*>(dout), state,
                                   static_cast<OT*>(dq), gpart, pl.N, pl.H, pl.L, pl.NB, bp.tpbq, eps);
            });
        });
    });
    return hipGetLastError();
}

hipError_t launch_bwd_merge(const BwdPlan& bp, const float* gpart, float* ghat, hipStream_t stream) {
    const Plan& pl = bp.fw;
    const unsigned grid = (unsigned)((size_t)pl.B * pl.H * kGroups);
    hipLaunchKernelGGL(k_bwd_merge_suffix, dim3(grid), dim3(kThreads), 0, stream, gpart, ghat, pl.NB, bp.tpbq);
    return hipGetLastError();
}

hipError_t launch_bwd_key(const BwdPlan& bp, const void* k, const void* v, const float* ghat, void* dk, void* dv,
                          hipStream_t stream) {
    const Plan& pl = bp.fw;
    const unsigned grid = (unsigned)((size_t)pl.B * pl.H * pl.NB * bp.tpbk);
    by_dtype(pl.in_dtype, [&](auto it) {
        by_dtype(bp.grad_dtype, [&](auto ot) {
            using IT = typename decltype(it)::type;
            using OT = typename decltype(ot)::type;
            hipLaunchKernelGGL((k_bwd_key_valu<IT, OT>), dim3(grid), dim3(kThreads), 0, stream,
                               static_cast<const IT*>(k), static_cast<const IT*>(v), ghat, static_cast<OT*>(dk),
                               static_cast<OT*>(dv), pl.N, pl.H, pl.L, pl.NB, bp.tpbk);
        });
    });
    return hipGetLastError();
}

}  // namespace sana
