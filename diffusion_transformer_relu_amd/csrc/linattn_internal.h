// Internal interface between the C-ABI layer (linattn_api.cpp) and the gfx950
// kernels (linattn_kernels.hip).  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <type_traits>

namespace sana {

constexpr int kD = 32;                    // head dim of the matrix-core kernels (every Sana model: 32)
constexpr int kW = kD + 1;                // state row: D value columns + the normaliser column
constexpr int kStateFloats = kD * kW;     // 1056 floats per (b, h) state
constexpr int kThreads = 256;             // 4 wave64 per work-group, every kernel
constexpr int kStateTile = 64;            // tokens per LDS tile, matrix-core state kernel
constexpr int kValuTile = 64;             // tokens per LDS tile, vector state kernel
constexpr int kValuApplyTokens = 256;     // tokens per work-group, vector apply kernel
constexpr int kMergeThreads = 256;        // state entries per merge work-group

// Work-group counts per launch, tuned on MI355X (256 CUs).  The state kernel
// streams K/V fastest with at most 2 work-groups on any CU: at the 4096px shape
// 490 groups of 1216-token chunks take 25.5 us, 560 groups of 1024 (some CUs
// holding 3) 26.7 us, 525 of 1152 27.7 us, 1120 of 512 28.9 us.  The apply
// kernel likewise prefers at most 4 per CU (1015 groups of 576 tokens:
// 35.3 us with fp32 out and 25.8 with bf16 out, against 35.7 and 26.7 for 1120
// groups of 512).
constexpr int kCUs = 256;
constexpr int kStateGroups = kCUs * 2;
constexpr int kApplyGroups = kCUs * 4;
// Smallest state chunk: the 1024px Sana shapes (2 x 1024 tokens) take 128-
// and 192-token chunks, 2 to 3 % faster than 256 (their partials are a larger
// share of the bytes there, but these calls are bound by their few
// work-groups, not by HBM); large problems have far longer chunks anyway.
constexpr int kMinChunk = 128;

// Element strides of a [B][N][H][D] tensor view: consecutive heads are D
// elements apart and features are contiguous; batch and token strides are free
// (e.g. q, k, v as views of one fused qkv projection output).
struct Strides {
    long long b, n;
};

struct Plan {
    int B, H, N;
    int L;        // block length in tokens (N for the non-causal operator)
    int NB;       // number of blocks
    int HP;       // units per batch: pairs of 32-feature groups (matrix path) or heads (vector path)
    int chunk;    // tokens per state chunk (multiple of 64)
    int cpb;      // chunks per block
    int P;        // chunks per (b, h) = NB * cpb
    int tile;     // tokens per apply work-group
    int tpb;      // apply work-groups per block
    int mfma;     // 1: matrix-core kernels, 0: vector kernels
    int mfma16;   // 1: mfma with 16-bit inputs
    int D;        // head dim: 16, 32 or 64
    int in_dtype, out_dtype;
    // qk_norm prologue: per-channel scales [H][D] of q and k (device fp32, or
    // nullptr for none) and the constant under the root
    const float* gq;
    const float* gk;
    float norm_eps;
    size_t off_part, off_state, bytes;
    Strides sq, sk, sv, so;   // element strides of q, k, v, out
};

// 32-feature groups of a token row: the "heads" of the matrix-core kernels (a
// head of dim 64 is two groups, a group holds two heads of dim 16).
inline int groups32(const Plan& pl) { return (pl.H * pl.D + kD - 1) / kD; }

// Calls f with std::integral_constant<int, D> for a head dim D of 16, 32 or 64.
template <typename F> void by_head_dim(int D, F&& f) {
    if (D == 16)
        f(std::integral_constant<int, 16>{});
    else if (D == 64)
        f(std::integral_constant<int, 64>{});
    else
        f(std::integral_constant<int, 32>{});
}

// The forward behind every forward entry point (linattn_api.cpp): argument
// checks, then the state, merge and apply kernels on `stream` with the given
// workspace; returns a sana_status_t code.
int forward_call(const void* q, const void* k, const void* v, void* out, int in_dtype, int out_dtype, int B, int H,
                 int N, int D, int block_len, float eps, void* workspace, size_t workspace_bytes, hipStream_t stream);
// Workspace bytes that forward_call needs for these arguments (0 for an empty
// problem); a sana_status_t code for invalid sizes, dtypes or head dims.
int forward_workspace(int in_dtype, int out_dtype, int B, int H, int N, int D, int block_len, size_t* bytes);

// Each launcher enqueues one kernel on `stream` and returns hipGetLastError().
hipError_t launch_state(const Plan& pl, const void* k, const void* v, float* part, hipStream_t stream);
hipError_t launch_merge(const Plan& pl, const float* part, float* state, const float* state_in,
                        float* state_out, hipStream_t stream);
hipError_t launch_apply(const Plan& pl, const void* q, const float* state, void* out, float eps,
                        hipStream_t stream);

// Backward: the forward's state and merge kernels rebuild the prefix states
// P (fw.off_part, fw.off_state), then
//   query kernel - per query tile: dq, and one partial gradient state
//                  G = sum_i f_i [dL/dnum_i | dL/dden_i] per tile;
//   suffix merge - Ghat of block beta = sum of the tiles' G over blocks >= beta;
//   key kernel   - per key: dk, dv from Ghat of its block.
struct BwdPlan {
    Plan fw;
    int dout_dtype, grad_dtype;
    int tq, tpbq, Pq;    // query tile, query tiles per block, query tiles per (b, h)
    int tk, tpbk;        // key tile, key tiles per block
    int query_mfma, key_mfma;   // 1: matrix-core query / key kernels
    int query_direct;           // 1: the head-dim-32 query kernel for 16-bit q and dout (per-wave row loads)
    size_t off_gpart, off_ghat, bytes;
};

hipError_t launch_bwd_query(const BwdPlan& bp, const void* q, const void* dout, const float* state, void* dq,
                            float* gpart, float eps, hipStream_t stream);
hipError_t launch_bwd_merge(const BwdPlan& bp, const float* gpart, float* ghat, hipStream_t stream);
hipError_t launch_bwd_key(const BwdPlan& bp, const void* k, const void* v, const float* ghat, void* dk, void* dv,
                          hipStream_t stream);

// Forward-mode derivative: partial and merged states hold the state and the
// tangent state of each head, [B][H][2][P or NB][kStateFloats]; the forward's
// merge kernel runs on them as 2 H heads.
hipError_t launch_jvp_state(const Plan& pl, const void* k, const void* v, const void* kt, const void* vt, float* part,
                            hipStream_t stream);
hipError_t launch_jvp_apply(const Plan& pl, const void* q, const void* qt, const float* state, void* out, void* outt,
                            float eps, hipStream_t stream);

}  // namespace sana
