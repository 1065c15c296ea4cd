// Internal interface between the C-ABI layer (linattn_api.cpp) and the gfx950
// kernels (linattn_kernels.hip).  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace sana {

constexpr int kD = 32;                    // head dim (every Sana model: linear_head_dim 32)
constexpr int kW = kD + 1;                // state row: D value columns + the normaliser column
constexpr int kStateFloats = kD * kW;     // 1056 floats per (b, h) state
constexpr int kThreads = 256;             // 4 wave64 per work-group, every kernel
constexpr int kStateTile = 128;           // tokens per LDS tile, matrix-core state kernel
constexpr int kValuTile = 64;             // tokens per LDS tile, vector state kernel
constexpr int kValuApplyTokens = 256;     // tokens per work-group, vector apply kernel

// Apply-side operand pack for one (b, h, block): the fp32 state split into three
// bf16 terms (hi + mid + lo), already in the per-lane order of the B operand of
// v_mfma_f32_32x32x16_bf16.
//   value part  [ks 2][split 3][lane 64][8 x bf16]   lane = 32*g + c, element e:
//               S[16*ks + 8*g + e][c]
//   norm part   [ks 2][split 3][g 2][8 x bf16]       element e: S[16*ks + 8*g + e][D]
constexpr int kPackValueBytes = 2 * 3 * 64 * 16;               // 6144
constexpr int kPackBytes = kPackValueBytes + 2 * 3 * 2 * 16;   // 6336

struct Plan {
    int B, H, N;
    int L;        // block length in tokens (N for the non-causal operator)
    int NB;       // number of blocks
    int HP;       // head units per batch: head pairs (matrix path) or heads (vector path)
    int chunk;    // tokens per state chunk (multiple of kStateTile)
    int cpb;      // chunks per block
    int P;        // chunks per (b, h) = NB * cpb
    int tile;     // tokens per apply work-group
    int tpb;      // apply work-groups per block
    int mfma;     // 1: bf16 matrix-core kernels, 0: vector kernels
    int in_dtype, out_dtype;
    size_t off_part, off_state, off_pack, bytes;
};

// Each launcher enqueues one kernel on `stream` and returns hipGetLastError().
hipError_t launch_state(const Plan& pl, const void* k, const void* v, float* part, hipStream_t stream);
hipError_t launch_merge(const Plan& pl, const float* part, float* state, uint8_t* pack, hipStream_t stream);
hipError_t launch_apply(const Plan& pl, const void* q, const float* state, const uint8_t* pack,
                        void* out, float eps, hipStream_t stream);

}  // namespace sana
