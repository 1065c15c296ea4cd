// C ABI of the LiteLA forward library: argument checks, work decomposition,
// workspace layout and the enqueueing of the three kernels.  The operator and
// the conventions are documented in include/sana_linattn.h.
#include "sana_linattn.h"

#include <algorithm>
#include <climits>
#include <cmath>
#include <cstdint>
#include <cstdlib>
#include <cstring>

#include "linattn_internal.h"

using sana::Plan;

namespace {

constexpr int kMaxN = 1 << 30;        // keeps every token index, and N + block_len, in int range
constexpr int kMaxBH = 1 << 24;       // batch and head counts

// Positive integer from the environment, or 0 when unset or not a positive integer.
int env_positive(const char* name) {
    const char* s = std::getenv(name);
    if (!s || !*s) return 0;
    char* end = nullptr;
    const long v = std::strtol(s, &end, 10);
    if (*end != '\0' || v <= 0 || v > kMaxN) return 0;
    return (int)v;
}

bool env_is(const char* name, const char* value) {
    const char* s = std::getenv(name);
    return s && std::strcmp(s, value) == 0;
}

int ceil_div(long a, long b) { return (int)((a + b - 1) / b); }
long round_up(long a, long m) { return (a + m - 1) / m * m; }

// Decomposition of one call.  Sizes were range-checked by the caller.
// allow_mfma = false gives the vector path's plan (for workspace queries).
// split_state: the keys take the split-term state kernel whatever their type
// (qk_norm), which holds 3 work-groups per CU like the fp32 one.
int make_plan(int in_dtype, int out_dtype, int B, int H, int N, int D, int block_len, Plan* pl,
              bool allow_mfma = true, bool split_state = false) {
    if (B < 0 || H < 0 || N < 0 || D < 1 || block_len < 0) return SANA_ERR_INVALID_ARG;
    if ((in_dtype != SANA_DT_F32 && in_dtype != SANA_DT_BF16 && in_dtype != SANA_DT_F16) ||
        (out_dtype != SANA_DT_F32 && out_dtype != SANA_DT_BF16 && out_dtype != SANA_DT_F16))
        return SANA_ERR_INVALID_ARG;
    if (D != 16 && D != 32 && D != 64) return SANA_ERR_UNSUPPORTED;
    if (N > kMaxN || B > kMaxBH || H > kMaxBH) return SANA_ERR_UNSUPPORTED;

    std::memset(pl, 0, sizeof *pl);
    pl->B = B;
    pl->H = H;
    pl->N = N;
    pl->in_dtype = in_dtype;
    pl->out_dtype = out_dtype;
    pl->D = D;
    if (B == 0 || H == 0 || N == 0) return SANA_OK;   // empty problem, no workspace

    pl->L = (block_len == 0 || block_len >= N) ? N : block_len;
    pl->NB = ceil_div(N, pl->L);
    // matrix cores for every head dim and input type (the kernels see a token
    // row as 32-feature groups: a head of 64 is two of them, a group holds two
    // heads of 16); units are pairs of groups
    pl->mfma = (allow_mfma && !env_is("SANA_LINATTN_PATH", "valu")) ? 1 : 0;
    pl->mfma16 = pl->mfma && in_dtype != SANA_DT_F32;
    pl->HP = pl->mfma ? ceil_div(ceil_div((long)H * D, sana::kD), 2) : H;
    const long units = (long)B * pl->HP * pl->NB;   // independent (b, head unit, block) triples

    // Work-groups per launch follow the tuned targets kStateGroups and
    // kApplyGroups (each launch is a single round on the chip).  Chunks and
    // apply tiles are whole multiples of 64 tokens and never cross a block.
    int chunk = env_positive("SANA_LINATTN_CHUNK");
    if (chunk) {
        chunk = (int)round_up(chunk, 64);
    } else {
        // the split-term state kernel (fp32 keys, and qk_norm keys of any
        // type) streams best with one full round of as many work-groups as
        // fit a CU: 3 with fp32 V (48 KB of LDS each), 4 with 16-bit V (32
        // or 40 KB)
        const long slots = !(pl->mfma && (in_dtype == SANA_DT_F32 || split_state)) ? sana::kStateGroups
                           : sana::kCUs * (in_dtype == SANA_DT_F32 ? 3 : 4);
        const long per_block = std::max<long>(1, slots / units);
        chunk = (int)std::max<long>(round_up(ceil_div(pl->L, per_block), 64), sana::kMinChunk);
    }
    chunk = (int)std::min<long>(chunk, round_up(pl->L, 64));
    pl->chunk = chunk;
    pl->cpb = ceil_div(pl->L, chunk);
    pl->P = pl->NB * pl->cpb;

    if (pl->mfma) {
        int tile = env_positive("SANA_LINATTN_APPLY_TILE");
        if (tile) {
            tile = (int)round_up(tile, 64);
        } else {
            // head dim 64 runs the apply kernel at 3 waves per SIMD (2 for fp32
            // q), so at most that many work-groups fit on a CU; the block count
            // per unit is rounded to nearest, so that many short units (the
            // block-causal shapes) still get about the target
            const long slots = D == 2 * sana::kD ? sana::kCUs * (in_dtype == SANA_DT_F32 ? 2 : 3) : sana::kApplyGroups;
            const long per_block = std::max<long>(1, (slots + units / 2) / units);
            tile = (int)round_up(ceil_div(pl->L, per_block), 64);
        }
        pl->tile = (int)std::min<long>(tile, round_up(pl->L, 64));
    } else {
        pl->tile = sana::kValuApplyTokens;
    }
    pl->tpb = ceil_div(pl->L, pl->tile);

    // Launch grids are one-dimensional.
    if ((long)B * pl->HP * pl->P > INT_MAX || units * pl->tpb > INT_MAX || (long)B * H > INT_MAX)
        return SANA_ERR_UNSUPPORTED;

    const size_t bh = (size_t)B * H;
    const size_t sf = (size_t)D * (D + 1);   // floats per state
    size_t off = 0;
    pl->off_part = off;
    off += round_up((long)(bh * pl->P * sf * sizeof(float)), 256);
    pl->off_state = off;
    off += round_up((long)(bh * pl->NB * sf * sizeof(float)), 256);
    pl->bytes = off;
    return SANA_OK;
}

bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
    const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
    return na && nb && x < y + nb && y < x + na;
}

bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

// Bytes spanned by a [B][N][H][D] view with element strides st (B, N >= 1).
size_t extent_bytes(sana::Strides st, int B, int N, int H, int D, size_t es) {
    return (size_t)((B - 1) * st.b + (long long)(N - 1) * st.n + (long long)H * D) * es;
}

// Whether the (b, n) rows of H*D elements of a view with strides st are
// pairwise disjoint (required of the output).
bool rows_disjoint(sana::Strides st, int B, int N, int H, int D) {
    const long long row = (long long)H * D;
    long long s1 = st.n, c1 = N, s2 = st.b, c2 = B;   // inner and outer row strides and counts
    if (c1 == 1) { s1 = s2; c1 = c2; s2 = 0; c2 = 1; }
    if (c2 > 1 && s2 < s1) { std::swap(s1, s2); std::swap(c1, c2); }
    if (c1 > 1 && s1 < row) return false;
    if (c2 > 1 && s2 < (c1 - 1) * s1 + row) return false;
    return true;
}

int forward(const void* q, const void* k, const void* v, void* out, int in_dtype, int out_dtype,
            int B, int H, int N, int D, int block_len, float eps, void* workspace,
            size_t workspace_bytes, hipStream_t stream, int stages,
            const float* state_in = nullptr, float* state_out = nullptr,
            const int64_t* strides = nullptr, const float* gamma_q = nullptr, const float* gamma_k = nullptr,
            float norm_eps = 0.f, float* states_out = nullptr) {
    Plan pl;
    const int st = make_plan(in_dtype, out_dtype, B, H, N, D, block_len, &pl, true, gamma_k != nullptr);
    if (st != SANA_OK) return st;
    if (!std::isfinite(eps) || eps < 0.f) return SANA_ERR_INVALID_ARG;
    if ((gamma_q || gamma_k) && !(std::isfinite(norm_eps) && norm_eps > 0.f)) return SANA_ERR_INVALID_ARG;
    pl.gq = gamma_q;
    pl.gk = gamma_k;
    pl.norm_eps = norm_eps;
    if (stages <= 0 || (stages & ~SANA_STAGE_ALL)) return SANA_ERR_INVALID_ARG;
    const size_t es_in = in_dtype == SANA_DT_F32 ? 4 : 2;
    const size_t es_out = out_dtype == SANA_DT_F32 ? 4 : 2;
    const sana::Strides dense = {(long long)N * H * D, (long long)H * D};
    pl.sq = pl.sk = pl.sv = pl.so = dense;
    if (strides) {
        for (int i = 0; i < 8; ++i)
            if (strides[i] < 0 || strides[i] > (1LL << 46)) return SANA_ERR_INVALID_ARG;
        pl.sq = {strides[0], strides[1]};
        pl.sk = {strides[2], strides[3]};
        pl.sv = {strides[4], strides[5]};
        pl.so = {strides[6], strides[7]};
        for (int i = 0; i < 8; ++i)   // every row starts 16-byte aligned
            if ((strides[i] * (long long)(i < 6 ? es_in : es_out)) % 16) return SANA_ERR_ALIGNMENT;
        if (B > 0 && H > 0 && N > 0 && !rows_disjoint(pl.so, B, N, H, D)) return SANA_ERR_ALIAS;
    }
    if (B == 0 || H == 0 || N == 0) return SANA_OK;
    if (!q || !k || !v || !out || !workspace) return SANA_ERR_INVALID_ARG;
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(out, 16) || !aligned(workspace, 256))
        return SANA_ERR_ALIGNMENT;
    const size_t q_bytes = extent_bytes(pl.sq, B, N, H, D, es_in);
    const size_t k_bytes = extent_bytes(pl.sk, B, N, H, D, es_in);
    const size_t v_bytes = extent_bytes(pl.sv, B, N, H, D, es_in);
    const size_t out_bytes = extent_bytes(pl.so, B, N, H, D, es_out);
    if (overlaps(out, out_bytes, q, q_bytes) || overlaps(out, out_bytes, k, k_bytes) ||
        overlaps(out, out_bytes, v, v_bytes))
        return SANA_ERR_ALIAS;
    if (overlaps(workspace, pl.bytes, q, q_bytes) || overlaps(workspace, pl.bytes, k, k_bytes) ||
        overlaps(workspace, pl.bytes, v, v_bytes) || overlaps(workspace, pl.bytes, out, out_bytes))
        return SANA_ERR_ALIAS;
    if (state_in || state_out) {
        const size_t sb = (size_t)B * H * D * (D + 1) * sizeof(float);
        if ((state_in && !aligned(state_in, 4)) || (state_out && !aligned(state_out, 4)))
            return SANA_ERR_ALIGNMENT;
        if (state_in && (overlaps(state_in, sb, out, out_bytes) || overlaps(state_in, sb, workspace, pl.bytes)))
            return SANA_ERR_ALIAS;
        if (state_out && (overlaps(state_out, sb, q, q_bytes) || overlaps(state_out, sb, k, k_bytes) ||
                          overlaps(state_out, sb, v, v_bytes) || overlaps(state_out, sb, out, out_bytes) ||
                          overlaps(state_out, sb, workspace, pl.bytes) ||
                          (state_in && state_in != state_out && overlaps(state_out, sb, state_in, sb))))
            return SANA_ERR_ALIAS;
    }
    if (states_out) {   // the per-block prefix states, [B][H][NB][D][D+1] (no entry point passes a carried state too)
        const size_t sb = (size_t)B * H * pl.NB * D * (D + 1) * sizeof(float);
        if (!aligned(states_out, 4)) return SANA_ERR_ALIGNMENT;
        if (overlaps(states_out, sb, q, q_bytes) || overlaps(states_out, sb, k, k_bytes) ||
            overlaps(states_out, sb, v, v_bytes) || overlaps(states_out, sb, out, out_bytes) ||
            overlaps(states_out, sb, workspace, pl.bytes))
            return SANA_ERR_ALIAS;
    }
    if (gamma_q || gamma_k) {
        const size_t gb = (size_t)H * D * sizeof(float);
        for (const float* gp : {gamma_q, gamma_k}) {
            if (!gp) continue;
            if (!aligned(gp, 4)) return SANA_ERR_ALIGNMENT;
            if (overlaps(gp, gb, out, out_bytes) || overlaps(gp, gb, workspace, pl.bytes)) return SANA_ERR_ALIAS;
        }
    }
    if (workspace_bytes < pl.bytes) return SANA_ERR_WORKSPACE;

    uint8_t* ws = static_cast<uint8_t*>(workspace);
    float* part = reinterpret_cast<float*>(ws + pl.off_part);
    float* state = states_out ? states_out : reinterpret_cast<float*>(ws + pl.off_state);
    if ((stages & SANA_STAGE_STATE) && sana::launch_state(pl, k, v, part, stream) != hipSuccess)
        return SANA_ERR_HIP;
    if ((stages & SANA_STAGE_MERGE) && sana::launch_merge(pl, part, state, state_in, state_out, stream) != hipSuccess)
        return SANA_ERR_HIP;
    if ((stages & SANA_STAGE_APPLY) && sana::launch_apply(pl, q, state, out, eps, stream) != hipSuccess)
        return SANA_ERR_HIP;
    return SANA_OK;
}

// Backward decomposition: the forward's state plan plus query/key tiles and
// the gradient-state workspace behind the forward's.
constexpr int kBwdTile = 256;   // tokens per query/key work-group (one per thread)

int make_bwd_plan(int in_dtype, int dout_dtype, int grad_dtype, int B, int H, int N, int D, int block_len,
                  sana::BwdPlan* bp, bool allow_mfma = true) {
    std::memset(bp, 0, sizeof *bp);
    const int st = make_plan(in_dtype, SANA_DT_F32, B, H, N, D, block_len, &bp->fw, allow_mfma);
    if (st != SANA_OK) return st;
    for (int c : {dout_dtype, grad_dtype})
        if (c != SANA_DT_F32 && c != SANA_DT_BF16 && c != SANA_DT_F16) return SANA_ERR_INVALID_ARG;
    bp->dout_dtype = dout_dtype;
    bp->grad_dtype = grad_dtype;
    if (B == 0 || H == 0 || N == 0) return SANA_OK;
    const Plan& pl = bp->fw;
    // the matrix-core query and key kernels take every head dim and input
    // type (the vector kernels only with SANA_LINATTN_PATH=valu)
    bp->query_mfma = pl.mfma;
    bp->key_mfma = pl.mfma;
    bp->tk = bp->tq = kBwdTile;
    if (bp->query_mfma || bp->key_mfma) {
        // Tiles (multiples of 64 tokens inside one block) for the (batch, head
        // pair, block) units: the key and query kernels' registers and LDS
        // fit 3 work-groups per CU (2 for fp32 inputs and for the head-dim-64
        // key kernel).  The tile count per block
        // minimises rounds of work-groups x (tile + 64), the 64 tokens
        // standing for a work-group's prologue and epilogue: one round when
        // the units allow it, else short tiles that fill the last round.
        const long units = (long)B * pl.HP * pl.NB;
        auto tile_for = [&](long per_cu) {
            const long slots = sana::kCUs * per_cu;
            const long max_tile = round_up(pl.L, 64);
            const long pb_max = std::min<long>(ceil_div(pl.L, 64), 4 * slots / units + 1);
            long best = max_tile, best_cost = LONG_MAX;
            for (long pb = 1; pb <= pb_max; ++pb) {
                const long tile = std::min<long>(round_up(ceil_div(pl.L, pb), 64), max_tile);
                const long rounds = (units * ceil_div(pl.L, tile) + slots - 1) / slots;
                const long cost = rounds * (tile + 64);
                if (cost < best_cost) {
                    best_cost = cost;
                    best = tile;
                }
            }
            return (int)best;
        };
        const int per_cu = pl.mfma16 ? 3 : 2;
        if (bp->key_mfma) bp->tk = tile_for(D == 2 * sana::kD ? 2 : per_cu);
        if (bp->query_mfma) bp->tq = tile_for(D == 2 * sana::kD ? 2 : per_cu);
        // 16-bit inputs and dout: the query kernels that load their rows per
        // wave (every head dim); for them and the 16-bit key kernel at head
        // dims 32 and 16 tiles sized for 2 work-groups per CU: they run faster
        // with fewer, longer work-groups (490 of 1216 tokens at 16384 x 70)
        // than with every slot of the CUs filled
        bp->query_direct = pl.mfma16 && dout_dtype != SANA_DT_F32;
        if (pl.mfma16 && D <= sana::kD) bp->tk = tile_for(2);
        if (bp->query_direct) bp->tq = tile_for(2);
        if (const int t = env_positive("SANA_LINATTN_BWD_TILE"))
            bp->tk = bp->tq = (int)std::min<long>(round_up(t, 64), round_up(pl.L, 64));
    }
    if (!bp->query_mfma && D == 2 * sana::kD) bp->tq = kBwdTile / 4;   // the vector query kernel's tokens per work-group
    bp->tpbq = ceil_div(pl.L, bp->tq);
    bp->tpbk = ceil_div(pl.L, bp->tk);
    bp->Pq = pl.NB * bp->tpbq;
    if ((long)B * H * pl.NB * std::max(bp->tpbq, bp->tpbk) > INT_MAX) return SANA_ERR_UNSUPPORTED;
    const size_t bh = (size_t)B * H;
    size_t off = pl.bytes;
    bp->off_gpart = off;
    off += round_up((long)(bh * bp->Pq * (size_t)D * (D + 1) * sizeof(float)), 256);
    bp->off_ghat = off;
    off += round_up((long)(bh * pl.NB * (size_t)D * (D + 1) * sizeof(float)), 256);
    bp->bytes = off;
    return SANA_OK;
}

// states_in: the forward's per-block prefix states ([B][H][NB][D][D+1]), or
// nullptr to rebuild them from k and v.
int backward(const void* q, const void* k, const void* v, const void* dout, void* dq, void* dk, void* dv,
             int in_dtype, int dout_dtype, int grad_dtype, int B, int H, int N, int D, int block_len, float eps,
             void* workspace, size_t workspace_bytes, hipStream_t stream, const float* states_in = nullptr) {
    sana::BwdPlan bp;
    const int st = make_bwd_plan(in_dtype, dout_dtype, grad_dtype, B, H, N, D, block_len, &bp);
    if (st != SANA_OK) return st;
    if (!std::isfinite(eps) || eps < 0.f) return SANA_ERR_INVALID_ARG;
    if (B == 0 || H == 0 || N == 0) return SANA_OK;
    const void* ins[4] = {q, k, v, dout};
    void* outs[3] = {dq, dk, dv};
    for (const void* p : ins)
        if (!p) return SANA_ERR_INVALID_ARG;
    for (void* p : outs)
        if (!p) return SANA_ERR_INVALID_ARG;
    if (!workspace) return SANA_ERR_INVALID_ARG;
    for (const void* p : ins)
        if (!aligned(p, 16)) return SANA_ERR_ALIGNMENT;
    for (void* p : outs)
        if (!aligned(p, 16)) return SANA_ERR_ALIGNMENT;
    if (!aligned(workspace, 256)) return SANA_ERR_ALIGNMENT;
    const size_t elems = (size_t)B * N * H * D;
    const size_t es_in = in_dtype == SANA_DT_F32 ? 4 : 2;
    const size_t in_b[4] = {elems * es_in, elems * es_in, elems * es_in,
                            elems * (dout_dtype == SANA_DT_F32 ? 4 : 2)};
    const size_t gb = elems * (grad_dtype == SANA_DT_F32 ? 4 : 2);
    for (int i = 0; i < 3; ++i) {
        for (int j = 0; j < 4; ++j)
            if (overlaps(outs[i], gb, ins[j], in_b[j])) return SANA_ERR_ALIAS;
        for (int j = i + 1; j < 3; ++j)
            if (overlaps(outs[i], gb, outs[j], gb)) return SANA_ERR_ALIAS;
        if (overlaps(outs[i], gb, workspace, bp.bytes)) return SANA_ERR_ALIAS;
    }
    for (int j = 0; j < 4; ++j)
        if (overlaps(workspace, bp.bytes, ins[j], in_b[j])) return SANA_ERR_ALIAS;
    if (states_in) {
        const size_t sb = (size_t)B * H * bp.fw.NB * D * (D + 1) * sizeof(float);
        if (!aligned(states_in, 4)) return SANA_ERR_ALIGNMENT;
        for (void* p : outs)
            if (overlaps(p, gb, states_in, sb)) return SANA_ERR_ALIAS;
        if (overlaps(workspace, bp.bytes, states_in, sb)) return SANA_ERR_ALIAS;
    }
    if (workspace_bytes < bp.bytes) return SANA_ERR_WORKSPACE;

    Plan& pl = bp.fw;
    pl.sq = pl.sk = pl.sv = pl.so = {(long long)N * H * D, (long long)H * D};
    uint8_t* ws = static_cast<uint8_t*>(workspace);
    float* part = reinterpret_cast<float*>(ws + pl.off_part);
    float* state = reinterpret_cast<float*>(ws + pl.off_state);
    float* gpart = reinterpret_cast<float*>(ws + bp.off_gpart);
    float* ghat = reinterpret_cast<float*>(ws + bp.off_ghat);
    if (!states_in && (sana::launch_state(pl, k, v, part, stream) != hipSuccess ||
                       sana::launch_merge(pl, part, state, nullptr, nullptr, stream) != hipSuccess))
        return SANA_ERR_HIP;
    if (sana::launch_bwd_query(bp, q, dout, states_in ? states_in : state, dq, gpart, eps, stream) != hipSuccess ||
        sana::launch_bwd_merge(bp, gpart, ghat, stream) != hipSuccess ||
        sana::launch_bwd_key(bp, k, v, ghat, dk, dv, stream) != hipSuccess)
        return SANA_ERR_HIP;
    return SANA_OK;
}

// Forward-mode derivative: the forward's plan with the workspace doubled (a
// state and a tangent state per head).
int make_jvp_plan(int in_dtype, int out_dtype, int B, int H, int N, int D, int block_len, Plan* pl,
                  bool allow_mfma = true) {
    const int st = make_plan(in_dtype, out_dtype, B, H, N, D, block_len, pl, allow_mfma);
    if (st != SANA_OK) return st;
    // head dims 16 and 64 on the matrix cores only (the vector kernels are built for 32)
    if (D != sana::kD && !pl->mfma && B > 0 && H > 0 && N > 0) return SANA_ERR_UNSUPPORTED;
    if (B == 0 || H == 0 || N == 0) return SANA_OK;
    const size_t bh2 = (size_t)B * H * 2;
    if ((long long)bh2 > INT_MAX) return SANA_ERR_UNSUPPORTED;
    const size_t sf = (size_t)D * (D + 1);
    pl->off_part = 0;
    pl->off_state = round_up((long)(bh2 * pl->P * sf * sizeof(float)), 256);
    pl->bytes = pl->off_state + round_up((long)(bh2 * pl->NB * sf * sizeof(float)), 256);
    return SANA_OK;
}

int jvp(const void* q, const void* k, const void* v, const void* qt, const void* kt, const void* vt, void* out,
        void* outt, int in_dtype, int out_dtype, int B, int H, int N, int D, int block_len, float eps, void* workspace,
        size_t workspace_bytes, hipStream_t stream) {
    Plan pl;
    const int st = make_jvp_plan(in_dtype, out_dtype, B, H, N, D, block_len, &pl);
    if (st != SANA_OK) return st;
    if (!std::isfinite(eps) || eps < 0.f) return SANA_ERR_INVALID_ARG;
    if (B == 0 || H == 0 || N == 0) return SANA_OK;
    const void* ins[6] = {q, k, v, qt, kt, vt};
    void* outs[2] = {out, outt};
    for (const void* p : ins)
        if (!p) return SANA_ERR_INVALID_ARG;
    if (!out || !outt || !workspace) return SANA_ERR_INVALID_ARG;
    for (const void* p : ins)
        if (!aligned(p, 16)) return SANA_ERR_ALIGNMENT;
    if (!aligned(out, 16) || !aligned(outt, 16) || !aligned(workspace, 256)) return SANA_ERR_ALIGNMENT;
    const size_t elems = (size_t)B * N * H * D;
    const size_t ib = elems * (in_dtype == SANA_DT_F32 ? 4 : 2), ob = elems * (out_dtype == SANA_DT_F32 ? 4 : 2);
    for (int i = 0; i < 2; ++i) {
        for (const void* p : ins)
            if (overlaps(outs[i], ob, p, ib)) return SANA_ERR_ALIAS;
        if (overlaps(outs[i], ob, workspace, pl.bytes)) return SANA_ERR_ALIAS;
    }
    if (overlaps(out, ob, outt, ob)) return SANA_ERR_ALIAS;
    for (const void* p : ins)
        if (overlaps(workspace, pl.bytes, p, ib)) return SANA_ERR_ALIAS;
    if (workspace_bytes < pl.bytes) return SANA_ERR_WORKSPACE;

    uint8_t* ws = static_cast<uint8_t*>(workspace);
    float* part = reinterpret_cast<float*>(ws + pl.off_part);
    float* state = reinterpret_cast<float*>(ws + pl.off_state);
    Plan pm = pl;   // the merge sees the state and the tangent state of a head as two heads
    pm.H = 2 * H;
    if (sana::launch_jvp_state(pl, k, v, kt, vt, part, stream) != hipSuccess ||
        sana::launch_merge(pm, part, state, nullptr, nullptr, stream) != hipSuccess ||
        sana::launch_jvp_apply(pl, q, qt, state, out, outt, eps, stream) != hipSuccess)
        return SANA_ERR_HIP;
    return SANA_OK;
}

}  // namespace

namespace sana {

int forward_call(const void* q, const void* k, const void* v, void* out, int in_dtype, int out_dtype, int B, int H,
                 int N, int D, int block_len, float eps, void* workspace, size_t workspace_bytes, hipStream_t stream) {
    return forward(q, k, v, out, in_dtype, out_dtype, B, H, N, D, block_len, eps, workspace, workspace_bytes, stream,
                   SANA_STAGE_ALL);
}

int forward_workspace(int in_dtype, int out_dtype, int B, int H, int N, int D, int block_len, size_t* bytes) {
    Plan pl;
    const int st = make_plan(in_dtype, out_dtype, B, H, N, D, block_len, &pl);
    if (st != SANA_OK) return st;
    *bytes = pl.bytes;
    return SANA_OK;
}

}  // namespace sana

extern "C" {

int sana_linattn_abi_version(void) { return SANA_LINATTN_ABI_VERSION; }

const char* sana_linattn_status_string(int status) {
    switch (status) {
        case SANA_OK: return "success";
        case SANA_ERR_INVALID_ARG: return "invalid argument";
        case SANA_ERR_UNSUPPORTED: return "unsupported size or head dim (D must be 16, 32 or 64)";
        case SANA_ERR_ALIGNMENT: return "misaligned pointer (tensors need 16 bytes, workspace 256)";
        case SANA_ERR_ALIAS: return "output or workspace overlaps another buffer";
        case SANA_ERR_WORKSPACE: return "workspace too small";
        case SANA_ERR_HIP: return "HIP runtime error while enqueueing";
        case SANA_ERR_SCRATCH:
            return "problem needs more scratch than the no-allocation entry point holds (SANA_LINATTN_SCRATCH_BYTES)";
        default: return "unknown status";
    }
}

int sana_linattn_workspace_bytes(int B, int H, int N, int D, int block_len, size_t* bytes) {
    if (!bytes) return SANA_ERR_INVALID_ARG;
    Plan pl;
    const int st = make_plan(SANA_DT_BF16, SANA_DT_F32, B, H, N, D, block_len, &pl);
    if (st != SANA_OK) return st;
    // fp32 inputs and qk_norm keys (the split-term state kernel's own
    // chunking) and the vector path (SANA_LINATTN_PATH=valu) may need more;
    // report the largest.
    Plan pf, pq, pv;
    make_plan(SANA_DT_F32, SANA_DT_F32, B, H, N, D, block_len, &pf);
    make_plan(SANA_DT_BF16, SANA_DT_F32, B, H, N, D, block_len, &pq, true, true);
    make_plan(SANA_DT_F32, SANA_DT_F32, B, H, N, D, block_len, &pv, false);
    *bytes = std::max({pl.bytes, pf.bytes, pq.bytes, pv.bytes});
    return SANA_OK;
}

int sana_linattn_bwd_workspace_bytes(int B, int H, int N, int D, int block_len, size_t* bytes) {
    if (!bytes) return SANA_ERR_INVALID_ARG;
    // the plan (its query tiles, and so the partial gradient states) depends
    // on the input type (16-bit or fp32) and on whether dout is 16-bit: the
    // most any of them needs
    size_t most = 0;
    for (int dt : {SANA_DT_BF16, SANA_DT_F32})
        for (int gt : {SANA_DT_BF16, SANA_DT_F32})
            for (bool mf : {true, false}) {   // the vector path's plan too (SANA_LINATTN_PATH=valu)
                sana::BwdPlan bp;
                const int st = make_bwd_plan(dt, gt, SANA_DT_F32, B, H, N, D, block_len, &bp, mf);
                if (st != SANA_OK) return st;
                most = std::max(most, bp.bytes);
            }
    *bytes = most;
    return SANA_OK;
}

int sana_linattn_bwd(const void* q, const void* k, const void* v, const void* dout, void* dq, void* dk,
                     void* dv, int in_dtype, int dout_dtype, int grad_dtype, int B, int H, int N, int D,
                     int block_len, float eps, void* workspace, size_t workspace_bytes, hipStream_t stream) {
    if (block_len < 0) return SANA_ERR_INVALID_ARG;
    return backward(q, k, v, dout, dq, dk, dv, in_dtype, dout_dtype, grad_dtype, B, H, N, D, block_len, eps,
                    workspace, workspace_bytes, stream);
}

int sana_linattn_states_bytes(int B, int H, int N, int D, int block_len, size_t* bytes) {
    if (!bytes) return SANA_ERR_INVALID_ARG;
    Plan pl;
    const int st = make_plan(SANA_DT_BF16, SANA_DT_F32, B, H, N, D, block_len, &pl);
    if (st != SANA_OK) return st;
    *bytes = (B == 0 || H == 0 || N == 0) ? 0 : (size_t)B * H * pl.NB * D * (D + 1) * sizeof(float);
    return SANA_OK;
}

int sana_linattn_fwd_save_states(const void* q, const void* k, const void* v, void* out, int in_dtype,
                                 int out_dtype, int B, int H, int N, int D, int block_len, float eps, float* states,
                                 void* workspace, size_t workspace_bytes, hipStream_t stream) {
    if (block_len < 0) return SANA_ERR_INVALID_ARG;
    if (!states && B > 0 && H > 0 && N > 0) return SANA_ERR_INVALID_ARG;
    return forward(q, k, v, out, in_dtype, out_dtype, B, H, N, D, block_len, eps, workspace, workspace_bytes,
                   stream, SANA_STAGE_ALL, nullptr, nullptr, nullptr, nullptr, nullptr, 0.f, states);
}

int sana_linattn_bwd_from_states(const void* q, const void* k, const void* v, const void* dout, const float* states,
                                 void* dq, void* dk, void* dv, int in_dtype, int dout_dtype, int grad_dtype, int B,
                                 int H, int N, int D, int block_len, float eps, void* workspace,
                                 size_t workspace_bytes, hipStream_t stream) {
    if (block_len < 0) return SANA_ERR_INVALID_ARG;
    if (!states && B > 0 && H > 0 && N > 0) return SANA_ERR_INVALID_ARG;
    return backward(q, k, v, dout, dq, dk, dv, in_dtype, dout_dtype, grad_dtype, B, H, N, D, block_len, eps,
                    workspace, workspace_bytes, stream, states);
}

int sana_linattn_jvp_workspace_bytes(int B, int H, int N, int D, int block_len, size_t* bytes) {
    if (!bytes) return SANA_ERR_INVALID_ARG;
    size_t most = 0;
    for (int dt : {SANA_DT_BF16, SANA_DT_F32})
        for (bool mf : {true, false}) {   // the vector path's plan too (SANA_LINATTN_PATH=valu)
            Plan pl;
            const int st = make_jvp_plan(dt, SANA_DT_F32, B, H, N, D, block_len, &pl, mf);
            if (st == SANA_ERR_UNSUPPORTED && !mf && D != sana::kD) continue;   // no vector path for that dim
            if (st != SANA_OK) return st;
            most = std::max(most, pl.bytes);
        }
    *bytes = most;
    return SANA_OK;
}

int sana_linattn_jvp(const void* q, const void* k, const void* v, const void* q_t, const void* k_t, const void* v_t,
                     void* out, void* out_t, int in_dtype, int out_dtype, int B, int H, int N, int D, int block_len,
                     float eps, void* workspace, size_t workspace_bytes, hipStream_t stream) {
    if (block_len < 0) return SANA_ERR_INVALID_ARG;
    return jvp(q, k, v, q_t, k_t, v_t, out, out_t, in_dtype, out_dtype, B, H, N, D, block_len, eps, workspace,
               workspace_bytes, stream);
}

int sana_linattn_plan_info(int in_dtype, int B, int H, int N, int D, int block_len, int* chunk_tokens,
                           int* num_chunks, int* apply_tokens, int* mfma) {
    Plan pl;
    const int st = make_plan(in_dtype, SANA_DT_F32, B, H, N, D, block_len, &pl);
    if (st != SANA_OK) return st;
    if (chunk_tokens) *chunk_tokens = pl.chunk;
    if (num_chunks) *num_chunks = pl.P;
    if (apply_tokens) *apply_tokens = pl.tile;
    if (mfma) *mfma = pl.mfma;
    return SANA_OK;
}

int sana_linattn_fwd(const void* q, const void* k, const void* v, void* out, int in_dtype, int out_dtype,
                     int B, int H, int N, int D, float eps, void* workspace, size_t workspace_bytes,
                     hipStream_t stream) {
    return forward(q, k, v, out, in_dtype, out_dtype, B, H, N, D, 0, eps, workspace, workspace_bytes,
                   stream, SANA_STAGE_ALL);
}

int sana_linattn_blockcausal_fwd(const void* q, const void* k, const void* v, void* out, int in_dtype,
                                 int out_dtype, int B, int H, int N, int D, int block_len, float eps,
                                 void* workspace, size_t workspace_bytes, hipStream_t stream) {
    if (block_len < 1) return SANA_ERR_INVALID_ARG;
    return forward(q, k, v, out, in_dtype, out_dtype, B, H, N, D, block_len, eps, workspace,
                   workspace_bytes, stream, SANA_STAGE_ALL);
}

int sana_linattn_blockcausal_stream_fwd(const void* q, const void* k, const void* v, void* out, int in_dtype,
                                        int out_dtype, int B, int H, int N, int D, int block_len, float eps,
                                        const float* state_in, float* state_out, void* workspace,
                                        size_t workspace_bytes, hipStream_t stream) {
    if (block_len < 1) return SANA_ERR_INVALID_ARG;
    return forward(q, k, v, out, in_dtype, out_dtype, B, H, N, D, block_len, eps, workspace,
                   workspace_bytes, stream, SANA_STAGE_ALL, state_in, state_out);
}

int sana_linattn_fwd_strided(const void* q, const void* k, const void* v, void* out, int in_dtype,
                             int out_dtype, int B, int H, int N, int D, int block_len, float eps,
                             const int64_t* strides, void* workspace, size_t workspace_bytes,
                             hipStream_t stream) {
    if (!strides || block_len < 0) return SANA_ERR_INVALID_ARG;
    return forward(q, k, v, out, in_dtype, out_dtype, B, H, N, D, block_len, eps, workspace,
                   workspace_bytes, stream, SANA_STAGE_ALL, nullptr, nullptr, strides);
}

int sana_linattn_fwd_qknorm(const void* q, const void* k, const void* v, void* out, int in_dtype, int out_dtype,
                            int B, int H, int N, int D, int block_len, float eps, const float* gamma_q,
                            const float* gamma_k, float norm_eps, const int64_t* strides, void* workspace,
                            size_t workspace_bytes, hipStream_t stream) {
    if (block_len < 0) return SANA_ERR_INVALID_ARG;
    return forward(q, k, v, out, in_dtype, out_dtype, B, H, N, D, block_len, eps, workspace, workspace_bytes,
                   stream, SANA_STAGE_ALL, nullptr, nullptr, strides, gamma_q, gamma_k, norm_eps);
}

int sana_linattn_fwd_stages(const void* q, const void* k, const void* v, void* out, int in_dtype,
                            int out_dtype, int B, int H, int N, int D, int block_len, float eps,
                            void* workspace, size_t workspace_bytes, hipStream_t stream, int stages) {
    return forward(q, k, v, out, in_dtype, out_dtype, B, H, N, D, block_len, eps, workspace,
                   workspace_bytes, stream, stages);
}

}  // extern "C"
