/*
 * sana_linattn.h -- C ABI of the MI355X (gfx950) LiteLA forward library.
 *
 * LiteLA is the ReLU-kernel linear self-attention of the Sana diffusion
 * transformer.  The operation is defined on "Sana: the autoencoder does more of
 * the work than the linear attention", section "What LiteLA actually computes"
 * (ReLU feature map on q and k, V padded with a row of ones so that one state
 * carries numerator and normaliser, cast to fp32, then divide by the normaliser
 * plus eps), and on "How Linear Attention Improves Efficiency in DiT for
 * High-Resolution Images", sections "Mathematical Foundation" and
 * "Implementation Details".  For every batch b and head h, with phi = ReLU:
 *
 *     S[j][c] = sum_n phi(k[b,n,h,j]) * v[b,n,h,c]    (c < D)
 *     S[j][D] = sum_n phi(k[b,n,h,j])
 *     out[b,i,h,c] = (sum_j phi(q[b,i,h,j]) S[j][c]) / (sum_j phi(q[b,i,h,j]) S[j][D] + eps)
 *
 * The block-causal variant is the video form ("block causal linear attention",
 * evermx.com SANA page, section "Model Family"; cumulative statistics per
 * temporal block, "How Linear Attention ..." page, section "Video Generation
 * and Constant-Memory KV Cache"): tokens are cut into contiguous blocks of
 * block_len tokens (the last block may be shorter) and a query in block beta
 * uses the state summed over the keys of blocks 0..beta.
 *
 * Conventions shared by every entry point below
 * ---------------------------------------------
 * Layout     q, k, v and out are contiguous row-major [B][N][H][D] arrays
 *            (sana_linattn_fwd_strided takes views with free batch and token
 *            strides).
 *            q and k are taken before the feature map: the library applies
 *            ReLU itself (ReLU is idempotent, so already-activated inputs give
 *            the same result).
 * Dtypes     q, k and v share in_dtype; out has its own out_dtype; each is
 *            fp32, bf16 or fp16.  All accumulation is fp32, as the Sana page
 *            ("What LiteLA actually computes") requires because fp16
 *            activations overflow.  A bf16 or fp16 out is the fp32 result
 *            rounded to nearest-even (outputs lie within the range of V, so an
 *            fp16 out cannot overflow).  D is 32 (the Sana head dim, on the matrix
 *            cores; fp32 inputs as three-term bf16 splits with the products
 *            below 2^-24 dropped), 16 or 64 (the same kernels on 32-feature
 *            groups of the token row) for every entry point.
 * Memory     Every pointer is device memory on the current HIP device, owned
 *            by the caller.  The library allocates nothing, keeps nothing
 *            after return, and never synchronises: work is enqueued on
 *            `stream` (0 = the null stream) and the call returns at once.
 *            Scratch space is the caller's `workspace`, sized by
 *            sana_linattn_workspace_bytes(); its contents on entry do not
 *            matter.  Two calls that run concurrently must not share a
 *            workspace.  There is no global mutable state; calls are
 *            re-entrant and thread-safe.  A call enqueues kernel launches
 *            only (no memset, copy or event), so it can be recorded into a
 *            HIP graph by stream capture; replays read the recorded
 *            buffers' current contents.
 * Errors     Every argument is checked before anything is enqueued; on a
 *            failed check nothing is enqueued and a sana_status_t code is
 *            returned.  The library never aborts or prints.  A launch failure
 *            reported by hipGetLastError() maps to SANA_ERR_HIP.
 * Empty      B, H or N equal to 0 is a valid empty problem: SANA_OK, nothing
 *            enqueued, no pointer dereferenced.
 * Results    For fixed arguments and tuning the results are bitwise
 *            repeatable (fixed-order reductions, no atomics).
 */
#ifndef SANA_LINATTN_H
#define SANA_LINATTN_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SANA_LINATTN_ABI_VERSION 1

/* Symbols of this header are the only ones the shared library exports. */
#if defined(__GNUC__) || defined(__clang__)
#define SANA_API __attribute__((visibility("default")))
#else
#define SANA_API
#endif

typedef enum {
    SANA_DT_F32 = 0,   /* IEEE float32 */
    SANA_DT_BF16 = 1,  /* bfloat16 (upper half of a float32) */
    SANA_DT_F16 = 2    /* IEEE binary16 */
} sana_dtype_t;

typedef enum {
    SANA_OK = 0,
    SANA_ERR_INVALID_ARG = 1,  /* null pointer, negative size, bad dtype code,
                                  eps non-finite or < 0, block_len < 1, unknown stage bit */
    SANA_ERR_UNSUPPORTED = 2,  /* D not 16, 32 or 64, or sizes
                                  beyond what the launch grid covers */
    SANA_ERR_ALIGNMENT = 3,    /* q, k, v, out not 16-byte aligned, workspace not 256-byte aligned */
    SANA_ERR_ALIAS = 4,        /* out or workspace overlaps an input, or each other */
    SANA_ERR_WORKSPACE = 5,    /* workspace_bytes smaller than required */
    SANA_ERR_HIP = 6,          /* a HIP runtime error while enqueueing */
    SANA_ERR_SCRATCH = 7       /* sana_linattn_fwd_noalloc: the problem needs more than
                                  SANA_LINATTN_SCRATCH_BYTES of scratch */
} sana_status_t;

/* Size of the library's static device scratch array used by
 * sana_linattn_fwd_noalloc (one copy per GPU, held until the process ends). */
#define SANA_LINATTN_SCRATCH_BYTES (16u << 20)

/* Stage bits for sana_linattn_fwd_stages(). */
#define SANA_STAGE_STATE 1  /* per-chunk partial states from k, v */
#define SANA_STAGE_MERGE 2  /* fixed-order sum of the partials (and per-block prefix) */
#define SANA_STAGE_APPLY 4  /* out from q and the merged state */
#define SANA_STAGE_ALL   7

/* Returns SANA_LINATTN_ABI_VERSION of the built library. */
SANA_API int sana_linattn_abi_version(void);

/* Static, NUL-terminated description of a status code ("unknown status" for
 * values outside sana_status_t).  Never NULL. */
SANA_API const char* sana_linattn_status_string(int status);

/*
 * Workspace needed by a call with these sizes.  block_len = 0 means the
 * non-causal operator; otherwise it is the block length of the block-causal
 * operator (a block_len >= N needs the same workspace as non-causal).
 * Writes the byte count to *bytes (0 for an empty problem).  The answer
 * depends on the tuning environment variables read by the library
 * (SANA_LINATTN_CHUNK, SANA_LINATTN_APPLY_TILE, SANA_LINATTN_PATH), so query it
 * in the same environment as the call.
 * Errors: INVALID_ARG (bytes NULL, negative sizes, block_len < 0),
 * UNSUPPORTED (D not 16, 32 or 64, sizes too large).
 */
SANA_API int sana_linattn_workspace_bytes(int B, int H, int N, int D, int block_len, size_t* bytes);

/*
 * How a call with these sizes is decomposed (for tests and benchmarks).  Any
 * output pointer may be NULL.
 *   chunk_tokens  tokens per state-reduction chunk
 *   num_chunks    chunks per (batch, head) across all blocks
 *   apply_tokens  tokens per apply work-group
 *   mfma          1 if the matrix-core path is used, 0 for the vector path
 * Errors as for sana_linattn_workspace_bytes (in_dtype must be a valid code).
 */
SANA_API int sana_linattn_plan_info(int in_dtype, int B, int H, int N, int D, int block_len,
                           int* chunk_tokens, int* num_chunks, int* apply_tokens, int* mfma);

/*
 * Non-causal LiteLA forward ("What LiteLA actually computes").
 *   q, k, v    [B][N][H][D] in in_dtype, device, read only.
 *   out        [B][N][H][D] in out_dtype, device, written; must not overlap
 *              q, k, v or the workspace.
 *   eps        added to the normaliser; finite and >= 0 (Sana uses a tiny
 *              positive value; with eps = 0 a row whose normaliser is 0 gives
 *              0/0 = NaN).
 *   workspace  device scratch of at least
 *              sana_linattn_workspace_bytes(B, H, N, D, 0) bytes.
 */
SANA_API int sana_linattn_fwd(const void* q, const void* k, const void* v, void* out,
                     int in_dtype, int out_dtype, int B, int H, int N, int D, float eps,
                     void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * Block-causal LiteLA forward: token i in block beta = i / block_len uses the
 * state of the keys in blocks 0..beta (inclusive prefix; full attention inside
 * the block).  block_len >= 1; block_len >= N equals sana_linattn_fwd.
 * Arguments otherwise as for sana_linattn_fwd; the workspace is
 * sana_linattn_workspace_bytes(B, H, N, D, block_len) bytes.
 */
SANA_API int sana_linattn_blockcausal_fwd(const void* q, const void* k, const void* v, void* out,
                                 int in_dtype, int out_dtype, int B, int H, int N, int D,
                                 int block_len, float eps,
                                 void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * Streaming block-causal forward with a carried state: the tokens of this call
 * continue a longer sequence whose earlier tokens are summarised by state_in,
 * the "constant-memory KV cache" of the video section ("How Linear Attention
 * ...", section "Video Generation and Constant-Memory KV Cache").  Token i in
 * block beta uses state_in plus the state of this call's blocks 0..beta; on
 * return state_out holds state_in plus the state of all of this call's tokens,
 * ready to be passed as state_in of the next call.  A sequence cut at block
 * boundaries (every call but the last covers whole blocks) and processed call
 * by call gives the outputs of one sana_linattn_blockcausal_fwd over it all.
 *   state_in   [B][H][D][D+1] fp32, device, read only; NULL = zero state (the
 *              first call).  Row j holds S[j][0..D-1] (sum of phi(k_j) * v)
 *              and S[j][D] (sum of phi(k_j)).
 *   state_out  [B][H][D][D+1] fp32, device, written; NULL = not wanted.  May be
 *              the same pointer as state_in (updated in place), must not
 *              otherwise overlap any other buffer.
 * Other arguments as for sana_linattn_blockcausal_fwd (block_len >= N makes the
 * call a single block).  With B, H or N = 0 nothing is enqueued and state_out
 * is left as it is.  Both state pointers need 4-byte alignment.
 */
SANA_API int sana_linattn_blockcausal_stream_fwd(const void* q, const void* k, const void* v, void* out,
                                                 int in_dtype, int out_dtype, int B, int H, int N, int D,
                                                 int block_len, float eps, const float* state_in,
                                                 float* state_out, void* workspace, size_t workspace_bytes,
                                                 hipStream_t stream);

/*
 * Forward on strided views: q, k, v and out are [B][N][H][D] views whose heads
 * are D elements apart and whose features are contiguous, but whose batch and
 * token strides are free -- e.g. q, k and v as the three slices of one fused
 * qkv projection output [B][N][3][H][D] (token stride 3*H*D), read in place
 * without a copy.
 *   block_len  0 = non-causal, >= 1 = block-causal.
 *   strides    int64[8], in elements: batch and token stride of q, k, v, out,
 *              in that order; all >= 0 and each a multiple of 16 bytes.  The
 *              rows of out must not overlap each other (error ALIAS); inputs
 *              may (a batch stride of 0 broadcasts).
 * Other arguments as for sana_linattn_fwd; the workspace size does not depend
 * on the strides.  Overlap checks use the byte range each view spans.
 */
SANA_API int sana_linattn_fwd_strided(const void* q, const void* k, const void* v, void* out,
                                      int in_dtype, int out_dtype, int B, int H, int N, int D,
                                      int block_len, float eps, const int64_t* strides,
                                      void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * Forward with the qk_norm prologue.  The Sana page ("What LiteLA actually
 * computes") has every Sana-1.5 and Sprint configuration normalise q and k
 * before the feature map, to keep the linear logits inside fp16 range, and
 * gives no formula; the reading taken here is the RMS normalisation of each
 * head's D features with a per-channel scale:
 *     xhat[b,n,h,j] = gamma[h][j] * x[b,n,h,j] / sqrt(mean_j'(x[b,n,h,j']^2) + norm_eps)
 * for q (gamma_q) and for k (gamma_k), then the operator of sana_linattn_fwd
 * on qhat and khat (v unchanged).
 *   gamma_q, gamma_k  device fp32 [H][D], 4-byte aligned, or NULL for no
 *              normalisation of that side; they may not overlap out or the
 *              workspace (error ALIAS).
 *   norm_eps   finite and > 0 when either gamma is given (error INVALID_ARG).
 *   strides    NULL for contiguous [B][N][H][D] views, else as for
 *              sana_linattn_fwd_strided.
 *   block_len  0 = non-causal, >= 1 = block-causal.
 * The workspace is sized by sana_linattn_workspace_bytes as for every other
 * forward.  In the kernels the query's row scale cancels between numerator
 * and normaliser except against eps, which becomes eps * rms of the row, and
 * |gamma_q| is folded into the state rows; the keys are normalised in fp32
 * and carried as three bf16 terms, like fp32 keys.  With both gammas NULL
 * the result is bitwise that of sana_linattn_fwd_strided.
 */
SANA_API int sana_linattn_fwd_qknorm(const void* q, const void* k, const void* v, void* out,
                                     int in_dtype, int out_dtype, int B, int H, int N, int D,
                                     int block_len, float eps, const float* gamma_q, const float* gamma_k,
                                     float norm_eps, const int64_t* strides, void* workspace,
                                     size_t workspace_bytes, hipStream_t stream);

/*
 * The same forward split into its three kernels, for per-kernel timing: a call
 * runs the stages whose bits are set in `stages`, in the order state, merge,
 * apply.  Calling it three times with SANA_STAGE_STATE, SANA_STAGE_MERGE and
 * SANA_STAGE_APPLY on one stream and one workspace produces the same bytes as
 * one call with SANA_STAGE_ALL.  block_len = 0 selects the non-causal
 * operator.  The merge stage reads what the state stage left in the
 * workspace, and the apply stage what the merge stage left.  All arguments
 * are checked on every call, whatever the stages.
 */
SANA_API int sana_linattn_fwd_stages(const void* q, const void* k, const void* v, void* out,
                            int in_dtype, int out_dtype, int B, int H, int N, int D,
                            int block_len, float eps,
                            void* workspace, size_t workspace_bytes, hipStream_t stream,
                            int stages);

/*
 * Backward: gradients of a scalar loss L with respect to q, k and v, given
 * dout = dL/dout of the forward with the same arguments.  The operator is the
 * forward above (non-causal when block_len is 0, block-causal otherwise); its
 * derivative, with f = ReLU(q), a = ReLU(k), P the state a query's block uses,
 * r = 1/(f.P[:, D] + eps), u = dout r, w = -r (dout . out):
 *   dq_i = [q_i > 0] (P [u_i | w_i])
 *   G^(b) = sum over queries i of block b of f_i [u_i | w_i]^T, and for a key n
 *   of block b, with Ghat = sum of G over blocks >= b (the key enters the state
 *   of every later block):
 *   dk_n = [k_n > 0] (Ghat [v_n | 1]),   dv_n = Ghat[:, :D]^T a_n.
 * The derivative of ReLU at 0 is taken as 0.  The states are rebuilt from k
 * and v (nothing needs to be kept from the forward call).
 *   q, k, v     [B][N][H][D] in in_dtype (fp32, bf16 or fp16), device, read only.
 *   dout        [B][N][H][D] in dout_dtype, device, read only (may alias nothing
 *               written).
 *   dq, dk, dv  [B][N][H][D] in grad_dtype, device, written; must not overlap
 *               each other, an input or the workspace (error ALIAS).
 *   block_len   0 = non-causal, >= 1 = block-causal.
 *   workspace   >= sana_linattn_bwd_workspace_bytes(B, H, N, D, block_len)
 *               bytes, 256-byte aligned (the query covers every combination
 *               of input, dout and gradient types; like the forward's, it
 *               depends on the tuning environment variables, here also
 *               SANA_LINATTN_BWD_TILE).
 * Other conventions as for sana_linattn_fwd (16-byte alignment of the tensors,
 * empty problems, error codes, asynchronous on `stream`, bitwise repeatable).
 */
SANA_API int sana_linattn_bwd_workspace_bytes(int B, int H, int N, int D, int block_len, size_t* bytes);

SANA_API int sana_linattn_bwd(const void* q, const void* k, const void* v, const void* dout, void* dq,
                              void* dk, void* dv, int in_dtype, int dout_dtype, int grad_dtype, int B, int H,
                              int N, int D, int block_len, float eps, void* workspace, size_t workspace_bytes,
                              hipStream_t stream);

/*
 * A training step runs the forward and then the backward over the same q, k,
 * v; the backward above rebuilds the forward's states (one more pass over k
 * and v).  These two entry points hand them over instead:
 *
 * sana_linattn_states_bytes: bytes of the per-block prefix states of a call,
 *   B * H * NB * D * (D + 1) * 4 with NB = ceil(N / block_len) (1 when
 *   block_len is 0 or >= N); 0 for an empty problem.
 *
 * sana_linattn_fwd_save_states: the forward of sana_linattn_fwd (block_len 0)
 *   or sana_linattn_blockcausal_fwd (block_len >= 1), which also writes the
 *   state each block's queries use, S_beta (the sum over the keys of blocks
 *   0..beta, with the ones column), into `states`: device fp32
 *   [B][H][NB][D][D+1], at least sana_linattn_states_bytes bytes, 4-byte
 *   aligned, not overlapping q, k, v, out or the workspace (error ALIAS),
 *   caller-owned.  The output is bitwise that of sana_linattn_fwd /
 *   sana_linattn_blockcausal_fwd.
 *
 * sana_linattn_bwd_from_states: the backward of sana_linattn_bwd with the
 *   states read from `states` (as written by sana_linattn_fwd_save_states for
 *   the same q, k, v, in_dtype, block_len; not checked) instead of rebuilt;
 *   `states` must not overlap dq, dk, dv or the workspace (error ALIAS).  The
 *   gradients are bitwise those of sana_linattn_bwd on the same arguments.
 *   The workspace is sized by sana_linattn_bwd_workspace_bytes.
 */
SANA_API int sana_linattn_states_bytes(int B, int H, int N, int D, int block_len, size_t* bytes);

SANA_API int sana_linattn_fwd_save_states(const void* q, const void* k, const void* v, void* out, int in_dtype,
                                          int out_dtype, int B, int H, int N, int D, int block_len, float eps,
                                          float* states, void* workspace, size_t workspace_bytes,
                                          hipStream_t stream);

SANA_API int sana_linattn_bwd_from_states(const void* q, const void* k, const void* v, const void* dout,
                                          const float* states, void* dq, void* dk, void* dv, int in_dtype,
                                          int dout_dtype, int grad_dtype, int B, int H, int N, int D, int block_len,
                                          float eps, void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * Forward-mode derivative (Jacobian-vector product): the forward's output and
 * its directional derivative along tangents (q_t, k_t, v_t) of the inputs, as
 * forward-mode differentiation through attention needs (the consistency-model
 * distillation on the Sana page, section "Sana-Sprint: two steps, on an arc",
 * differentiates the model this way).  With f = ReLU(q), a = ReLU(k),
 * f_t = [q > 0] q_t, a_t = [k > 0] k_t, S the state of the forward and
 * S_t = sum (a_t [v | 1]^T + a [v_t | 0]^T) (prefix over blocks likewise):
 *   out   = num / (den + eps)  as in the forward,
 *   out_t = (num_t - out den_t) / (den + eps),
 *   num_t = S_t[:, :D]^T f + S[:, :D]^T f_t,  den_t = S_t[:, D] . f + S[:, D] . f_t.
 * The derivative of ReLU at 0 is taken as 0.
 *   q, k, v, q_t, k_t, v_t  [B][N][H][D] in in_dtype, device, read only.
 *   out, out_t   [B][N][H][D] in out_dtype, device, written; must not overlap
 *                each other, an input or the workspace (error ALIAS).
 *   block_len    0 = non-causal, >= 1 = block-causal.
 *   workspace    >= sana_linattn_jvp_workspace_bytes(...) bytes, 256-byte aligned.
 * Other conventions as for sana_linattn_fwd.
 */
SANA_API int sana_linattn_jvp_workspace_bytes(int B, int H, int N, int D, int block_len, size_t* bytes);

SANA_API int sana_linattn_jvp(const void* q, const void* k, const void* v, const void* q_t, const void* k_t,
                              const void* v_t, void* out, void* out_t, int in_dtype, int out_dtype, int B, int H,
                              int N, int D, int block_len, float eps, void* workspace, size_t workspace_bytes,
                              hipStream_t stream);

/*
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the forward
 * of sana_linattn_fwd with the same arguments and results, minus the
 * workspace.  Scratch space is a static device array of the library,
 * SANA_LINATTN_SCRATCH_BYTES per GPU (its address is looked up once per device
 * with hipGetSymbolAddress, on the first call on that device); the call
 * allocates nothing (no hipMalloc, no allocating library routine).
 *   Returns SANA_ERR_SCRATCH, before anything is enqueued, when the problem
 *   needs more scratch than that (sana_linattn_workspace_bytes tells how much it
 *   needs); other errors as for sana_linattn_fwd.
 *   Every call on one GPU uses that GPU's one array: calls that may overlap on
 *   one GPU (different streams or host threads without ordering) race and must
 *   not be made; calls ordered on one stream are fine.  The array keeps the
 *   last call's contents; nothing in it needs to start at zero.
 */
SANA_API int sana_linattn_fwd_noalloc(const void* q, const void* k, const void* v, void* out,
                                      int in_dtype, int out_dtype, int B, int H, int N, int D, float eps,
                                      hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* SANA_LINATTN_H */
