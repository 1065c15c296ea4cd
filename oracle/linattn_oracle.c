/*
 * LiteLA forward oracle: plain fp64 CPU implementation.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the checker for the HIP library; only
 * the tests, the smoke check and the CPU-baseline leg of the benchmark may load
 * it.  It shares no code, header or constant with the HIP path.
 *
 * What it computes (ReLU-kernel linear self-attention, as described on
 * "Sana: the autoencoder does more of the work than the linear attention",
 * section "What LiteLA actually computes", and on "How Linear Attention
 * Improves Efficiency in DiT for High-Resolution Images", sections
 * "Mathematical Foundation" and "Implementation Details"):
 *
 *   for every batch b and head h, with phi(x) = max(x, 0) applied elementwise,
 *     a_n = phi(k[b,n,h,:]),  f_i = phi(q[b,i,h,:])               (vectors in R^D)
 *     S[j][c] = sum_n a_n[j] * v[b,n,h,c]     for c < D             (D x D)
 *     S[j][D] = sum_n a_n[j]                                        (the row of ones
 *               appended to V makes this extra column the normaliser)
 *     num_c = sum_j f_i[j] * S[j][c],   den = sum_j f_i[j] * S[j][D]
 *     out[b,i,h,c] = num_c / (den + eps)                            (eps added to the
 *               denominator only, after the cast to full precision)
 *
 * Block-causal variant (the video form named on the evermx.com SANA page,
 * section "Model Family", and on the "How Linear Attention ..." page, section
 * "Video Generation and Constant-Memory KV Cache", which keeps cumulative
 * statistics per temporal block): the tokens are cut into contiguous blocks of
 * block_len tokens (the last one may be shorter).  Blocks are visited in order;
 * block beta's tokens are first added into S, and then block beta's queries are
 * applied against that S.  So a query in block beta sees every key in blocks
 * 0..beta (bidirectional inside its own block, causal across blocks).
 * block_len <= 0, or >= N, is the non-causal operator.
 *
 * Carried state (the same page, same section: the running statistics act as a
 * constant-memory cache that lets a long video be generated piece by piece):
 * an optional state_in gives S before the first token of this call, so that a
 * sequence cut at block boundaries and processed call by call, each call
 * starting from the previous call's final state, gives the same outputs as one
 * call over the whole sequence.
 *
 * qk_norm (optional; the Sana page, section "What LiteLA actually computes",
 * says every Sana-1.5 and Sprint configuration turns on `qk_norm` to keep the
 * ReLU-linear logits from growing out of fp16 range, without giving a formula):
 * read here as an RMS normalisation of each head's D features of q and of k,
 * with a per-channel scale and a small constant under the root, before phi:
 *     xhat[j] = gamma[h][j] * x[j] / sqrt((sum_j' x[j']^2) / D + norm_eps)
 * separately for q (gamma_q) and k (gamma_k); a NULL gamma leaves that side as
 * it is.  The rest of the operator is unchanged.
 *
 * Arithmetic: every input element is decoded exactly to double (bf16 bits are
 * the upper half of an IEEE float32; fp16 is IEEE binary16), and all sums run
 * sequentially in token order in double precision.  No blocking or reordering
 * beyond that.
 *
 * Layout: q, k, v and out are contiguous [B][N][H][D].
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

enum { ORACLE_F32 = 0, ORACLE_BF16 = 1, ORACLE_F16 = 2 };

/* IEEE 754 binary16 from its bits: 1 sign bit, 5 exponent bits (bias 15), 10
 * fraction bits; exponent 0 holds the subnormals frac * 2^-24, exponent 31
 * infinities and NaNs.  Every binary16 value is exact in double. */
static double half_to_double(uint16_t h) {
    const int sign = h >> 15, e = (h >> 10) & 0x1f, frac = h & 0x3ff;
    double x;
    if (e == 0)
        x = ldexp((double)frac, -24);
    else if (e == 31)
        x = frac ? NAN : INFINITY;
    else
        x = ldexp((double)(frac | 0x400), e - 25);
    return sign ? -x : x;
}

/* Decode element idx of an array of float32, of bfloat16 bit patterns or of
 * binary16 bit patterns. */
static double load_elem(const void* base, int dtype, size_t idx) {
    if (dtype == ORACLE_BF16) {
        uint32_t bits = (uint32_t)((const uint16_t*)base)[idx] << 16;
        float f;
        memcpy(&f, &bits, sizeof f);
        return (double)f;
    }
    if (dtype == ORACLE_F16) return half_to_double(((const uint16_t*)base)[idx]);
    return (double)((const float*)base)[idx];
}

/* The decoding above, exposed so that tests can pin it: out[i] = element i. */
int oracle_decode(const void* src, int dtype, size_t n, double* out) {
    if (dtype != ORACLE_F32 && dtype != ORACLE_BF16 && dtype != ORACLE_F16) return -1;
    for (size_t i = 0; i < n; ++i) out[i] = load_elem(src, dtype, i);
    return 0;
}

static double relu(double x) { return x > 0.0 ? x : 0.0; }

/* Decodes row `row` (D elements) into x and, when gamma (the [H][D] scales of
 * head h) is given, RMS-normalises it: x[j] = gamma[h][j] * x[j] / rms, with
 * rms = sqrt(mean of x^2 over the row + norm_eps).  Then applies phi. */
static void load_phi_row(const void* src, int dtype, size_t row, int D, const double* gamma, int h,
                         double norm_eps, double* x) {
    for (int j = 0; j < D; ++j) x[j] = load_elem(src, dtype, row + j);
    if (gamma) {
        double ss = 0.0;
        for (int j = 0; j < D; ++j) ss += x[j] * x[j];
        const double rms = sqrt(ss / D + norm_eps);
        for (int j = 0; j < D; ++j) x[j] = gamma[(size_t)h * D + j] * x[j] / rms;
    }
    for (int j = 0; j < D; ++j) x[j] = relu(x[j]);
}

int oracle_abi_version(void) { return 1; }

/*
 * out      : [B][N][H][D] doubles (written).
 * states   : optional, [B][H][NB][D][D+1] doubles: S after each block has been
 *            added (inclusive prefix); NB = number of blocks (1 if non-causal).
 * state_in : optional, [B][H][D][D+1] doubles: S before the first token
 *            (NULL = zero).
 * nthreads <= 0 leaves the OpenMP default.
 * Returns 0 on success, -1 on bad arguments.
 */
int oracle_linattn_fwd_qknorm(const void* q, const void* k, const void* v, int in_dtype,
                              int B, int H, int N, int D, int block_len, double eps,
                              const double* gamma_q, const double* gamma_k, double norm_eps,
                              double* out, double* states, const double* state_in, int nthreads);

int oracle_linattn_fwd(const void* q, const void* k, const void* v, int in_dtype,
                       int B, int H, int N, int D, int block_len, double eps,
                       double* out, double* states, const double* state_in, int nthreads) {
    return oracle_linattn_fwd_qknorm(q, k, v, in_dtype, B, H, N, D, block_len, eps, NULL, NULL, 0.0, out,
                                     states, state_in, nthreads);
}

/*
 * The same with the optional qk_norm prologue (see the file header):
 * gamma_q, gamma_k: [H][D] doubles or NULL; norm_eps >= 0.
 */
int oracle_linattn_fwd_qknorm(const void* q, const void* k, const void* v, int in_dtype,
                              int B, int H, int N, int D, int block_len, double eps,
                              const double* gamma_q, const double* gamma_k, double norm_eps,
                              double* out, double* states, const double* state_in, int nthreads) {
    if (B < 0 || H < 0 || N < 0 || D < 1 || !(norm_eps >= 0.0)) return -1;
    if (in_dtype != ORACLE_F32 && in_dtype != ORACLE_BF16 && in_dtype != ORACLE_F16) return -1;
    if (B == 0 || H == 0 || N == 0) return 0;
    if (!q || !k || !v || !out) return -1;
    const int L = (block_len <= 0 || block_len >= N) ? N : block_len;
    const int NB = (N + L - 1) / L;
    const int W = D + 1; /* width of a state row: D value columns + normaliser */

#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif

    int failed = 0;
#pragma omp parallel
    {
        double* S = (double*)malloc(sizeof(double) * (size_t)D * W);
        double* a = (double*)malloc(sizeof(double) * (size_t)D);
        double* f = (double*)malloc(sizeof(double) * (size_t)D);
        if (!S || !a || !f) {
#pragma omp atomic write
            failed = 1;
        } else {
#pragma omp for schedule(dynamic, 1)
            for (long bh = 0; bh < (long)B * H; ++bh) {
                const int b = (int)(bh / H), h = (int)(bh % H);
                if (state_in)
                    memcpy(S, state_in + (size_t)bh * D * W, sizeof(double) * (size_t)D * W);
                else
                    memset(S, 0, sizeof(double) * (size_t)D * W);
                for (int beta = 0; beta < NB; ++beta) {
                    const int n0 = beta * L;
                    const int n1 = (n0 + L < N) ? n0 + L : N;
                    /* add this block's keys and values into the state */
                    for (int n = n0; n < n1; ++n) {
                        const size_t row = (((size_t)b * N + n) * H + h) * (size_t)D;
                        load_phi_row(k, in_dtype, row, D, gamma_k, h, norm_eps, a);
                        for (int j = 0; j < D; ++j) {
                            for (int c = 0; c < D; ++c)
                                S[j * W + c] += a[j] * load_elem(v, in_dtype, row + c);
                            S[j * W + D] += a[j];
                        }
                    }
                    if (states) {
                        double* dst = states + (((size_t)b * H + h) * NB + beta) * (size_t)D * W;
                        memcpy(dst, S, sizeof(double) * (size_t)D * W);
                    }
                    /* apply the state to this block's queries */
                    for (int i = n0; i < n1; ++i) {
                        const size_t row = (((size_t)b * N + i) * H + h) * (size_t)D;
                        load_phi_row(q, in_dtype, row, D, gamma_q, h, norm_eps, f);
                        double den = 0.0;
                        for (int j = 0; j < D; ++j) den += f[j] * S[j * W + D];
                        for (int c = 0; c < D; ++c) {
                            double num = 0.0;
                            for (int j = 0; j < D; ++j) num += f[j] * S[j * W + c];
                            out[row + c] = num / (den + eps);
                        }
                    }
                }
            }
        }
        free(S);
        free(a);
        free(f);
    }
    return failed ? -1 : 0;
}

/*
 * Backward of the same operator (test infrastructure, like the forward).
 *
 * Given dout = dL/dout, with f_i = phi(q_i), a_n = phi(k_n) and P = the state a
 * query's block uses (the whole-sequence state when non-causal):
 *   r_i   = 1 / (den_i + eps),  out_i = num_i * r_i
 *   u_i   = dL/dnum_i = dout_i * r_i                                  (D)
 *   w_i   = dL/dden_i = -r_i * (dout_i . out_i)                       (scalar)
 *   dq_ij = [q_ij > 0] * (sum_c P[j][c] u_ic + P[j][D] w_i)
 *   G^(beta)[j][c] = sum over queries i of block beta of f_ij [u_i | w_i]_c
 *                    (dL/dP of the state block beta uses, D x (D+1))
 * A key of block beta enters the state of every block >= beta, so it sees the
 * suffix sum Ghat^(beta) = sum_{beta' >= beta} G^(beta'):
 *   dk_nj = [k_nj > 0] * (sum_c Ghat[j][c] v_nc + Ghat[j][D])
 *   dv_nc = sum_j a_nj Ghat[j][c]
 * The derivative of ReLU at 0 is taken as 0.  dout has its own dtype code.
 * dq, dk, dv: [B][N][H][D] doubles (written).  Returns 0, or -1 on bad
 * arguments.
 */
int oracle_linattn_bwd(const void* q, const void* k, const void* v, const void* dout, int in_dtype,
                       int dout_dtype, int B, int H, int N, int D, int block_len, double eps,
                       double* dq, double* dk, double* dv, int nthreads) {
    if (B < 0 || H < 0 || N < 0 || D < 1) return -1;
    if (in_dtype != ORACLE_F32 && in_dtype != ORACLE_BF16 && in_dtype != ORACLE_F16) return -1;
    if (dout_dtype != ORACLE_F32 && dout_dtype != ORACLE_BF16 && dout_dtype != ORACLE_F16) return -1;
    if (B == 0 || H == 0 || N == 0) return 0;
    if (!q || !k || !v || !dout || !dq || !dk || !dv) return -1;
    const int L = (block_len <= 0 || block_len >= N) ? N : block_len;
    const int NB = (N + L - 1) / L;
    const int W = D + 1;

#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif

    int failed = 0;
#pragma omp parallel
    {
        /* per (b, h): prefix states P[NB][D][W], gradient states G[NB][D][W] */
        double* P = (double*)malloc(sizeof(double) * (size_t)NB * D * W);
        double* G = (double*)malloc(sizeof(double) * (size_t)NB * D * W);
        double* f = (double*)malloc(sizeof(double) * (size_t)D);
        double* uw = (double*)malloc(sizeof(double) * (size_t)W);
        double* x = (double*)malloc(sizeof(double) * (size_t)D);
        if (!P || !G || !f || !uw || !x) {
#pragma omp atomic write
            failed = 1;
        } else {
#pragma omp for schedule(dynamic, 1)
            for (long bh = 0; bh < (long)B * H; ++bh) {
                const int b = (int)(bh / H), h = (int)(bh % H);
                /* forward states, inclusive prefix over blocks */
                memset(P, 0, sizeof(double) * (size_t)NB * D * W);
                for (int beta = 0; beta < NB; ++beta) {
                    double* Pb = P + (size_t)beta * D * W;
                    if (beta > 0) memcpy(Pb, Pb - (size_t)D * W, sizeof(double) * (size_t)D * W);
                    const int n1 = (beta * L + L < N) ? beta * L + L : N;
                    for (int n = beta * L; n < n1; ++n) {
                        const size_t row = (((size_t)b * N + n) * H + h) * (size_t)D;
                        for (int j = 0; j < D; ++j) f[j] = relu(load_elem(k, in_dtype, row + j));
                        for (int j = 0; j < D; ++j) {
                            for (int c = 0; c < D; ++c) Pb[j * W + c] += f[j] * load_elem(v, in_dtype, row + c);
                            Pb[j * W + D] += f[j];
                        }
                    }
                }
                /* queries: dq and the per-block gradient states */
                memset(G, 0, sizeof(double) * (size_t)NB * D * W);
                for (int i = 0; i < N; ++i) {
                    const int beta = i / L;
                    const double* Pb = P + (size_t)beta * D * W;
                    double* Gb = G + (size_t)beta * D * W;
                    const size_t row = (((size_t)b * N + i) * H + h) * (size_t)D;
                    for (int j = 0; j < D; ++j) f[j] = relu(load_elem(q, in_dtype, row + j));
                    double den = 0.0;
                    for (int j = 0; j < D; ++j) den += f[j] * Pb[j * W + D];
                    const double r = 1.0 / (den + eps);
                    double g_dot_out = 0.0;
                    for (int c = 0; c < D; ++c) {
                        double num = 0.0;
                        for (int j = 0; j < D; ++j) num += f[j] * Pb[j * W + c];
                        const double g = load_elem(dout, dout_dtype, row + c);
                        uw[c] = g * r;
                        g_dot_out += g * (num * r);
                    }
                    uw[D] = -r * g_dot_out;
                    for (int j = 0; j < D; ++j) {
                        double s = 0.0;
                        for (int c = 0; c < W; ++c) s += Pb[j * W + c] * uw[c];
                        dq[row + j] = load_elem(q, in_dtype, row + j) > 0.0 ? s : 0.0;
                        for (int c = 0; c < W; ++c) Gb[j * W + c] += f[j] * uw[c];
                    }
                }
                /* suffix sums over blocks */
                for (int beta = NB - 2; beta >= 0; --beta)
                    for (int e = 0; e < D * W; ++e) G[(size_t)beta * D * W + e] += G[(size_t)(beta + 1) * D * W + e];
                /* keys: dk, dv */
                for (int n = 0; n < N; ++n) {
                    const double* Gb = G + (size_t)(n / L) * D * W;
                    const size_t row = (((size_t)b * N + n) * H + h) * (size_t)D;
                    for (int c = 0; c < D; ++c) x[c] = load_elem(v, in_dtype, row + c);
                    for (int j = 0; j < D; ++j) f[j] = relu(load_elem(k, in_dtype, row + j));
                    for (int j = 0; j < D; ++j) {
                        double s = Gb[j * W + D];
                        for (int c = 0; c < D; ++c) s += Gb[j * W + c] * x[c];
                        dk[row + j] = load_elem(k, in_dtype, row + j) > 0.0 ? s : 0.0;
                    }
                    for (int c = 0; c < D; ++c) {
                        double s = 0.0;
                        for (int j = 0; j < D; ++j) s += f[j] * Gb[j * W + c];
                        dv[row + c] = s;
                    }
                }
            }
        }
        free(P);
        free(G);
        free(f);
        free(uw);
        free(x);
    }
    return failed ? -1 : 0;
}

/*
 * Forward-mode derivative (JVP) of the same operator (test infrastructure).
 *
 * Given tangents qt, kt, vt of q, k, v, with f = phi(q), a_n = phi(k_n) and
 * the derivative of ReLU taken as [x > 0]:
 *   ft   = [q > 0] * qt,   at_n = [k_n > 0] * kt_n
 *   S    = sum_n a_n [v_n | 1]^T                 (prefix over blocks when causal)
 *   St   = sum_n (at_n [v_n | 1]^T + a_n [vt_n | 0]^T)
 *   num  = S[:, :D]^T f,   den  = S[:, D] . f
 *   numt = St[:, :D]^T f + S[:, :D]^T ft,   dent = St[:, D] . f + S[:, D] . ft
 *   out  = num / (den + eps),   outt = (numt - out * dent) / (den + eps)
 * Tangents have the inputs' dtype code.  out and outt: [B][N][H][D] doubles.
 * Returns 0, or -1 on bad arguments.
 */
int oracle_linattn_jvp(const void* q, const void* k, const void* v, const void* qt, const void* kt,
                       const void* vt, int in_dtype, int B, int H, int N, int D, int block_len, double eps,
                       double* out, double* outt, int nthreads) {
    if (B < 0 || H < 0 || N < 0 || D < 1) return -1;
    if (in_dtype != ORACLE_F32 && in_dtype != ORACLE_BF16 && in_dtype != ORACLE_F16) return -1;
    if (B == 0 || H == 0 || N == 0) return 0;
    if (!q || !k || !v || !qt || !kt || !vt || !out || !outt) return -1;
    const int L = (block_len <= 0 || block_len >= N) ? N : block_len;
    const int NB = (N + L - 1) / L;
    const int W = D + 1;

#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif

    int failed = 0;
#pragma omp parallel
    {
        double* S = (double*)malloc(sizeof(double) * (size_t)D * W);
        double* St = (double*)malloc(sizeof(double) * (size_t)D * W);
        double* a = (double*)malloc(sizeof(double) * (size_t)D);
        double* at = (double*)malloc(sizeof(double) * (size_t)D);
        double* x = (double*)malloc(sizeof(double) * (size_t)D);
        double* xt = (double*)malloc(sizeof(double) * (size_t)D);
        if (!S || !St || !a || !at || !x || !xt) {
#pragma omp atomic write
            failed = 1;
        } else {
#pragma omp for schedule(dynamic, 1)
            for (long bh = 0; bh < (long)B * H; ++bh) {
                const int b = (int)(bh / H), h = (int)(bh % H);
                memset(S, 0, sizeof(double) * (size_t)D * W);
                memset(St, 0, sizeof(double) * (size_t)D * W);
                for (int beta = 0; beta < NB; ++beta) {
                    const int n0 = beta * L;
                    const int n1 = (n0 + L < N) ? n0 + L : N;
                    for (int n = n0; n < n1; ++n) {   /* this block's keys into S and St */
                        const size_t row = (((size_t)b * N + n) * H + h) * (size_t)D;
                        for (int j = 0; j < D; ++j) {
                            const double kk = load_elem(k, in_dtype, row + j);
                            a[j] = relu(kk);
                            at[j] = kk > 0.0 ? load_elem(kt, in_dtype, row + j) : 0.0;
                            x[j] = load_elem(v, in_dtype, row + j);
                            xt[j] = load_elem(vt, in_dtype, row + j);
                        }
                        for (int j = 0; j < D; ++j) {
                            for (int c = 0; c < D; ++c) {
                                S[j * W + c] += a[j] * x[c];
                                St[j * W + c] += at[j] * x[c] + a[j] * xt[c];
                            }
                            S[j * W + D] += a[j];
                            St[j * W + D] += at[j];
                        }
                    }
                    for (int i = n0; i < n1; ++i) {   /* this block's queries */
                        const size_t row = (((size_t)b * N + i) * H + h) * (size_t)D;
                        for (int j = 0; j < D; ++j) {
                            const double qq = load_elem(q, in_dtype, row + j);
                            a[j] = relu(qq);                                           /* f */
                            at[j] = qq > 0.0 ? load_elem(qt, in_dtype, row + j) : 0.0;   /* ft */
                        }
                        double den = 0.0, dent = 0.0;
                        for (int j = 0; j < D; ++j) {
                            den += a[j] * S[j * W + D];
                            dent += St[j * W + D] * a[j] + S[j * W + D] * at[j];
                        }
                        for (int c = 0; c < D; ++c) {
                            double num = 0.0, numt = 0.0;
                            for (int j = 0; j < D; ++j) {
                                num += a[j] * S[j * W + c];
                                numt += St[j * W + c] * a[j] + S[j * W + c] * at[j];
                            }
                            const double o = num / (den + eps);
                            out[row + c] = o;
                            outt[row + c] = (numt - o * dent) / (den + eps);
                        }
                    }
                }
            }
        }
        free(S);
        free(St);
        free(a);
        free(at);
        free(x);
        free(xt);
    }
    return failed ? -1 : 0;
}

/* Number of threads an OpenMP parallel region would use right now. */
int oracle_max_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
