"""Pins for the fp64 oracle (CPU only).

The pages print no numeric example of the operator, so the oracle is pinned by
things other than itself: a hand-worked example, exact rational arithmetic,
the quadratic form it is re-bracketed from, closed forms that reduce to a
textbook routine (group means), and the invariants the pages state (rank bound,
degree-zero homogeneity) or that follow from the definition (permutation
equivariance, convex hull, the eps path).  Each is chosen so that a plausible
slip in the oracle (a dropped normaliser, a transposed state, an exclusive
instead of inclusive block prefix, a wrong bf16 decode) fails at least one.
"""
import json
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
import workloads
from oracle.brute import brute_fwd, decode, weights
from oracle.exact import exact_fwd

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def rand_inputs(seed, B, N, H, D, bf16=True, scale=1.0):
    """bf16=True: bfloat16 bits; False: float32; "f16": float16."""
    rng = np.random.default_rng(seed)
    xs = [(rng.standard_normal((B, N, H, D)).astype(np.float32) * np.float32(scale)) for _ in range(3)]
    if bf16 == "f16":
        xs = [x.astype(np.float16) for x in xs]
    elif bf16:
        xs = [workloads.f32_to_bf16_bits(x) for x in xs]
    return xs


def rel_err(a, b):
    return np.linalg.norm((a - b).ravel()) / max(np.linalg.norm(b.ravel()), 1e-300)


# ---------------------------------------------------------------- hand-worked example
def test_hand_worked_golden():
    g = json.load(open(os.path.join(GOLDEN, "hand_worked_N3_D2.json")))
    q = np.array(g["q"], dtype=np.float32)[None, :, None, :]
    k = np.array(g["k"], dtype=np.float32)[None, :, None, :]
    v = np.array(g["v"], dtype=np.float32)[None, :, None, :]
    for case in g["cases"]:
        eps = float(Fraction(case["eps"])) if "/" in case["eps"] else float(case["eps"])
        out = oracle.linattn_fwd(q, k, v, block_len=case["block_len"], eps=eps)[0, :, 0, :]
        want = np.array([[float(Fraction(x)) for x in row] for row in case["out"]])
        nz = want != 0
        assert np.all(out[~nz] == 0.0), case
        np.testing.assert_allclose(out[nz], want[nz], rtol=1e-14, atol=0)


# ---------------------------------------------------------------- bf16 decode
def test_bf16_decode_known_patterns():
    # D=1, N=1, q=k=1.0: out = v * 1 / (1 + 0) = v exactly, so out exposes the decode.
    bits = np.array([0x3F80, 0x4049, 0xC2F7, 0x0001, 0x7F7F, 0x8000], dtype=np.uint16)
    want = [1.0, 3.140625, -123.5, 2.0 ** -133, 3.3895313892515355e38, -0.0]
    one = np.full((1, 1, 1, 1), 0x3F80, dtype=np.uint16)
    for b, w in zip(bits, want):
        v = np.full((1, 1, 1, 1), b, dtype=np.uint16)
        out = oracle.linattn_fwd(one, one, v, eps=0.0)
        assert out[0, 0, 0, 0] == w, (hex(b), out[0, 0, 0, 0], w)


def test_bf16_and_f32_inputs_agree_with_torch_decode():
    q, k, v = rand_inputs(11, 2, 64, 3, 32, bf16=True)
    as_f32 = [torch.from_numpy(x.astype(np.int16)).view(torch.bfloat16).float().numpy() for x in (q, k, v)]
    a = oracle.linattn_fwd(q, k, v)
    b = oracle.linattn_fwd(*as_f32)
    assert np.array_equal(a, b)


# ---------------------------------------------------------------- fp16 decode
def test_f16_decode_known_patterns():
    # IEEE 754 binary16: sign, 5 exponent bits (bias 15), 10 fraction bits.
    cases = {0x3C00: 1.0, 0x3555: 0.333251953125, 0xC000: -2.0, 0x7BFF: 65504.0,
             0x0400: 2.0 ** -14, 0x0001: 2.0 ** -24, 0x03FF: 1023 * 2.0 ** -24,
             0x8000: -0.0, 0x7C00: np.inf, 0xFC00: -np.inf}
    bits = np.array(list(cases), dtype=np.uint16).view(np.float16)
    got = oracle.decode(bits)
    for b, g in zip(cases, got):
        assert g == cases[b] and np.signbit(g) == np.signbit(cases[b]), (hex(b), g)
    assert np.isnan(oracle.decode(np.array([0x7E00, 0xFD01], dtype=np.uint16).view(np.float16))).all()


def test_f16_decode_every_pattern_matches_numpy():
    allbits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16).view(np.float16)
    got, want = oracle.decode(allbits), allbits.astype(np.float64)
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], want[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(want[~nan]))


def test_f16_inputs_agree_with_their_f32_widening():
    q, k, v = rand_inputs(12, 2, 64, 3, 32, bf16="f16")
    a = oracle.linattn_fwd(q, k, v)
    b = oracle.linattn_fwd(*[x.astype(np.float32) for x in (q, k, v)])
    assert np.array_equal(a, b)


# ---------------------------------------------------------------- exact and quadratic forms
@pytest.mark.parametrize("block_len,dt", [(0, True), (4, True), (1, True), (7, True), (0, "f16"), (3, "f16")])
def test_matches_exact_rational(block_len, dt):
    q, k, v = rand_inputs(3, 1, 7, 2, 4, bf16=dt)
    ex = exact_fwd(q, k, v, block_len=block_len)
    want = np.array([[[[float(x) for x in c] for c in h] for h in n] for n in ex])
    got = oracle.linattn_fwd(q, k, v, block_len=block_len)
    np.testing.assert_allclose(got, want, rtol=1e-13, atol=1e-15)


@pytest.mark.parametrize("shape,bf16", [((1, 256, 2, 32), False), ((2, 300, 3, 32), True),
                                        ((1, 129, 1, 8), True), ((3, 33, 5, 16), False),
                                        ((2, 200, 3, 32), "f16")])
def test_linear_form_equals_quadratic_form(shape, bf16):
    q, k, v = rand_inputs(5, *shape, bf16=bf16)
    got = oracle.linattn_fwd(q, k, v)
    want = brute_fwd(q, k, v)
    assert rel_err(got, want) <= 1e-12
    assert np.max(np.abs(got - want)) <= 1e-12 * np.max(np.abs(decode(v)))


def test_tiny_workload_against_quadratic_form_and_eps_path():
    w = workloads.TINY
    q, k, v = workloads.make_inputs(w)
    got = oracle.linattn_fwd(q, k, v, eps=w.eps)
    assert rel_err(got, brute_fwd(q, k, v, eps=w.eps)) <= 1e-12
    # head 1 has all keys negative: every weight is 0, every output exactly 0
    assert np.all(got[:, :, 1, :] == 0.0)
    assert np.any(got[:, :, 0, :] != 0.0)


def test_negative_query_row_gives_zero():
    w = workloads.with_shape(workloads.TINY, negative_q_rows=((0, 17, 0), (0, 200, 0)), name="negq")
    q, k, v = workloads.make_inputs(w)
    out = oracle.linattn_fwd(q, k, v, eps=w.eps)
    assert np.all(out[0, 17, 0] == 0.0) and np.all(out[0, 200, 0] == 0.0)
    assert np.all(out[0, 18, 0] != 0.0)


def test_quadratic_weights_have_rank_at_most_head_dim():
    # Section "What LiteLA actually computes": the implied map relu(Q) relu(K)^T
    # has rank <= head dim for any N.  Pins the brute-force weights themselves.
    q, k, v = rand_inputs(8, 1, 200, 1, 32, bf16=False)
    W = weights(decode(q)[0, :, 0], decode(k)[0, :, 0])
    assert np.linalg.matrix_rank(W) <= 32
    # a genuine N x N softmax-like map of the same inputs would be full rank
    assert np.linalg.matrix_rank(np.exp(decode(q)[0, :, 0] @ decode(k)[0, :, 0].T / 32)) > 32


# ---------------------------------------------------------------- state and closed forms
def test_state_is_relu_k_transpose_v_with_ones_column():
    q, k, v = rand_inputs(9, 2, 100, 3, 32, bf16=True)
    _, st = oracle.linattn_fwd(q, k, v, return_states=True)
    K = np.maximum(decode(k), 0.0)
    V = decode(v)
    for b in range(2):
        for h in range(3):
            S = st[b, h, 0]
            np.testing.assert_allclose(S[:, :32], K[b, :, h, :].T @ V[b, :, h, :], rtol=1e-12, atol=1e-12)
            # the appended row of ones makes the last column the key sums
            np.testing.assert_allclose(S[:, 32], K[b, :, h, :].sum(axis=0), rtol=1e-13, atol=0)


def test_group_mean_closed_form():
    # One-hot keys and queries: token n belongs to group g(n); query i asks for
    # group g'(i).  The weight is t_i [g(n) == g'(i)], so the output is the plain
    # mean of V over the group (a textbook group-by mean, via np.bincount).
    rng = np.random.default_rng(21)
    N, D, G = 300, 32, 20
    g_k = rng.integers(0, G, N)
    g_q = rng.integers(0, G + 3, N)          # some queries ask for empty groups (>= G)
    k = np.zeros((1, N, 1, D), np.float32)
    k[0, np.arange(N), 0, g_k] = 1.0
    k[0, :, 0, G:] = -rng.random((N, D - G)).astype(np.float32)   # negative: phi = 0
    q = np.full((1, N, 1, D), -1.0, np.float32)
    t = (rng.random(N) * 4 + 0.25).astype(np.float32)
    q[0, np.arange(N), 0, np.minimum(g_q, D - 1)] = t
    v = rng.standard_normal((1, N, 1, D)).astype(np.float32)
    out = oracle.linattn_fwd(q, k, v, eps=1e-15)[0, :, 0, :]
    cnt = np.bincount(g_k, minlength=D)
    for c in range(D):
        sums = np.bincount(g_k, weights=v[0, :, 0, c].astype(np.float64), minlength=D)
        mean = np.divide(sums, cnt, out=np.zeros(D), where=cnt > 0)
        want = mean[np.minimum(g_q, D - 1)]
        np.testing.assert_allclose(out[:, c], want, rtol=1e-12, atol=1e-14)
    assert np.all(out[g_q >= G] == 0.0)


def test_identical_keys_give_value_mean():
    rng = np.random.default_rng(4)
    N, D = 77, 32
    k = np.tile(np.abs(rng.standard_normal(D)).astype(np.float32), (1, N, 1, 1))
    q = rng.standard_normal((1, N, 1, D)).astype(np.float32)
    v = rng.standard_normal((1, N, 1, D)).astype(np.float32)
    out = oracle.linattn_fwd(q, k, v)[0, :, 0, :]
    np.testing.assert_allclose(out, np.broadcast_to(v[0, :, 0, :].astype(np.float64).mean(0), (N, D)),
                               rtol=1e-12, atol=1e-14)


# ---------------------------------------------------------------- invariants
def test_permutation_equivariance():
    q, k, v = rand_inputs(12, 2, 150, 2, 32, bf16=True)
    perm = np.random.default_rng(1).permutation(150)
    a = oracle.linattn_fwd(q, k, v)
    b = oracle.linattn_fwd(q[:, perm], k[:, perm], v[:, perm])
    np.testing.assert_allclose(b, a[:, perm], rtol=1e-12, atol=1e-14)


def test_convex_hull_of_values():
    q, k, v = rand_inputs(13, 1, 120, 2, 32, bf16=False)
    out = oracle.linattn_fwd(q, k, v)
    qd, kd, vd = decode(q), decode(k), decode(v)
    for h in range(2):
        W = weights(qd[0, :, h], kd[0, :, h])
        for i in range(120):
            sel = W[i] > 0
            if not sel.any():
                assert np.all(out[0, i, h] == 0.0)
                continue
            lo = vd[0, sel, h].min(axis=0)
            hi = vd[0, sel, h].max(axis=0)
            assert np.all(out[0, i, h] >= lo - 1e-12) and np.all(out[0, i, h] <= hi + 1e-12)


def test_degree_zero_homogeneity_and_value_linearity():
    q, k, v = rand_inputs(14, 1, 90, 2, 32, bf16=False)
    base = oracle.linattn_fwd(q, k, v)
    # scaling q or k by any gamma > 0 changes nothing (section "What LiteLA
    # actually computes": ReLU-then-normalise has no temperature); powers of two
    # are exact, so only the eps term can differ
    for g in (4.0, 0.125):
        assert np.allclose(oracle.linattn_fwd(q * np.float32(g), k, v), base, rtol=1e-14, atol=0)
        assert np.allclose(oracle.linattn_fwd(q, k * np.float32(g), v), base, rtol=1e-14, atol=0)
    # a non-power-of-two gamma rounds q in float32 (relative 2^-24), nothing more
    scale = np.max(np.abs(base))
    np.testing.assert_allclose(oracle.linattn_fwd(q * np.float32(3.0), k, v), base, rtol=0, atol=1e-6 * scale)
    # linear in V (alpha = -2 is exact in float32), and a constant shift of V
    # passes straight through (v + 7 is rounded in float32: tolerance 2^-24 * 8)
    np.testing.assert_allclose(oracle.linattn_fwd(q, k, v * np.float32(-2.0)), -2.0 * base, rtol=1e-13, atol=1e-15)
    out_shift = oracle.linattn_fwd(q, k, v + np.float32(7.0))
    np.testing.assert_allclose(out_shift, base + 7.0, rtol=0, atol=1e-6)


def test_eps_enters_denominator_only():
    q, k, v = rand_inputs(15, 1, 40, 1, 32, bf16=False)
    qd, kd, vd = decode(q), decode(k), decode(v)
    W = weights(qd[0, :, 0], kd[0, :, 0])
    for eps in (0.5, 10.0):
        want = (W @ vd[0, :, 0]) / (W.sum(1) + eps)[:, None]
        np.testing.assert_allclose(oracle.linattn_fwd(q, k, v, eps=eps)[0, :, 0], want, rtol=1e-12, atol=1e-15)


# ---------------------------------------------------------------- block-causal
@pytest.mark.parametrize("N,L", [(256, 64), (250, 64), (100, 1), (100, 3), (64, 64), (64, 1000)])
def test_block_causal_matches_masked_quadratic_form(N, L):
    q, k, v = rand_inputs(16, 2, N, 2, 32, bf16=True)
    got = oracle.linattn_fwd(q, k, v, block_len=L)
    want = brute_fwd(q, k, v, block_len=L)
    assert rel_err(got, want) <= 1e-12


def test_block_causal_structure():
    N, L = 300, 64                 # 5 blocks, the last one ragged (44 tokens)
    q, k, v = rand_inputs(17, 1, N, 3, 32, bf16=True)
    full = oracle.linattn_fwd(q, k, v)
    bc, st = oracle.linattn_fwd(q, k, v, block_len=L, return_states=True)
    last0 = (N - 1) // L * L
    # the last block sees every key: identical to the non-causal output
    assert np.array_equal(bc[:, last0:], full[:, last0:])
    # block 0 sees only itself: identical to running non-causal on block 0 alone
    assert np.array_equal(bc[:, :L], oracle.linattn_fwd(q[:, :L], k[:, :L], v[:, :L]))
    # block_len >= N is the non-causal operator
    assert np.array_equal(oracle.linattn_fwd(q, k, v, block_len=N), full)
    # inclusive prefix: state after block beta minus state after beta-1 is block beta's own state
    K = np.maximum(decode(k), 0.0)
    V = decode(v)
    for beta in range(st.shape[2]):
        sl = slice(beta * L, min((beta + 1) * L, N))
        prev = st[0, :, beta - 1] if beta else 0.0
        inc = st[0, :, beta] - prev
        for h in range(3):
            np.testing.assert_allclose(inc[h, :, :32], K[0, sl, h].T @ V[0, sl, h], rtol=1e-9, atol=1e-9)
            np.testing.assert_allclose(inc[h, :, 32], K[0, sl, h].sum(0), rtol=1e-9, atol=1e-9)


def test_block_len_one_is_token_causal_cumsum():
    # block_len = 1: token i sees keys 0..i, i.e. causal linear attention, here
    # with the state built as a running cumulative sum of outer products.
    N, D = 60, 32
    q, k, v = rand_inputs(18, 1, N, 1, D, bf16=False)
    got = oracle.linattn_fwd(q, k, v, block_len=1)[0, :, 0]
    A = np.maximum(decode(k)[0, :, 0], 0.0)
    Vp = np.concatenate([decode(v)[0, :, 0], np.ones((N, 1))], axis=1)
    S = np.cumsum(A[:, :, None] * Vp[:, None, :], axis=0)       # [N, D, D+1]
    F = np.maximum(decode(q)[0, :, 0], 0.0)
    r = np.einsum("nj,njc->nc", F, S)
    np.testing.assert_allclose(got, r[:, :D] / (r[:, D:] + 1e-15), rtol=1e-12, atol=1e-14)


@pytest.mark.parametrize("L,cuts", [(64, (0, 128, 192, 300)), (1, (0, 5, 6, 40)), (100, (0, 300))])
def test_carried_state_chunks_equal_one_shot(L, cuts):
    # A sequence cut at block boundaries and processed call by call, each call
    # starting from the previous call's final state, equals one call over it all
    # (the summation order is the same, so the fp64 results are identical).
    N = 300
    q, k, v = rand_inputs(19, 2, N, 3, 32, bf16=True)
    full = oracle.linattn_fwd(q, k, v, block_len=L)
    st = None
    for a, b in zip(cuts, list(cuts[1:]) + [N]):
        if a == b:
            continue
        part, states = oracle.linattn_fwd(q[:, a:b], k[:, a:b], v[:, a:b], block_len=L,
                                          return_states=True, state_in=st)
        assert np.array_equal(part, full[:, a:b])
        st = states[:, :, -1]
    # and the final carried state is relu(K)^T [V | 1] over the whole sequence
    K = np.maximum(decode(k), 0.0)
    V = decode(v)
    for b in range(2):
        for h in range(3):
            np.testing.assert_allclose(st[b, h, :, :32], K[b, :, h].T @ V[b, :, h], rtol=1e-12, atol=1e-12)
            np.testing.assert_allclose(st[b, h, :, 32], K[b, :, h].sum(0), rtol=1e-13, atol=0)


def test_empty_inputs():
    z = np.zeros((1, 0, 2, 32), np.float32)
    assert oracle.linattn_fwd(z, z, z).shape == (1, 0, 2, 32)


def test_workload_generator_matches_torch_rounding():
    rng = np.random.default_rng(0)
    x = (rng.standard_normal(100000) * 10).astype(np.float32)
    ours = workloads.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)


def test_f16_workload_generator_matches_torch_rounding():
    w = workloads.Workload("f16_gen", 1, 64, 3, 32, workloads.DT_F16, seed=9, v_scale=0.5)
    q, k, v = workloads.make_inputs(w)
    assert q.dtype == np.float16
    for t, x in enumerate((q, k, v)):
        f = np.random.default_rng([9, t]).standard_normal(size=(1, 64, 3, 32), dtype=np.float32)
        if t == 2:
            f *= np.float32(0.5)
        assert np.array_equal(x, torch.from_numpy(f).to(torch.float16).numpy())
