"""Pins for the oracle's backward (CPU only).

The gradients are pinned to torch autograd of the quadratic form in float64
(a library differentiation of a different formula), to identities that follow
from the pages' statements (degree-zero homogeneity in q and in k, [Sana]
"What LiteLA actually computes"; the shift rule in V), and to the eps path.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from oracle.brute import decode


def rand(seed, shape, kind="f32", scale=1.0):
    x = np.random.default_rng(seed).standard_normal(shape).astype(np.float32) * np.float32(scale)
    if kind == "bf16":
        return workloads.f32_to_bf16_bits(x)
    if kind == "f16":
        return x.astype(np.float16)
    return x


def autograd_quadratic(q, k, v, g, block_len=0, eps=1e-15):
    """dL/d(q, k, v) of L = sum(out * g), out from the quadratic form, float64 autograd."""
    Q, K, V = (torch.tensor(decode(x), dtype=torch.float64, requires_grad=True) for x in (q, k, v))
    G = torch.tensor(decode(g), dtype=torch.float64)
    N = Q.shape[1]
    W = torch.einsum("bihd,bnhd->bhin", torch.relu(Q), torch.relu(K))
    if block_len and block_len < N:
        blk = torch.arange(N) // block_len
        W = W * (blk[:, None] >= blk[None, :]).double()
    den = W.sum(-1).permute(0, 2, 1)[..., None]
    out = torch.einsum("bhin,bnhd->bihd", W, V) / (den + eps)
    (out * G).sum().backward()
    return Q.grad.numpy(), K.grad.numpy(), V.grad.numpy()


CASES = [((1, 37, 2, 8), "f32", "f32", 0), ((2, 64, 3, 32), "bf16", "bf16", 0),
         ((1, 100, 2, 32), "bf16", "f32", 16), ((2, 33, 1, 16), "f16", "f16", 7),
         ((1, 50, 2, 32), "f16", "bf16", 1), ((1, 40, 2, 8), "f32", "f32", 40)]


@pytest.mark.parametrize("shape,kind,gkind,L", CASES, ids=[f"{c[0]}-{c[1]}-{c[2]}-L{c[3]}" for c in CASES])
def test_bwd_matches_autograd_of_quadratic_form(shape, kind, gkind, L):
    q, k, v = (rand(s, shape, kind) for s in (1, 2, 3))
    g = rand(4, shape, gkind)
    got = oracle.linattn_bwd(q, k, v, g, block_len=L)
    want = autograd_quadratic(q, k, v, g, L)
    for name, a, b in zip(("dq", "dk", "dv"), got, want):
        scale = np.max(np.abs(b))
        assert np.max(np.abs(a - b)) <= 1e-12 * scale, name


@pytest.mark.parametrize("L", [0, 8])
def test_bwd_euler_identities_of_homogeneity(L):
    """out(gamma q_i) = out(q_i) and out(gamma k) = out(k) up to eps, so
    q_i . dq_i = 0 for every token and sum_n k_n . dk_n = 0 per (b, h)."""
    shape = (2, 64, 3, 32)
    q, k, v, g = (rand(s, shape) for s in (5, 6, 7, 8))
    dq, dk, _ = oracle.linattn_bwd(q, k, v, g, block_len=L)
    qd, kd = decode(q), decode(k)
    per_token = np.sum(qd * dq, axis=-1)
    assert np.max(np.abs(per_token)) <= 1e-12 * np.max(np.abs(qd)) * np.max(np.abs(dq)) * 32
    per_head = np.sum(kd * dk, axis=(1, 3))
    assert np.max(np.abs(per_head)) <= 1e-11 * np.max(np.abs(kd)) * np.max(np.abs(dk)) * 64 * 32
    assert np.max(np.abs(dq)) > 1e-3 and np.max(np.abs(dk)) > 1e-3   # the identities are not vacuous


@pytest.mark.parametrize("L", [0, 5])
def test_bwd_value_shift_rule(L):
    """out(V + c) = out(V) + c * den / (den + eps), so sum_n dv[n, c] = sum_i g[i, c] * den_i / (den_i + eps)
    = sum_i g[i, c] whenever every den_i > 0."""
    shape = (1, 48, 2, 32)
    q, k, v, g = (rand(s, shape) for s in (9, 10, 11, 12))
    _, _, dv = oracle.linattn_bwd(q, k, v, g, block_len=L)
    np.testing.assert_allclose(dv.sum(axis=1), g.astype(np.float64).sum(axis=1), rtol=1e-11, atol=1e-11)


def test_bwd_eps_path_gives_zero_gradients():
    w = workloads.Workload("bwd_eps", 1, 64, 2, 32, workloads.DT_F32, seed=13, negative_k_heads=(1,),
                           negative_q_rows=((0, 5, 0),))
    q, k, v = workloads.make_inputs(w)
    g = rand(14, q.shape)
    dq, dk, dv = oracle.linattn_bwd(q, k, v, g)
    assert np.all(dq[:, :, 1] == 0) and np.all(dk[:, :, 1] == 0) and np.all(dv[:, :, 1] == 0)
    assert np.all(dq[0, 5, 0] == 0)
    assert np.any(dq[:, :, 0] != 0)


def test_bwd_block_len_at_least_n_is_non_causal_and_linear_in_dout():
    shape = (1, 40, 2, 16)
    q, k, v = (rand(s, shape) for s in (15, 16, 17))
    # dyadic upstream gradients, so that g1 + g2 is exact in float32
    g1, g2 = (np.round(rand(s, shape) * 64) / np.float32(64) for s in (18, 19))
    a = oracle.linattn_bwd(q, k, v, g1)
    b = oracle.linattn_bwd(q, k, v, g1, block_len=40)
    c = oracle.linattn_bwd(q, k, v, g1, block_len=1000)
    for x, y, z in zip(a, b, c):
        assert np.array_equal(x, y) and np.array_equal(x, z)
    s = oracle.linattn_bwd(q, k, v, (g1 + g2).astype(np.float32))
    b2 = oracle.linattn_bwd(q, k, v, g2)
    for x, y, z in zip(s, a, b2):
        np.testing.assert_allclose(x, y + z, rtol=1e-12, atol=1e-14)


def test_bwd_first_block_queries_match_a_call_on_the_first_block():
    """Queries of block 0 see only block 0's keys, so their dq equals that of a
    non-causal call on block 0 alone."""
    shape = (1, 48, 2, 16)
    q, k, v, g = (rand(s, shape) for s in (20, 21, 22, 23))
    dq, _, _ = oracle.linattn_bwd(q, k, v, g, block_len=16)
    dq0, _, _ = oracle.linattn_bwd(q[:, :16], k[:, :16], v[:, :16], g[:, :16])
    np.testing.assert_allclose(dq[:, :16], dq0, rtol=1e-13, atol=1e-15)


def test_bwd_empty_inputs():
    z = np.zeros((1, 0, 2, 32), np.float32)
    dq, dk, dv = oracle.linattn_bwd(z, z, z, z)
    assert dq.shape == dk.shape == dv.shape == (1, 0, 2, 32)
