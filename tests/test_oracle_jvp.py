"""Pins for the oracle's forward-mode derivative (CPU only): torch.func.jvp in
float64 of the masked quadratic form (forward-mode differentiation of a
different formula by a library), the adjoint identity with the backward
<g, J t> = <J^T g, t>, and the primal output equal to the forward's."""
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


def quadratic(Q, K, V, block_len, eps):
    N = Q.shape[1]
    W = torch.einsum("bihd,bnhd->bhin", torch.relu(Q), torch.relu(K))
    if block_len and block_len < N:
        blk = torch.arange(N) // block_len
        W = W * (blk[:, None] >= blk[None, :]).double()
    den = W.sum(-1).permute(0, 2, 1)[..., None]
    return torch.einsum("bhin,bnhd->bihd", W, V) / (den + eps)


CASES = [((1, 37, 2, 8), "f32", 0), ((2, 64, 3, 32), "bf16", 0), ((1, 100, 2, 32), "bf16", 16),
         ((2, 33, 1, 16), "f16", 7), ((1, 50, 2, 32), "f32", 1)]


@pytest.mark.parametrize("shape,kind,L", CASES, ids=[f"{c[0]}-{c[1]}-L{c[2]}" for c in CASES])
def test_jvp_matches_torch_func_jvp_of_quadratic_form(shape, kind, L):
    q, k, v, qt, kt, vt = (rand(s, shape, kind) for s in range(30, 36))
    out, outt = oracle.linattn_jvp(q, k, v, qt, kt, vt, block_len=L)
    prim = [torch.tensor(decode(x), dtype=torch.float64) for x in (q, k, v)]
    tang = [torch.tensor(decode(x), dtype=torch.float64) for x in (qt, kt, vt)]
    o, ot = torch.func.jvp(lambda Q, K, V: quadratic(Q, K, V, L, 1e-15), tuple(prim), tuple(tang))
    np.testing.assert_allclose(out, o.numpy(), rtol=1e-12, atol=1e-14)
    assert np.max(np.abs(outt - ot.numpy())) <= 1e-12 * np.max(np.abs(ot.numpy()))


@pytest.mark.parametrize("L", [0, 8])
def test_jvp_is_the_adjoint_of_the_backward(L):
    shape = (2, 48, 3, 32)
    q, k, v, qt, kt, vt, g = (rand(s, shape) for s in range(40, 47))
    _, outt = oracle.linattn_jvp(q, k, v, qt, kt, vt, block_len=L)
    dq, dk, dv = oracle.linattn_bwd(q, k, v, g, block_len=L)
    lhs = float(np.sum(g.astype(np.float64) * outt))
    rhs = float(np.sum(dq * qt) + np.sum(dk * kt) + np.sum(dv * vt))
    assert abs(lhs - rhs) <= 1e-11 * max(abs(lhs), 1.0)


def test_jvp_primal_equals_forward_and_special_directions():
    shape = (1, 64, 2, 32)
    q, k, v, qt, kt, vt = (rand(s, shape) for s in range(50, 56))
    out, _ = oracle.linattn_jvp(q, k, v, qt, kt, vt, block_len=16)
    assert np.array_equal(out, oracle.linattn_fwd(q, k, v, block_len=16))
    z = np.zeros(shape, np.float32)
    # along v only the output moves linearly: tangent = forward with V := vt (no eps effect on the weights)
    _, t_v = oracle.linattn_jvp(q, k, v, z, z, vt)
    np.testing.assert_allclose(t_v, oracle.linattn_fwd(q, k, vt), rtol=1e-12, atol=1e-14)
    # scaling q or k (degree-zero homogeneity): tangent along q itself vanishes up to eps
    _, t_q = oracle.linattn_jvp(q, k, v, q, z, z)
    _, t_k = oracle.linattn_jvp(q, k, v, z, k, z)
    assert np.max(np.abs(t_q)) < 1e-12 and np.max(np.abs(t_k)) < 1e-12
    _, t0 = oracle.linattn_jvp(q, k, v, z, z, z)
    assert np.all(t0 == 0)
