"""Pins for the oracle's qk_norm prologue (CPU only).

The Sana page ("What LiteLA actually computes") only says that Sana-1.5 and
Sprint configurations switch `qk_norm` on to keep the ReLU-linear logits in
range; the reading taken is an RMS normalisation of each head's D features of q
and of k, xhat = gamma * x / sqrt(mean(x^2) + norm_eps), before phi.  Pinned by
what that reading fixes without re-typing it: rows of constant magnitude whose
RMS is known by hand (a 3-4-5 triple puts norm_eps under the root, the mean
over D rather than a sum), the reduction to plain LiteLA on unit rows, and the
invariance of each (token, head) row to a positive rescale (which a norm over
the wrong axis, over tokens or over heads, breaks)."""
import numpy as np
import pytest

import oracle
from oracle.brute import brute_fwd


def signs(rng, shape):
    return np.where(rng.random(shape) < 0.5, -1.0, 1.0)


def rel(a, b):
    return np.linalg.norm((a - b).ravel()) / max(np.linalg.norm(b.ravel()), 1e-300)


@pytest.mark.parametrize("block_len", [0, 5])
def test_constant_magnitude_rows_normalise_to_gamma_times_sign(block_len):
    """Every q and k row has entries +-4: its mean square is 16, so with
    norm_eps = 9 the RMS is 5 and each element becomes gamma * sign * 4/5.  With
    eps = 1 the output's scale depends on that 4/5 (a norm with eps outside the
    root, a sum instead of a mean or a missing gamma gives another value)."""
    rng = np.random.default_rng(3)
    B, N, H, D = 2, 12, 3, 8
    sq, sk = signs(rng, (B, N, H, D)), signs(rng, (B, N, H, D))
    q = (4.0 * sq).astype(np.float32)
    k = (4.0 * sk).astype(np.float32)
    v = rng.standard_normal((B, N, H, D)).astype(np.float32)
    gq = rng.uniform(-2, 2, (H, D))
    gk = rng.uniform(-2, 2, (H, D))
    got = oracle.linattn_fwd(q, k, v, block_len=block_len, eps=1.0, gamma_q=gq, gamma_k=gk, norm_eps=9.0)
    qhat = gq[None, None] * sq * 0.8
    khat = gk[None, None] * sk * 0.8
    want = brute_fwd(qhat, khat, v, block_len=block_len, eps=1.0)
    assert rel(got, want) < 1e-13


def test_gamma_one_on_unit_rows_is_plain_litela():
    rng = np.random.default_rng(4)
    B, N, H, D = 1, 40, 2, 32
    q = signs(rng, (B, N, H, D)).astype(np.float32)
    k = signs(rng, (B, N, H, D)).astype(np.float32)
    v = rng.standard_normal((B, N, H, D)).astype(np.float32)
    ones = np.ones((H, D))
    plain = oracle.linattn_fwd(q, k, v)
    normed = oracle.linattn_fwd(q, k, v, gamma_q=ones, gamma_k=ones, norm_eps=0.0)
    assert np.array_equal(plain, normed)            # rms = 1 exactly: xhat = x
    only_q = oracle.linattn_fwd(q, k, v, gamma_q=ones)
    assert np.array_equal(plain, only_q)


def test_per_channel_gamma_reweights_the_features():
    """On unit rows (norm_eps 0) qk_norm with per-channel gamma is plain LiteLA
    on gamma * x: a positive gamma_q reweights the rows of the state; it is not a
    no-op, unlike a per-token scale."""
    rng = np.random.default_rng(5)
    B, N, H, D = 1, 30, 2, 16
    q, k = signs(rng, (B, N, H, D)), signs(rng, (B, N, H, D))
    v = rng.standard_normal((B, N, H, D))
    gq = rng.uniform(0.1, 3.0, (H, D))
    gk = rng.uniform(-3.0, 3.0, (H, D))
    got = oracle.linattn_fwd(q.astype(np.float32), k.astype(np.float32), v.astype(np.float32),
                             gamma_q=gq, gamma_k=gk)
    want = brute_fwd(gq[None, None] * q, gk[None, None] * k, v.astype(np.float32))
    assert rel(got, want) < 1e-13
    plain_gk = oracle.linattn_fwd(q.astype(np.float32), k.astype(np.float32), v.astype(np.float32), gamma_k=gk)
    assert rel(got, plain_gk) > 1e-3


@pytest.mark.parametrize("side", ["q", "k"])
def test_each_token_head_row_is_scale_free(side):
    """With norm_eps = 0 a positive rescale of one (token, head) row of q or k
    leaves the output unchanged, whatever the scale of the other rows and heads
    (powers of two keep the rescaled inputs exact)."""
    rng = np.random.default_rng(6)
    B, N, H, D = 2, 50, 3, 32
    q, k, v = (rng.standard_normal((B, N, H, D)).astype(np.float32) for _ in range(3))
    g = {"gamma_q": rng.uniform(-1, 2, (H, D)), "gamma_k": rng.uniform(-1, 2, (H, D))}
    base = oracle.linattn_fwd(q, k, v, block_len=7, **g)
    scale = np.exp2(rng.integers(-6, 7, (B, N, H, 1))).astype(np.float32)
    if side == "q":
        got = oracle.linattn_fwd(q * scale, k, v, block_len=7, **g)
    else:
        got = oracle.linattn_fwd(q, k * scale, v, block_len=7, **g)
    assert rel(got, base) < 1e-13
    # without the norm a per-token rescale of k reweights the keys
    plain = oracle.linattn_fwd(q, k, v, block_len=7)
    plain_scaled = oracle.linattn_fwd(q, k * scale, v, block_len=7)
    if side == "k":
        assert rel(plain_scaled, plain) > 1e-3


def test_norm_eps_and_bf16_inputs():
    """norm_eps damps rows whose mean square is small: with every k row scaled
    far below sqrt(norm_eps) the keys' weights shrink towards gamma * x /
    sqrt(norm_eps), i.e. back to plain LiteLA on gamma * k (up to the overall
    scale, which phi's homogeneity removes)."""
    rng = np.random.default_rng(7)
    B, N, H, D = 1, 64, 2, 32
    q, k, v = (rng.standard_normal((B, N, H, D)) for _ in range(3))
    k = k * 1e-6
    gk = rng.uniform(0.5, 1.5, (H, D))
    got = oracle.linattn_fwd(q.astype(np.float32), k.astype(np.float32), v.astype(np.float32),
                             gamma_k=gk, norm_eps=1.0)
    want = oracle.linattn_fwd(q.astype(np.float32), (gk[None, None] * k).astype(np.float32), v.astype(np.float32))
    assert rel(got, want) < 1e-6
