"""Exact rational LiteLA (quadratic form) for tiny inputs.

TEST INFRASTRUCTURE ONLY.  Pure-Python loops over ``fractions.Fraction``: every
float32/bf16 input is converted exactly, every product and sum is exact, and the
single division per output is exact.  The result is the true value of the
operator defined in section "What LiteLA actually computes" of "Sana: the
autoencoder does more of the work than the linear attention" (weights
phi(q_i).phi(k_n) with phi = ReLU, output = weighted sum of values over the sum
of weights plus eps), with the block-causal mask "key block <= query block".
Use only for N*N*D up to a few hundred thousand.
"""
from __future__ import annotations

from fractions import Fraction

import numpy as np

from .brute import decode


def exact_fwd(q, k, v, *, block_len: int | None = None, eps=Fraction(1, 10**15)):
    """Returns a nested list out[b][i][h][c] of Fractions."""
    qd, kd, vd = decode(q), decode(k), decode(v)
    B, N, H, D = qd.shape
    eps = Fraction(eps)
    L = block_len if (block_len and block_len > 0) else N
    F = np.vectorize(Fraction, otypes=[object])
    qf, kf, vf = F(qd), F(kd), F(vd)
    zero = Fraction(0)
    out = [[[[zero] * D for _ in range(H)] for _ in range(N)] for _ in range(B)]
    for b in range(B):
        for h in range(H):
            a = [[x if x > 0 else zero for x in kf[b, n, h, :]] for n in range(N)]
            for i in range(N):
                f = [x if x > 0 else zero for x in qf[b, i, h, :]]
                num = [zero] * D
                den = zero
                for n in range(N):
                    if n // L > i // L:
                        continue
                    w = sum((f[j] * a[n][j] for j in range(D)), zero)
                    if w == 0:
                        continue
                    den += w
                    for c in range(D):
                        num[c] += w * vf[b, n, h, c]
                out[b][i][h] = [num[c] / (den + eps) for c in range(D)]
    return out
