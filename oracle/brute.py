"""Quadratic-form LiteLA in numpy, fp64: the pin for the linear-form oracle.

TEST INFRASTRUCTURE ONLY.

The pages derive the linear form from the quadratic one by re-bracketing
(phi(Q) phi(K)^T) V as phi(Q) (phi(K)^T V) ("Sana: the autoencoder does more of
the work than the linear attention", section "What LiteLA actually computes";
"How Linear Attention Improves Efficiency in DiT for High-Resolution Images",
section "Mathematical Foundation", which writes the operator as
phi(Q) phi(K)^T V divided row-wise by phi(Q) phi(K)^T 1).  This module
evaluates that quadratic form directly: it builds the N x N weight matrix
W[i, n] = phi(q_i) . phi(k_n), masks it for the block-causal variant (query
block >= key block), and returns (W V) / (W 1 + eps).  O(N^2): tiny inputs only.
"""
from __future__ import annotations

import numpy as np


def decode(x: np.ndarray) -> np.ndarray:
    """float32 or float16 array (numpy's own widening), or uint16 array of
    bfloat16 bits -> float64."""
    if x.dtype == np.uint16:
        return (x.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    return x.astype(np.float64)


def block_ids(N: int, block_len: int | None) -> np.ndarray:
    if not block_len or block_len <= 0:
        return np.zeros(N, dtype=np.int64)
    return np.arange(N) // block_len


def weights(q_bh: np.ndarray, k_bh: np.ndarray, block_len: int | None = None) -> np.ndarray:
    """W[i, n] for one (b, h): phi(q_i).phi(k_n), zero where key block > query block."""
    W = np.maximum(q_bh, 0.0) @ np.maximum(k_bh, 0.0).T
    blk = block_ids(q_bh.shape[0], block_len)
    return W * (blk[:, None] >= blk[None, :])


def brute_fwd(q, k, v, *, block_len: int | None = None, eps: float = 1e-15) -> np.ndarray:
    """[B, N, H, D] inputs (float32 or bf16 bits) -> float64 [B, N, H, D]."""
    q, k, v = decode(q), decode(k), decode(v)
    B, N, H, D = q.shape
    out = np.empty((B, N, H, D), dtype=np.float64)
    for b in range(B):
        for h in range(H):
            W = weights(q[b, :, h, :], k[b, :, h, :], block_len)
            out[b, :, h, :] = (W @ v[b, :, h, :]) / (W.sum(axis=1) + eps)[:, None]
    return out
