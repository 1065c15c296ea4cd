"""Seeded synthetic inputs for the LiteLA forward: the one module that both the
oracle-side tests and the HIP-path tests/bench draw their inputs from.

It holds no part of the attention arithmetic.  It only defines the workload
shapes and draws q/k/v, so that the oracle (under ``oracle/``) and the HIP
library see the very same bytes.

Shapes follow the Sana models described on "Sana: the autoencoder does more of
the work than the linear attention" (summary table and section "Two levers, and
only one of them is the famous one"): head dim 32, hidden 1152 -> 36 heads,
hidden 2240 -> 70 heads, N = (resolution / 32)^2 latent tokens, B = 2 for a
conditional/unconditional pair.  The block-causal case (16 frame-blocks of
32x32 tokens) follows the video variant named on the evermx.com SANA page
(section "Model Family") and on "How Linear Attention Improves Efficiency in
DiT for High-Resolution Images" (section "Video Generation and Constant-Memory
KV Cache").  Real activations need trained weights; these synthetic tensors of
the same shape and a unit-normal value distribution stand in for them.

Recipe: ``numpy.random.default_rng([seed, t])`` with t = 0, 1, 2 for q, k, v
draws ``standard_normal`` in float32, an optional scale is applied, and bf16
inputs are then rounded to bfloat16 with round-to-nearest-even (the rounding of
``torch.Tensor.to(torch.bfloat16)`` for finite values); fp16 inputs are rounded
to IEEE binary16 the same way (numpy's cast).  Layout is contiguous
[B, N, H, D].
"""
from __future__ import annotations

from dataclasses import dataclass, replace

import numpy as np

DT_F32 = 0   # matches the C-ABI dtype code for float32
DT_BF16 = 1  # matches the C-ABI dtype code for bfloat16
DT_F16 = 2   # matches the C-ABI dtype code for IEEE binary16


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    N: int
    H: int
    D: int
    in_dtype: int          # DT_F32, DT_BF16 or DT_F16
    seed: int
    block_len: int = 0     # 0 = non-causal; otherwise frame-block length in tokens
    v_scale: float = 1.0
    negative_k_heads: tuple = ()   # heads whose K is forced to -|K| (all of phi(K) = 0)
    negative_q_rows: tuple = ()    # (b, n, h) rows whose q is forced to -|q| (phi(q_i) = 0)
    eps: float = 1e-15
    note: str = ""

    @property
    def token_heads(self) -> int:
        return self.B * self.N * self.H

    def algorithmic_bytes(self, out_bytes: int) -> int:
        """Bytes the method must move: read q, k, v once, write out once."""
        s_in = 4 if self.in_dtype == DT_F32 else 2
        return self.token_heads * self.D * (3 * s_in + out_bytes)

    def algorithmic_flops(self) -> int:
        """4*D*(D+1) flops per token-head: D*(D+1) multiply-adds to build the
        state plus D*(D+1) to apply it (the LiteLA term 2*N*d*(d_h+1) MACs of
        the FLOP model in section "Two levers, and only one of them is the
        famous one"), counting a multiply-add as 2 flops."""
        return self.token_heads * 4 * self.D * (self.D + 1)


# The five workloads; index 3 is the headline bandwidth case.
TINY = Workload("tiny_oracle_B1_N256_H2_D32_f32", 1, 256, 2, 32, DT_F32, seed=0,
                negative_k_heads=(1,), note="head 1 has all K < 0 (eps path)")
S600M_1024 = Workload("sana600m_1024px_B2_N1024_H36_D32_bf16", 2, 1024, 36, 32, DT_BF16, seed=1)
S1600M_1024 = Workload("sana1600m_1024px_B2_N1024_H70_D32_bf16", 2, 1024, 70, 32, DT_BF16, seed=2)
S1600M_2048 = Workload("sana1600m_2048px_B2_N4096_H70_D32_bf16", 2, 4096, 70, 32, DT_BF16, seed=3)
HEADLINE = Workload("sana1600m_4096px_B1_N16384_H70_D32_bf16", 1, 16384, 70, 32, DT_BF16, seed=4,
                    v_scale=0.5)
BLOCK_CAUSAL = Workload("blockcausal_16x1024_B1_N16384_H70_D32_bf16", 1, 16384, 70, 32, DT_BF16,
                        seed=5, block_len=1024)

ALL = (TINY, S600M_1024, S1600M_1024, S1600M_2048, HEADLINE, BLOCK_CAUSAL)
BY_NAME = {w.name: w for w in ALL}


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (nearest, ties to even); returns uint16 bits.
    Valid for finite inputs, which is all this module produces."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = u >> np.uint32(16)     # r = ((u >> 16) & 1) + 0x7FFF + u, then >> 16
    r &= np.uint32(1)
    r += np.uint32(0x7FFF)
    r += u
    r >>= np.uint32(16)
    return r.astype(np.uint16)


def make_inputs(w: Workload):
    """Return (q, k, v) as numpy arrays of shape [B, N, H, D]: uint16 bf16 bits
    when w.in_dtype is DT_BF16, float16 (numpy's round-to-nearest-even cast)
    when it is DT_F16, float32 otherwise."""
    shape = (w.B, w.N, w.H, w.D)
    out = []
    for t in range(3):
        rng = np.random.default_rng([w.seed, t])
        x = rng.standard_normal(size=shape, dtype=np.float32)
        if t == 2 and w.v_scale != 1.0:
            x *= np.float32(w.v_scale)
        if t == 1:
            for h in w.negative_k_heads:
                x[:, :, h, :] = -np.abs(x[:, :, h, :])
        if t == 0:
            for (b, n, h) in w.negative_q_rows:
                x[b, n, h, :] = -np.abs(x[b, n, h, :])
        if w.in_dtype == DT_BF16:
            x = f32_to_bf16_bits(x)
        elif w.in_dtype == DT_F16:
            x = x.astype(np.float16)
        out.append(x)
    return tuple(out)


def with_shape(w: Workload, **kw) -> Workload:
    """A copy of workload w with some fields changed (e.g. a smaller N)."""
    name = kw.pop("name", None) or (w.name + "_" + "_".join(f"{k}{v}" for k, v in kw.items()))
    return replace(w, name=name, **kw)


def make_dout(w: Workload, dtype: int | None = None):
    """Seeded upstream gradient dL/dout for backward tests, [B, N, H, D]:
    ``default_rng([seed, 3])`` standard normal, in dtype (default w.in_dtype)
    with the same rounding as make_inputs."""
    dtype = w.in_dtype if dtype is None else dtype
    x = np.random.default_rng([w.seed, 3]).standard_normal(size=(w.B, w.N, w.H, w.D), dtype=np.float32)
    if dtype == DT_BF16:
        return f32_to_bf16_bits(x)
    if dtype == DT_F16:
        return x.astype(np.float16)
    return x


def make_tangents(w: Workload):
    """Seeded tangents (q_t, k_t, v_t) for forward-mode derivative tests, in the
    inputs' dtype: ``default_rng([seed, t])`` standard normal, t = 4, 5, 6."""
    out = []
    for t in (4, 5, 6):
        x = np.random.default_rng([w.seed, t]).standard_normal(size=(w.B, w.N, w.H, w.D), dtype=np.float32)
        if w.in_dtype == DT_BF16:
            x = f32_to_bf16_bits(x)
        elif w.in_dtype == DT_F16:
            x = x.astype(np.float16)
        out.append(x)
    return tuple(out)


def make_gammas(w: Workload, negative_every: int = 0):
    """Seeded per-channel scales (gamma_q, gamma_k) of the qk_norm prologue,
    float32 [H, D]: ``default_rng([seed, t])`` with t = 7, 8, drawn as
    1 + 0.25 * standard normal (learned RMS-norm scales start at 1).  With
    negative_every = m > 0 every channel j with j % m == 0 is negated, so the
    sign of a scale matters to phi."""
    out = []
    for t in (7, 8):
        g = 1.0 + 0.25 * np.random.default_rng([w.seed, t]).standard_normal(size=(w.H, w.D), dtype=np.float32)
        g = g.astype(np.float32)
        if negative_every > 0:
            g[:, ::negative_every] *= np.float32(-1.0)
        out.append(g)
    return tuple(out)
