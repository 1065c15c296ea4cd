"""Shared helpers of the GPU tests: upload seeded inputs, run the C ABI, compare
with the fp64 oracle.  Not collected by pytest (no test_ prefix)."""
import functools

import numpy as np
import torch

import oracle
import workloads

# Parity bar: max-abs error <= 2e-3 * max|V| and relative L2 <= 1e-4, element by
# element against the fp64 oracle on the same inputs.
MAX_ABS_FRAC = 2e-3
REL_L2 = 1e-4


def to_device(a: np.ndarray) -> torch.Tensor:
    t = torch.from_numpy(a.view(np.int16)).view(torch.bfloat16) if a.dtype == np.uint16 else torch.from_numpy(a)
    return t.to("cuda:0")


def decode(a: np.ndarray) -> np.ndarray:
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    return a.astype(np.float64)


@functools.lru_cache(maxsize=8)
def inputs_and_oracle(w: workloads.Workload):
    q, k, v = workloads.make_inputs(w)
    want = oracle.linattn_fwd(q, k, v, block_len=w.block_len, eps=w.eps)
    return (q, k, v), want


def bf16_round(x64: np.ndarray) -> np.ndarray:
    return torch.from_numpy(x64).float().to(torch.bfloat16).double().numpy()


def f16_round(x64: np.ndarray) -> np.ndarray:
    return x64.astype(np.float32).astype(np.float16).astype(np.float64)


# Absolute error allowance of the fp32 pipeline for a 16-bit gradient or
# tangent, relative to its scale (max |exact|).  An empirical allowance, not a
# bound: a rigorous one would also carry the fp32 error of the states P and
# Ghat, sums over up to N tokens, into the final contractions.  The largest
# error seen was 1.8e-6 of the scale (an exact dq of ~1e-14 computed as
# 3.1e-6 with scale 1.7, head dim 16, 16384 tokens x 140 heads); 64 u
# (u = 2^-24, 3.8e-6) leaves twice that.  It matters only where the terms
# cancel (an exact value of ~0); the rel-L2 <= 1e-4 and max-abs bars hold
# for every gradient regardless.
FP32_PIPELINE_FRAC = 64 * 2.0 ** -24


def compare(got: np.ndarray, want: np.ndarray, v: np.ndarray, out_bf16, label: str = ""):
    """Returns (max_abs, rel_l2) and asserts the parity bar.  out_bf16: False
    (fp32 out), True (bf16 out) or "f16" (fp16 out)."""
    out_f16 = isinstance(out_bf16, str) and out_bf16 == "f16"
    out_bf16 = out_bf16 is True
    vmax = np.max(np.abs(decode(v))) if v.size else 1.0
    ref = bf16_round(want) if out_bf16 else f16_round(want) if out_f16 else want
    diff = got - ref
    max_abs = float(np.max(np.abs(diff))) if diff.size else 0.0
    norm = float(np.linalg.norm(ref))
    rel = float(np.linalg.norm(diff) / norm) if norm > 0 else float(np.linalg.norm(diff))
    assert np.all(np.isfinite(got)), label
    assert max_abs <= MAX_ABS_FRAC * vmax, f"{label}: max abs {max_abs:.3e} > {MAX_ABS_FRAC}*{vmax:.3e}"
    assert rel <= REL_L2, f"{label}: rel L2 {rel:.3e} > {REL_L2}"
    if out_bf16 or out_f16:
        # A 16-bit result is the fp32 result rounded once: within one ulp of
        # the exact value (bf16: 8 significant bits; fp16: 11, with subnormal
        # spacing 2^-24), plus the fp32 pipeline's own absolute error, which
        # dominates for outputs near zero (cancellation in the weighted sum).
        e = np.floor(np.log2(np.maximum(np.abs(want), 1e-300)))
        ulp = np.exp2(e - 7) if out_bf16 else np.exp2(np.maximum(e, -14) - 10)
        fp32_abs = 1e-6 * vmax
        bad = np.abs(got - want) > ulp + fp32_abs
        name = "bf16" if out_bf16 else "fp16"
        assert not np.any(bad), f"{label}: {int(bad.sum())} values beyond one {name} ulp + {fp32_abs:.1e}"
    return max_abs, rel


def run_hip(q_np, k_np, v_np, *, block_len=0, eps=1e-15, out_dtype=torch.float32, stream=None):
    import diffusion_transformer_relu_amd as sana
    q, k, v = to_device(q_np), to_device(k_np), to_device(v_np)
    out = sana.linattn_fwd(q, k, v, eps=eps, out_dtype=out_dtype, block_len=block_len or None, stream=stream)
    torch.cuda.synchronize()
    return out.float().cpu().double().numpy()
