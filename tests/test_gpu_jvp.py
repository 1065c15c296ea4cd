"""GPU parity of the forward-mode derivative (out and its tangent) through the
C ABI against the fp64 oracle, element by element, on the same seeded inputs."""
import functools

import numpy as np
import pytest
import torch

import oracle
import workloads
from hip_helpers import FP32_PIPELINE_FRAC, bf16_round, compare, f16_round, to_device

pytestmark = pytest.mark.gpu

# Tangent bar: rel-L2 <= 1e-4 and max-abs <= 2e-3 * max|exact tangent| (fp32
# out); a 16-bit tangent against the rounded exact one, within one ulp plus
# the fp32 pipeline's error (FP32_PIPELINE_FRAC of the scale).  The primal
# output has the forward's bar.
REL_L2 = 1e-4
MAX_ABS_FRAC = 2e-3


@pytest.fixture(autouse=True)
def _announce(request):
    print(f"\n[gpu] {request.node.name}", flush=True)


@functools.lru_cache(maxsize=4)
def case(w):
    x = workloads.make_inputs(w) + workloads.make_tangents(w)
    return x, oracle.linattn_jvp(*x, block_len=w.block_len, eps=w.eps)


def check_tangent(got, want, out_t, label):
    ref = want if out_t == torch.float32 else (bf16_round(want) if out_t == torch.bfloat16 else f16_round(want))
    scale = float(np.max(np.abs(want)))
    diff = got - ref
    rel = float(np.linalg.norm(diff) / np.linalg.norm(ref))
    assert np.all(np.isfinite(got)), label
    assert rel <= REL_L2, f"{label}: tangent rel L2 {rel:.3e}"
    if out_t == torch.float32:
        assert float(np.max(np.abs(diff))) <= MAX_ABS_FRAC * scale, f"{label}: tangent max abs"
    else:
        e = np.floor(np.log2(np.maximum(np.abs(want), 1e-300)))
        ulp = np.exp2(e - 7) if out_t == torch.bfloat16 else np.exp2(np.maximum(e, -14) - 10)
        assert not np.any(np.abs(got - want) > ulp + FP32_PIPELINE_FRAC * scale), f"{label}: tangent beyond one ulp"


def run(x, w, out_t):
    import diffusion_transformer_relu_amd as sana
    o, ot = sana.linattn_jvp(*(to_device(a) for a in x), eps=w.eps, out_dtype=out_t, block_len=w.block_len or None)
    torch.cuda.synchronize()
    return o.float().cpu().double().numpy(), ot.float().cpu().double().numpy()


FULL = [workloads.S600M_1024, workloads.S1600M_2048, workloads.HEADLINE, workloads.BLOCK_CAUSAL]


@pytest.mark.parametrize("w", FULL, ids=lambda w: w.name)
@pytest.mark.parametrize("out_t", [torch.float32, torch.bfloat16], ids=["f32out", "bf16out"])
def test_jvp_full_size(w, out_t):
    x, (want, want_t) = case(w)
    got, got_t = run(x, w, out_t)
    compare(got, want, x[2], out_t == torch.bfloat16, w.name)
    check_tangent(got_t, want_t, out_t, w.name)


F32_IN = [workloads.with_shape(workloads.HEADLINE, in_dtype=workloads.DT_F32, name="sana1600m_4096px_f32in"),
          workloads.with_shape(workloads.BLOCK_CAUSAL, in_dtype=workloads.DT_F32, name="blockcausal_16x1024_f32in")]


@pytest.mark.parametrize("w", F32_IN, ids=lambda w: w.name)
@pytest.mark.parametrize("out_t", [torch.float32, torch.bfloat16], ids=["f32out", "bf16out"])
def test_jvp_full_size_fp32_inputs(w, out_t):
    """fp32 inputs and tangents: the matrix-core kernels on three-term bf16
    splits of a, v, a_t, v_t, f and f_t."""
    x, (want, want_t) = case(w)
    got, got_t = run(x, w, out_t)
    compare(got, want, x[2], out_t == torch.bfloat16, w.name)
    check_tangent(got_t, want_t, out_t, w.name)


EDGE = [(2, 33, 3, 0, 1), (1, 257, 2, 64, 1), (3, 1000, 5, 100, 2), (1, 300, 2, 1, 0), (1, 4097, 1, 0, 2),
        (1, 1, 1, 0, 1)]


@pytest.mark.parametrize("path", ["mfma", "valu"])
@pytest.mark.parametrize("B,N,H,L,dt", EDGE, ids=[f"B{b}N{n}H{h}L{l}dt{d}" for b, n, h, l, d in EDGE])
def test_jvp_edge_shapes(monkeypatch, path, B, N, H, L, dt):
    if path == "valu":
        monkeypatch.setenv("SANA_LINATTN_PATH", "valu")
    w = workloads.Workload(f"jvp_B{B}N{N}H{H}L{L}dt{dt}", B, N, H, 32, dt, seed=100 + N % 13, block_len=L)
    x, (want, want_t) = case(w)
    for out_t in (torch.float32, torch.float16):
        got, got_t = run(x, w, out_t)
        compare(got, want, x[2], "f16" if out_t == torch.float16 else False, f"{w.name}/{path}")
        check_tangent(got_t, want_t, out_t, f"{w.name}/{path}")


HEAD_DIMS = [(2, 1000, 5, 100, 1, 64), (1, 777, 7, 0, 2, 16), (2, 33, 1, 0, 0, 16), (1, 4097, 3, 1, 0, 64),
             (1, 16384, 35, 0, 1, 64), (1, 16384, 140, 0, 1, 16), (1, 16384, 35, 0, 0, 64)]


@pytest.mark.parametrize("B,N,H,L,dt,D", HEAD_DIMS, ids=[f"B{b}N{n}H{h}L{l}dt{t}D{d}" for b, n, h, l, t, d in HEAD_DIMS])
def test_jvp_other_head_dims(B, N, H, L, dt, D):
    """Head dims 16 and 64 (32-feature groups on the matrix cores): ragged N,
    odd and single heads (a group that is a lone head of 16), block lengths 1
    and 100, the headline's token-head-feature count, fp32/bf16/fp16 inputs."""
    w = workloads.Workload(f"jvp_B{B}N{N}H{H}L{L}dt{dt}D{D}", B, N, H, D, dt, seed=140 + N % 17 + D, block_len=L)
    x, (want, want_t) = case(w)
    for out_t in ((torch.float32, torch.bfloat16) if N < 16384 else (torch.float32,)):
        got, got_t = run(x, w, out_t)
        compare(got, want, x[2], out_t == torch.bfloat16, w.name)
        check_tangent(got_t, want_t, out_t, w.name)


@pytest.mark.parametrize("D,H", [(32, 6), (16, 7)], ids=["D32", "D16"])
def test_jvp_primal_is_the_forward_and_repeatable(D, H):
    """The primal output equals sana_linattn_fwd's bit for bit (16-bit inputs:
    the state kernels sum the tokens in the same order), and two calls agree
    bit for bit."""
    import diffusion_transformer_relu_amd as sana
    w = workloads.Workload("jvp_prim", 2, 2048, H, D, workloads.DT_BF16, seed=110, block_len=512)
    x = [to_device(a) for a in workloads.make_inputs(w) + workloads.make_tangents(w)]
    o1, t1 = sana.linattn_jvp(*x, block_len=512)
    o2, t2 = sana.linattn_jvp(*x, block_len=512)
    f = sana.linattn_fwd(*x[:3], block_len=512)
    torch.cuda.synchronize()
    assert torch.equal(o1, f) and torch.equal(o1, o2) and torch.equal(t1, t2)
