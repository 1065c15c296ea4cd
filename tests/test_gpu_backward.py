"""GPU parity of the backward (dq, dk, dv) through the C ABI against the fp64
oracle's backward, element by element, on the same seeded inputs."""
import functools

import numpy as np
import pytest
import torch

import oracle
import workloads
from hip_helpers import FP32_PIPELINE_FRAC, bf16_round, f16_round, to_device

pytestmark = pytest.mark.gpu

# Bar: the forward's (rel-L2 <= 1e-4) with max-abs taken relative to each
# gradient's own scale, max-abs <= 2e-3 * max|exact gradient|.  A 16-bit
# gradient is compared with the rounded exact gradient instead, and each
# element must lie within one ulp of the exact value plus the fp32 pipeline's
# own error (FP32_PIPELINE_FRAC of the scale).
REL_L2 = 1e-4
MAX_ABS_FRAC = 2e-3

DT = {workloads.DT_F32: torch.float32, workloads.DT_BF16: torch.bfloat16, workloads.DT_F16: torch.float16}


@pytest.fixture(autouse=True)
def _announce(request):
    print(f"\n[gpu] {request.node.name}", flush=True)


@functools.lru_cache(maxsize=4)
def case(w, gdt):
    q, k, v = workloads.make_inputs(w)
    g = workloads.make_dout(w, gdt)
    return (q, k, v, g), oracle.linattn_bwd(q, k, v, g, block_len=w.block_len, eps=w.eps)


def check(got, want, grad_t, label):
    for name, a, b in zip(("dq", "dk", "dv"), got, want):
        a = a.float().cpu().double().numpy()
        ref = b if grad_t == torch.float32 else (bf16_round(b) if grad_t == torch.bfloat16 else f16_round(b))
        diff = a - ref
        scale = float(np.max(np.abs(b))) if b.size else 1.0
        rel = float(np.linalg.norm(diff) / max(np.linalg.norm(ref), 1e-300))
        assert np.all(np.isfinite(a)), f"{label}/{name}"
        assert rel <= REL_L2, f"{label}/{name}: rel L2 {rel:.3e}"
        if grad_t == torch.float32:
            assert float(np.max(np.abs(diff))) <= MAX_ABS_FRAC * scale, f"{label}/{name}: max abs"
        else:
            e = np.floor(np.log2(np.maximum(np.abs(b), 1e-300)))
            ulp = np.exp2(e - 7) if grad_t == torch.bfloat16 else np.exp2(np.maximum(e, -14) - 10)
            bad = np.abs(a - b) > ulp + FP32_PIPELINE_FRAC * scale
            assert not np.any(bad), f"{label}/{name}: {int(bad.sum())} values beyond one ulp"


def run(q, k, v, g, block_len, eps, grad_t):
    import diffusion_transformer_relu_amd as sana
    out = sana.linattn_bwd(to_device(q), to_device(k), to_device(v), to_device(g), eps=eps, grad_dtype=grad_t,
                           block_len=block_len or None)
    torch.cuda.synchronize()
    return out


FULL = [workloads.S600M_1024, workloads.S1600M_2048, workloads.HEADLINE, workloads.BLOCK_CAUSAL]


@pytest.mark.parametrize("w", FULL, ids=lambda w: w.name)
@pytest.mark.parametrize("grad_t", [torch.float32, torch.bfloat16], ids=["f32grad", "bf16grad"])
def test_backward_full_size(w, grad_t):
    (q, k, v, g), want = case(w, workloads.DT_BF16)
    check(run(q, k, v, g, w.block_len, w.eps, grad_t), want, grad_t, w.name)


F32_IN = [workloads.with_shape(workloads.HEADLINE, in_dtype=workloads.DT_F32, name="sana1600m_4096px_f32in"),
          workloads.with_shape(workloads.BLOCK_CAUSAL, in_dtype=workloads.DT_F32, name="blockcausal_16x1024_f32in")]


@pytest.mark.parametrize("w", F32_IN, ids=lambda w: w.name)
@pytest.mark.parametrize("gdt,grad_t", [(workloads.DT_F32, torch.float32), (workloads.DT_BF16, torch.bfloat16)],
                         ids=["f32dout_f32grad", "bf16dout_bf16grad"])
def test_backward_full_size_fp32_inputs(w, gdt, grad_t):
    """fp32 q, k, v: the matrix-core query and key kernels on three-term bf16
    splits of the inputs, with an fp32 or a 16-bit upstream gradient."""
    (q, k, v, g), want = case(w, gdt)
    check(run(q, k, v, g, w.block_len, w.eps, grad_t), want, grad_t, w.name)


EDGE = [(2, 33, 3, 0, 1), (1, 257, 2, 64, 1), (3, 1000, 5, 100, 2), (1, 300, 2, 1, 0),
        (1, 4097, 1, 0, 2), (2, 256, 3, 0, 0)]


@pytest.mark.parametrize("B,N,H,L,dt", EDGE, ids=[f"B{b}N{n}H{h}L{l}dt{d}" for b, n, h, l, d in EDGE])
def test_backward_edge_shapes(B, N, H, L, dt):
    w = workloads.Workload(f"bwd_B{B}N{N}H{H}L{L}dt{dt}", B, N, H, 32, dt, seed=80 + N % 11, block_len=L)
    (q, k, v, g), want = case(w, dt)
    check(run(q, k, v, g, L, w.eps, DT[dt]), want, DT[dt], w.name)
    check(run(q, k, v, g, L, w.eps, torch.float32), want, torch.float32, w.name + "/f32grad")


HEAD_DIMS = [(2, 1000, 5, 100, 1, 64), (1, 777, 7, 0, 2, 16), (2, 33, 1, 0, 0, 16), (1, 300, 3, 1, 0, 64),
             (1, 513, 3, 64, 2, 64), (1, 777, 5, 100, 0, 16), (1, 16384, 35, 0, 1, 64), (1, 16384, 140, 0, 1, 16)]


@pytest.mark.parametrize("B,N,H,L,dt,D", HEAD_DIMS, ids=[f"B{b}N{n}H{h}L{l}dt{t}D{d}" for b, n, h, l, t, d in HEAD_DIMS])
def test_backward_other_head_dims(B, N, H, L, dt, D):
    """Head dims 16 and 64 (matrix-core passes): ragged N, odd and single
    heads, block lengths 1, 64 and 100, the headline's token-head-feature
    count."""
    w = workloads.Workload(f"bwd_B{B}N{N}H{H}L{L}dt{dt}D{D}", B, N, H, D, dt, seed=150 + N % 19 + D, block_len=L)
    (q, k, v, g), want = case(w, dt)
    check(run(q, k, v, g, L, w.eps, DT[dt]), want, DT[dt], w.name)
    if N < 16384:
        other = torch.bfloat16 if dt == workloads.DT_F32 else torch.float32
        check(run(q, k, v, g, L, w.eps, other), want, other, w.name + "/" + str(other))


D64_MIXED = [(1, 1000, 3, 100, workloads.DT_F32, workloads.DT_BF16), (2, 333, 2, 0, workloads.DT_F32, workloads.DT_F16),
             (1, 1000, 3, 100, workloads.DT_BF16, workloads.DT_F32), (1, 513, 1, 64, workloads.DT_F16, workloads.DT_F32),
             (1, 16384, 35, 0, workloads.DT_F32, workloads.DT_F32)]


@pytest.mark.parametrize("B,N,H,L,dt,gdt", D64_MIXED, ids=[f"B{b}N{n}H{h}L{l}in{t}dout{g}" for b, n, h, l, t, g in D64_MIXED])
def test_backward_head_dim_64_mixed_types(B, N, H, L, dt, gdt):
    """Head dim 64 with fp32 q and a 16-bit upstream gradient (q read by each
    wave), 16-bit q and an fp32 gradient (the gradient goes in as the split u
    of both groups), and fp32 throughout at the headline's feature count."""
    w = workloads.Workload(f"bwd64_B{B}N{N}H{H}L{L}in{dt}dout{gdt}", B, N, H, 64, dt, seed=170 + N % 23, block_len=L)
    (q, k, v, g), want = case(w, gdt)
    check(run(q, k, v, g, L, w.eps, torch.float32), want, torch.float32, w.name)
    if N < 16384:
        check(run(q, k, v, g, L, w.eps, torch.bfloat16), want, torch.bfloat16, w.name + "/bf16grad")


MIXED16 = [(2, 1000, 5, 100, workloads.DT_BF16, workloads.DT_F16, 32), (1, 777, 3, 0, workloads.DT_F16, workloads.DT_BF16, 32),
           (1, 2049, 1, 512, workloads.DT_BF16, workloads.DT_F16, 32), (1, 777, 7, 100, workloads.DT_BF16, workloads.DT_F16, 16),
           (2, 1000, 3, 0, workloads.DT_F16, workloads.DT_BF16, 16), (1, 513, 1, 64, workloads.DT_BF16, workloads.DT_BF16, 16),
           (1, 777, 3, 100, workloads.DT_BF16, workloads.DT_F16, 64), (2, 333, 2, 0, workloads.DT_F16, workloads.DT_BF16, 64)]


@pytest.mark.parametrize("B,N,H,L,dt,gdt,D", MIXED16,
                         ids=[f"B{b}N{n}H{h}L{l}in{t}dout{g}D{d}" for b, n, h, l, t, g, d in MIXED16])
def test_backward_mixed_16bit_types(B, N, H, L, dt, gdt, D):
    """Head dims 32, 16 and 64 with 16-bit q and a 16-bit upstream gradient
    of either format (the per-wave query kernels' four q/dout format pairs;
    identity operands of both formats), ragged tails, odd and single heads
    (head dim 16: a group that is a lone head), fp32, bf16 and fp16
    gradients."""
    w = workloads.Workload(f"bwdmix_B{B}N{N}H{H}L{L}in{dt}dout{gdt}D{D}", B, N, H, D, dt, seed=190 + N % 29 + D,
                           block_len=L)
    (q, k, v, g), want = case(w, gdt)
    for grad_t in (torch.float32, torch.bfloat16, torch.float16):
        check(run(q, k, v, g, L, w.eps, grad_t), want, grad_t, f"{w.name}/{grad_t}")


def test_backward_single_token_is_identity_in_v():
    """N = 1: out = v * den / (den + eps) does not depend on q or k (their
    exact gradients vanish; what is left is rounding of cancelling terms), and
    dv = dout * den / (den + eps)."""
    w = workloads.Workload("bwd_N1", 2, 1, 3, 32, workloads.DT_F32, seed=93)
    (q, k, v, g), (dq0, dk0, dv0) = case(w, workloads.DT_F32)
    dq, dk, dv = (t.cpu().double().numpy() for t in run(q, k, v, g, 0, w.eps, torch.float32))
    assert np.max(np.abs(dq0)) < 1e-12 and np.max(np.abs(dk0)) < 1e-12
    assert np.max(np.abs(dq)) < 1e-5 and np.max(np.abs(dk)) < 1e-5
    np.testing.assert_allclose(dv, dv0, rtol=1e-6, atol=1e-7)


def test_backward_eps_path_and_repeatability():
    w = workloads.Workload("bwd_eps", 1, 512, 3, 32, workloads.DT_BF16, seed=91, negative_k_heads=(1,),
                           negative_q_rows=((0, 7, 0), (0, 300, 2)))
    (q, k, v, g), want = case(w, workloads.DT_BF16)
    a = run(q, k, v, g, 0, w.eps, torch.float32)
    b = run(q, k, v, g, 0, w.eps, torch.float32)
    check(a, want, torch.float32, w.name)
    for x, y in zip(a, b):
        assert torch.equal(x, y)
    for t in a:
        assert torch.all(t[:, :, 1] == 0)
    assert torch.all(a[0][0, 7, 0] == 0) and torch.all(a[0][0, 300, 2] == 0)


def test_backward_mixed_dtypes():
    """fp16 inputs with an fp32 upstream gradient and bf16 gradients out."""
    w = workloads.Workload("bwd_mixed", 2, 2048, 6, 32, workloads.DT_F16, seed=92, block_len=512)
    (q, k, v, g), want = case(w, workloads.DT_F32)
    check(run(q, k, v, g, w.block_len, w.eps, torch.bfloat16), want, torch.bfloat16, w.name)
