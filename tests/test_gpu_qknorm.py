"""GPU parity of the qk_norm prologue (each head's q and k rows RMS-normalised
over their D features, scaled per channel, before phi) through
sana_linattn_fwd_qknorm, element by element against the fp64 oracle's
oracle.linattn_fwd(..., gamma_q=, gamma_k=, norm_eps=) on the same seeded
inputs and scales."""
import functools

import numpy as np
import pytest
import torch

import oracle
import workloads
from hip_helpers import compare, to_device

pytestmark = pytest.mark.gpu

NORM_EPS = 1e-6


@pytest.fixture(autouse=True)
def _announce(request):
    print(f"\n[gpu] {request.node.name}", flush=True)


@functools.lru_cache(maxsize=6)
def case(w, sides="qk", negative_every=3):
    q, k, v = workloads.make_inputs(w)
    gq, gk = workloads.make_gammas(w, negative_every)
    gq = gq if "q" in sides else None
    gk = gk if "k" in sides else None
    want = oracle.linattn_fwd(q, k, v, block_len=w.block_len, eps=w.eps, gamma_q=gq, gamma_k=gk,
                              norm_eps=NORM_EPS)
    return (q, k, v), (gq, gk), want


def gpu_gamma(g):
    return None if g is None else torch.from_numpy(g).to("cuda:0")


def run_qknorm(q, k, v, gq, gk, *, block_len=0, eps=1e-15, out_dtype=torch.float32):
    import diffusion_transformer_relu_amd as sana
    qd, kd, vd = to_device(q), to_device(k), to_device(v)
    out = sana.linattn_fwd(qd, kd, vd, eps=eps, out_dtype=out_dtype, block_len=block_len or None,
                           gamma_q=gpu_gamma(gq), gamma_k=gpu_gamma(gk), norm_eps=NORM_EPS)
    torch.cuda.synchronize()
    return out.float().cpu().double().numpy()


FULL = [workloads.HEADLINE, workloads.BLOCK_CAUSAL]


@pytest.mark.parametrize("w", FULL, ids=lambda w: w.name)
@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16], ids=["f32out", "bf16out"])
def test_full_size(w, out_dtype):
    """The 4096px Sana-1600M shape and the 16-block video shape, both sides
    normalised, a third of the channel scales negative."""
    (q, k, v), (gq, gk), want = case(w)
    got = run_qknorm(q, k, v, gq, gk, block_len=w.block_len, eps=w.eps, out_dtype=out_dtype)
    max_abs, rel = compare(got, want, v, out_dtype == torch.bfloat16, w.name + "/qknorm")
    print(f"[gpu] {w.name} qknorm {out_dtype}: max_abs={max_abs:.3e} rel_l2={rel:.3e}", flush=True)


OTHER = [
    workloads.Workload("qk_f32_B2_N4096_H70", 2, 4096, 70, 32, workloads.DT_F32, seed=301),
    workloads.Workload("qk_f16_B1_N8192_H70_L1024", 1, 8192, 70, 32, workloads.DT_F16, seed=302, block_len=1024),
    workloads.Workload("qk_d16_B1_N4097_H5_bf16", 1, 4097, 5, 16, workloads.DT_BF16, seed=303),
    workloads.Workload("qk_d16_B2_N1000_H7_L100_f32", 2, 1000, 7, 16, workloads.DT_F32, seed=304, block_len=100),
    workloads.Workload("qk_d64_B1_N4096_H18_bf16", 1, 4096, 18, 64, workloads.DT_BF16, seed=305),
    workloads.Workload("qk_d64_B3_N1000_H7_L100_f16", 3, 1000, 7, 64, workloads.DT_F16, seed=306, block_len=100),
    workloads.Workload("qk_d64_B2_N1000_H5_f32", 2, 1000, 5, 64, workloads.DT_F32, seed=307),
    workloads.Workload("qk_B1_N1_H1_bf16", 1, 1, 1, 32, workloads.DT_BF16, seed=308),
    workloads.Workload("qk_B2_N257_H3_L1_bf16", 2, 257, 3, 32, workloads.DT_BF16, seed=309, block_len=1),
]


@pytest.mark.parametrize("path", ["mfma", "valu"])
@pytest.mark.parametrize("w", OTHER, ids=lambda w: w.name)
def test_dtypes_head_dims_and_edges(monkeypatch, path, w):
    """Every input type, head dims 16 and 64 (odd head counts leave a
    32-feature group half empty), ragged tails, one token, blocks of one
    token; the matrix-core and the vector kernels."""
    if path == "valu":
        monkeypatch.setenv("SANA_LINATTN_PATH", "valu")
    (q, k, v), (gq, gk), want = case(w)
    for out_dtype in (torch.float32, torch.bfloat16):
        got = run_qknorm(q, k, v, gq, gk, block_len=w.block_len, eps=w.eps, out_dtype=out_dtype)
        compare(got, want, v, out_dtype == torch.bfloat16, f"{w.name} {path} {out_dtype}")


@pytest.mark.parametrize("sides", ["q", "k"])
def test_one_side_only(sides):
    """Only q or only k normalised (the other gamma NULL)."""
    w = workloads.Workload("qk_one_side_B2_N3000_H6", 2, 3000, 6, 32, workloads.DT_BF16, seed=310, block_len=1000)
    (q, k, v), (gq, gk), want = case(w, sides)
    got = run_qknorm(q, k, v, gq, gk, block_len=w.block_len, eps=w.eps)
    compare(got, want, v, False, f"{w.name} {sides}")


def test_all_positive_scales_and_large_rows():
    """Positive scales and rows of very different magnitudes (k scaled by 1e3,
    q by 1e-3): normalisation makes the result independent of a row's scale."""
    w = workloads.Workload("qk_scaled_B1_N2048_H4", 1, 2048, 4, 32, workloads.DT_F32, seed=311)
    q, k, v = workloads.make_inputs(w)
    q = (q * np.float32(1e-3)).astype(np.float32)
    k = (k * np.float32(1e3)).astype(np.float32)
    gq, gk = workloads.make_gammas(w)
    want = oracle.linattn_fwd(q, k, v, eps=w.eps, gamma_q=gq, gamma_k=gk, norm_eps=NORM_EPS)
    got = run_qknorm(q, k, v, gq, gk, eps=w.eps)
    compare(got, want, v, False, w.name)


def test_fused_qkv_views_and_null_gammas():
    """q, k, v as slices of one fused projection output read in place; with
    both gammas NULL the entry point gives bitwise the strided forward."""
    import diffusion_transformer_relu_amd as sana
    w = workloads.Workload("qk_qkv_B2_N1000_H3_bf16", 2, 1000, 3, 32, workloads.DT_BF16, seed=312, block_len=256)
    (q, k, v), (gq, gk), want = case(w)
    qkv = to_device(np.stack([q, k, v], axis=2))
    qv, kv, vv = qkv[:, :, 0], qkv[:, :, 1], qkv[:, :, 2]
    B, N, H, D = qv.shape
    ws = torch.empty(sana.sana_linattn_workspace_bytes(B, H, N, D, 256), dtype=torch.uint8, device="cuda:0")
    out = torch.empty((B, N, H, D), dtype=torch.float32, device="cuda:0")
    sana.sana_linattn_fwd_qknorm(qv, kv, vv, out, ws, gpu_gamma(gq), gpu_gamma(gk), norm_eps=NORM_EPS,
                                 block_len=256, eps=w.eps)
    plain = torch.empty_like(out)
    plain_ref = torch.empty_like(out)
    sana.sana_linattn_fwd_qknorm(qv, kv, vv, plain, ws, None, None, block_len=256, eps=w.eps)
    sana.sana_linattn_fwd_strided(qv, kv, vv, plain_ref, ws, block_len=256, eps=w.eps)
    torch.cuda.synchronize()
    compare(out.cpu().double().numpy(), want, v, False, w.name)
    assert torch.equal(plain.view(torch.int32), plain_ref.view(torch.int32))


def test_bitwise_repeatable():
    import diffusion_transformer_relu_amd as sana
    w = workloads.with_shape(workloads.HEADLINE, N=4096, name="qk_determinism")
    q, k, v = (to_device(a) for a in workloads.make_inputs(w))
    gq, gk = (gpu_gamma(g) for g in workloads.make_gammas(w, 3))
    outs = [sana.linattn_fwd(q, k, v, gamma_q=gq, gamma_k=gk, norm_eps=NORM_EPS) for _ in range(3)]
    torch.cuda.synchronize()
    for o in outs[1:]:
        assert torch.equal(o.view(torch.int32), outs[0].view(torch.int32))
