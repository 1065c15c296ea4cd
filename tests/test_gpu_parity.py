"""GPU parity: the HIP path through the C ABI against the fp64 oracle, element
by element, on the same seeded inputs."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from hip_helpers import compare, inputs_and_oracle, run_hip, to_device

pytestmark = pytest.mark.gpu

FULL = [workloads.S600M_1024, workloads.S1600M_1024, workloads.S1600M_2048,
        workloads.HEADLINE, workloads.BLOCK_CAUSAL]


@pytest.fixture(autouse=True)
def _announce(request):
    print(f"\n[gpu] {request.node.name}", flush=True)


def test_tiny_config_f32():
    w = workloads.TINY
    (q, k, v), want = inputs_and_oracle(w)
    got = run_hip(q, k, v, eps=w.eps)
    compare(got, want, v, False, w.name)
    assert np.all(got[:, :, 1, :] == 0.0)          # all-negative K head: the eps path gives exact zeros


@pytest.mark.parametrize("w", FULL, ids=lambda w: w.name)
@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16], ids=["f32out", "bf16out"])
def test_full_size_configs(w, out_dtype):
    (q, k, v), want = inputs_and_oracle(w)
    got = run_hip(q, k, v, block_len=w.block_len, eps=w.eps, out_dtype=out_dtype)
    max_abs, rel = compare(got, want, v, out_dtype == torch.bfloat16, w.name)
    print(f"[gpu] {w.name} {out_dtype}: max_abs={max_abs:.3e} rel_l2={rel:.3e}", flush=True)


F32_IN = [workloads.with_shape(workloads.HEADLINE, in_dtype=workloads.DT_F32, name="sana1600m_4096px_f32in"),
          workloads.with_shape(workloads.BLOCK_CAUSAL, in_dtype=workloads.DT_F32, name="blockcausal_16x1024_f32in")]


@pytest.mark.parametrize("w", F32_IN, ids=lambda w: w.name)
@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16], ids=["f32out", "bf16out"])
def test_full_size_fp32_inputs(w, out_dtype):
    """fp32 q, k, v at the bench shapes: the matrix-core kernels on three-term
    bf16 splits of the inputs."""
    (q, k, v), want = inputs_and_oracle(w)
    got = run_hip(q, k, v, block_len=w.block_len, eps=w.eps, out_dtype=out_dtype)
    max_abs, rel = compare(got, want, v, out_dtype == torch.bfloat16, w.name)
    print(f"[gpu] {w.name} {out_dtype}: max_abs={max_abs:.3e} rel_l2={rel:.3e}", flush=True)


EDGE = [
    # (B, N, H, block_len, in_dtype)
    (1, 1, 1, 0, workloads.DT_BF16),
    (1, 31, 3, 0, workloads.DT_BF16),
    (2, 257, 5, 0, workloads.DT_BF16),
    (3, 1000, 7, 0, workloads.DT_BF16),
    (1, 4097, 2, 0, workloads.DT_BF16),
    (1, 16384, 2, 0, workloads.DT_BF16),     # one head pair: 64 work-group ranges per block (>32 merge slots)
    (2, 5000, 3, 1100, workloads.DT_BF16),   # ranges crossing head-pair, batch and block boundaries
    (2, 1000, 3, 100, workloads.DT_BF16),
    (1, 999, 4, 1, workloads.DT_BF16),
    (1, 1024, 2, 1024, workloads.DT_BF16),
    (1, 700, 3, 5000, workloads.DT_BF16),
    (1, 3000, 1, 257, workloads.DT_BF16),
    (2, 300, 3, 0, workloads.DT_F32),
    (1, 1000, 2, 64, workloads.DT_F32),
]


@pytest.mark.parametrize("path", ["mfma", "valu"])
@pytest.mark.parametrize("B,N,H,L,dt", EDGE, ids=[f"B{b}N{n}H{h}L{l}{'bf16' if d else 'f32'}" for b, n, h, l, d in EDGE])
def test_edge_shapes(monkeypatch, path, B, N, H, L, dt):
    if path == "valu":
        monkeypatch.setenv("SANA_LINATTN_PATH", "valu")
    w = workloads.Workload(f"edge_{B}_{N}_{H}_{L}", B, N, H, 32, dt, seed=1000 + N + H, block_len=L)
    (q, k, v), want = inputs_and_oracle(w)
    for out_dtype in (torch.float32, torch.bfloat16):
        got = run_hip(q, k, v, block_len=L, eps=w.eps, out_dtype=out_dtype)
        compare(got, want, v, out_dtype == torch.bfloat16, f"{w.name} {path} {out_dtype}")


@pytest.mark.parametrize("chunk,tile", [("128", "64"), ("256", "128"), ("1024", "256"), ("2048", "512")])
def test_decomposition_does_not_change_result(monkeypatch, chunk, tile):
    monkeypatch.setenv("SANA_LINATTN_CHUNK", chunk)
    monkeypatch.setenv("SANA_LINATTN_APPLY_TILE", tile)
    w = workloads.with_shape(workloads.BLOCK_CAUSAL, N=5000, H=6, block_len=1024, name="decomp")
    (q, k, v), want = inputs_and_oracle(w)
    compare(run_hip(q, k, v, block_len=w.block_len, eps=w.eps), want, v, False, f"chunk {chunk} tile {tile}")
    w2 = workloads.with_shape(workloads.HEADLINE, N=5000, H=6, name="decomp_nc")
    (q, k, v), want = inputs_and_oracle(w2)
    compare(run_hip(q, k, v, eps=w2.eps), want, v, False, f"nc chunk {chunk} tile {tile}")


def test_bitwise_repeatable_and_stages_equal_full_call():
    import diffusion_transformer_relu_amd as sana
    w = workloads.with_shape(workloads.HEADLINE, N=4096, H=70, name="determinism")
    q, k, v = [to_device(a) for a in workloads.make_inputs(w)]
    B, N, H, D = q.shape
    ws = torch.empty(sana.sana_linattn_workspace_bytes(B, H, N, D, 0), dtype=torch.uint8, device="cuda:0")
    outs = []
    for _ in range(3):
        out = torch.empty(q.shape, dtype=torch.float32, device="cuda:0")
        sana.sana_linattn_fwd(q, k, v, out, ws)
        outs.append(out)
    staged = torch.empty(q.shape, dtype=torch.float32, device="cuda:0")
    for st in (sana.SANA_STAGE_STATE, sana.SANA_STAGE_MERGE, sana.SANA_STAGE_APPLY):
        sana.sana_linattn_fwd_stages(q, k, v, staged, ws, st)
    torch.cuda.synchronize()
    for o in outs[1:] + [staged]:
        assert torch.equal(o.view(torch.int32), outs[0].view(torch.int32))


def test_eps_path_rows_are_exact_zeros():
    w = workloads.Workload("eps_rows", 1, 2000, 4, 32, workloads.DT_BF16, seed=77, negative_k_heads=(2,),
                           negative_q_rows=((0, 5, 0), (0, 1999, 3), (0, 640, 1)))
    (q, k, v), want = inputs_and_oracle(w)
    for L in (0, 512):
        got = run_hip(q, k, v, block_len=L, eps=w.eps)
        assert np.all(got[0, :, 2] == 0.0)
        for (_, n, h) in w.negative_q_rows:
            assert np.all(got[0, n, h] == 0.0)
    compare(run_hip(q, k, v, eps=w.eps), want, v, False, w.name)


def test_non_default_stream_and_empty_problem():
    import diffusion_transformer_relu_amd as sana
    w = workloads.with_shape(workloads.S600M_1024, B=1, N=512, H=4, name="stream")
    (q, k, v), want = inputs_and_oracle(w)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        got = run_hip(q, k, v, eps=w.eps, stream=s)
    compare(got, want, v, False, w.name)
    z = torch.empty((1, 0, 2, 32), dtype=torch.bfloat16, device="cuda:0")
    out = torch.empty((1, 0, 2, 32), dtype=torch.float32, device="cuda:0")
    ws = torch.empty(1, dtype=torch.uint8, device="cuda:0")
    sana.sana_linattn_fwd(z, z, z, out, ws)
    sana.sana_linattn_blockcausal_fwd(z, z, z, out, ws, 16)


def test_allocating_wrappers_with_a_stream_that_is_not_current():
    """linattn_fwd / linattn_bwd / linattn_jvp given `stream=` without making it
    current: their output and workspace are allocated on that stream, so memory
    that the current stream allocates and writes meanwhile (while the side
    stream is still busy) never aliases them."""
    import diffusion_transformer_relu_amd as sana
    w = workloads.with_shape(workloads.S600M_1024, B=1, N=2048, H=8, name="side_stream")
    (q, k, v), want = inputs_and_oracle(w)
    qd, kd, vd = to_device(q), to_device(k), to_device(v)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())   # the inputs are ready on s
    big = torch.randn((4096, 4096), device="cuda:0")
    with torch.cuda.stream(s):
        for _ in range(8):                      # keep s busy before the LiteLA kernels
            big = big @ big
            big /= big.abs().max()
    out = sana.linattn_fwd(qd, kd, vd, eps=w.eps, stream=s)
    dq, dk, dv = sana.linattn_bwd(qd, kd, vd, qd, eps=w.eps, stream=s)
    o2, ot = sana.linattn_jvp(qd, kd, vd, qd, kd, vd, eps=w.eps, stream=s)
    junk = [torch.full((1 << 22,), 3.0, device="cuda:0") for _ in range(8)]   # the current stream
    s.synchronize()
    torch.cuda.synchronize()
    compare(out.cpu().double().numpy(), want, v, False, w.name)
    assert torch.equal(o2.view(torch.int32), out.view(torch.int32))
    ref = sana.linattn_bwd(qd, kd, vd, qd, eps=w.eps)
    torch.cuda.synchronize()
    for a, b in zip((dq, dk, dv), ref):
        assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    assert all(torch.all(j == 3.0) for j in junk)
    del big


def test_device_argument_errors_leave_output_untouched():
    import diffusion_transformer_relu_amd as sana
    w = workloads.with_shape(workloads.S600M_1024, B=1, N=256, H=2, name="errs")
    q, k, v = [to_device(a) for a in workloads.make_inputs(w)]
    out = torch.full(q.shape, 7.0, dtype=torch.float32, device="cuda:0")
    need = sana.sana_linattn_workspace_bytes(1, 2, 256, 32, 0)
    ws = torch.empty(need + 256, dtype=torch.uint8, device="cuda:0")
    P, I = sana.lib.sana_linattn_fwd, q.data_ptr()
    args = lambda qp, op, wp, wb: (qp, k.data_ptr(), v.data_ptr(), op, 1, 0, 1, 2, 256, 32, 1e-15, wp, wb, None)
    assert P(*args(I + 2, out.data_ptr(), ws.data_ptr(), need)) == sana.SANA_ERR_ALIGNMENT
    assert P(*args(I, I, ws.data_ptr(), need)) == sana.SANA_ERR_ALIAS
    assert P(*args(I, out.data_ptr(), ws.data_ptr(), need - 1)) == sana.SANA_ERR_WORKSPACE
    assert P(*args(I, out.data_ptr(), ws.data_ptr() + 128, need)) == sana.SANA_ERR_ALIGNMENT
    torch.cuda.synchronize()
    assert torch.all(out == 7.0)


@pytest.mark.parametrize("w,cuts", [
    (workloads.Workload("stream_B2_N4096_H6_L512", 2, 4096, 6, 32, workloads.DT_BF16, seed=31, block_len=512),
     (0, 1024, 2560)),
    (workloads.Workload("stream_B1_N1000_H3_L64_f32", 1, 1000, 3, 32, workloads.DT_F32, seed=32, block_len=64),
     (0, 64, 640)),
    (workloads.BLOCK_CAUSAL, (0, 4096, 8192, 12288)),
], ids=lambda x: x.name if hasattr(x, "name") else str(len(x)))
def test_streaming_chunks_match_one_shot(w, cuts):
    """Block-aligned chunks, each call continuing from the previous call's
    carried state (updated in place), reproduce the one-shot block-causal
    output; the final carried state is the whole sequence's state."""
    import diffusion_transformer_relu_amd as sana
    (q, k, v), want = inputs_and_oracle(w)
    _, st_want = oracle.linattn_fwd(q, k, v, block_len=w.block_len, return_states=True)
    qd, kd, vd = to_device(q), to_device(k), to_device(v)
    B, N, H, D = qd.shape
    out = torch.empty((B, N, H, D), dtype=torch.float32, device="cuda:0")
    state = torch.empty((B, H, D, D + 1), dtype=torch.float32, device="cuda:0")
    bounds = list(cuts) + [N]
    for c, (a, b) in enumerate(zip(bounds[:-1], bounds[1:])):
        n = b - a
        ws = torch.empty(sana.sana_linattn_workspace_bytes(B, H, n, D, w.block_len), dtype=torch.uint8,
                         device="cuda:0")
        o = torch.empty((B, n, H, D), dtype=torch.float32, device="cuda:0")
        sana.sana_linattn_blockcausal_stream_fwd(qd[:, a:b].contiguous(), kd[:, a:b].contiguous(),
                                                 vd[:, a:b].contiguous(), o, ws, w.block_len,
                                                 state_in=state if c else None, state_out=state, eps=w.eps)
        out[:, a:b] = o
    torch.cuda.synchronize()
    compare(out.cpu().double().numpy(), want, v, False, w.name)
    got_state = state.cpu().double().numpy()
    final = st_want[:, :, -1]
    assert np.max(np.abs(got_state - final)) <= 1e-5 * np.max(np.abs(final))


STRIDED = [
    workloads.Workload("qkv_B2_N1000_H3_bf16", 2, 1000, 3, 32, workloads.DT_BF16, seed=41),
    workloads.Workload("qkv_B2_N1000_H3_L128_f32", 2, 1000, 3, 32, workloads.DT_F32, seed=42, block_len=128),
    workloads.S1600M_1024,
]


@pytest.mark.parametrize("w", STRIDED, ids=lambda w: w.name)
@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16], ids=["f32out", "bf16out"])
def test_fused_qkv_views_read_in_place(w, out_dtype):
    """q, k, v as the three slices of one [B, N, 3, H, D] projection output and
    out as one slice of a [B, N, 2, H, D] buffer: the result equals the oracle's
    on the contiguous tensors, and the other output slice stays untouched."""
    import diffusion_transformer_relu_amd as sana
    (q, k, v), want = inputs_and_oracle(w)
    qkv = to_device(np.stack([q, k, v], axis=2))              # [B, N, 3, H, D]
    qv, kv, vv = qkv[:, :, 0], qkv[:, :, 1], qkv[:, :, 2]
    assert not qv.is_contiguous() and qv.stride(1) == 3 * w.H * 32
    B, N, H, D = qv.shape
    buf = torch.full((B, N, 2, H, D), 7.0, dtype=out_dtype, device="cuda:0")
    out = buf[:, :, 1]
    ws = torch.empty(sana.sana_linattn_workspace_bytes(B, H, N, D, w.block_len), dtype=torch.uint8, device="cuda:0")
    sana.sana_linattn_fwd_strided(qv, kv, vv, out, ws, block_len=w.block_len, eps=w.eps)
    torch.cuda.synchronize()
    compare(out.float().cpu().double().numpy(), want, v, out_dtype == torch.bfloat16, w.name)
    assert torch.all(buf[:, :, 0] == 7.0)


@pytest.mark.parametrize("path", ["mfma", "valu"])
def test_broadcast_and_transposed_views(monkeypatch, path):
    """A batch stride of 0 (k, v shared by both batches) and an output laid out
    [N, B, H, D] give the oracle's result on the materialised tensors; the
    strided result is bitwise the contiguous call's."""
    import diffusion_transformer_relu_amd as sana
    if path == "valu":
        monkeypatch.setenv("SANA_LINATTN_PATH", "valu")
    w = workloads.Workload("bcast_B1_N777_H4_bf16", 1, 777, 4, 32, workloads.DT_BF16, seed=43)
    q1, k1, v1 = workloads.make_inputs(w)
    q2, _, _ = workloads.make_inputs(workloads.with_shape(w, seed=44))
    q = np.concatenate([q1, q2], axis=0)
    k, v = np.concatenate([k1, k1], axis=0), np.concatenate([v1, v1], axis=0)
    want = oracle.linattn_fwd(q, k, v, eps=w.eps)
    qd, kd, vd = to_device(q), to_device(k1).expand(2, -1, -1, -1), to_device(v1).expand(2, -1, -1, -1)
    assert kd.stride(0) == 0
    B, N, H, D = qd.shape
    out = torch.empty((N, B, H, D), dtype=torch.float32, device="cuda:0").permute(1, 0, 2, 3)
    ws = torch.empty(sana.sana_linattn_workspace_bytes(B, H, N, D, 0), dtype=torch.uint8, device="cuda:0")
    sana.sana_linattn_fwd_strided(qd, kd, vd, out, ws, eps=w.eps)
    dense = torch.empty((B, N, H, D), dtype=torch.float32, device="cuda:0")
    sana.sana_linattn_fwd(qd, kd.contiguous(), vd.contiguous(), dense, ws, eps=w.eps)
    torch.cuda.synchronize()
    compare(out.cpu().double().numpy(), want, v, False, w.name)
    assert torch.equal(out, dense)



F16_CASES = [
    workloads.Workload("f16_sana1600m_2048px_B2_N4096_H70", 2, 4096, 70, 32, workloads.DT_F16, seed=51),
    workloads.Workload("f16_sana1600m_4096px_B1_N16384_H70", 1, 16384, 70, 32, workloads.DT_F16, seed=52,
                       v_scale=0.5),
    workloads.Workload("f16_blockcausal_B1_N8192_H70_L1024", 1, 8192, 70, 32, workloads.DT_F16, seed=53,
                       block_len=1024),
]


@pytest.mark.parametrize("w", F16_CASES, ids=lambda w: w.name)
@pytest.mark.parametrize("out_dtype", [torch.float32, torch.float16, torch.bfloat16], ids=["f32out", "f16out", "bf16out"])
def test_f16_inputs(w, out_dtype):
    """fp16 q, k, v (fp32 accumulation) at Sana shapes, every output dtype."""
    (q, k, v), want = inputs_and_oracle(w)
    got = run_hip(q, k, v, block_len=w.block_len, eps=w.eps, out_dtype=out_dtype)
    kind = {torch.float32: False, torch.float16: "f16", torch.bfloat16: True}[out_dtype]
    compare(got, want, v, kind, w.name)


F16_EDGE = [(1, 1, 1, 0), (2, 33, 3, 0), (1, 1000, 5, 64), (3, 257, 7, 100), (1, 4097, 2, 0)]


@pytest.mark.parametrize("path", ["mfma", "valu"])
@pytest.mark.parametrize("B,N,H,L", F16_EDGE, ids=[f"B{b}N{n}H{h}L{l}" for b, n, h, l in F16_EDGE])
def test_f16_edge_shapes(monkeypatch, path, B, N, H, L):
    if path == "valu":
        monkeypatch.setenv("SANA_LINATTN_PATH", "valu")
    w = workloads.Workload(f"f16edge_B{B}N{N}H{H}L{L}", B, N, H, 32, workloads.DT_F16, seed=60 + N % 7,
                           block_len=L)
    (q, k, v), want = inputs_and_oracle(w)
    for out_dtype, kind in ((torch.float32, False), (torch.float16, "f16")):
        got = run_hip(q, k, v, block_len=L, eps=w.eps, out_dtype=out_dtype)
        compare(got, want, v, kind, f"{w.name}/{path}/{kind}")


@pytest.mark.parametrize("k_scale,v_scale", [(1e-5, 1.0), (30.0, 1e4), (1.0, 1e-4)],
                         ids=["subnormal_k", "large_kv", "tiny_v"])
def test_f16_extreme_magnitudes(k_scale, v_scale):
    """fp16 inputs far from unit scale: subnormal keys, values near the top of
    the fp16 range (the state and the normaliser grow far beyond it, which fp32
    accumulation absorbs), tiny values.  fp16 out cannot overflow since every
    output lies within the range of V."""
    rng = np.random.default_rng(71)
    shape = (2, 2048, 6, 32)
    q = rng.standard_normal(shape, dtype=np.float32).astype(np.float16)
    k = (rng.standard_normal(shape, dtype=np.float32) * np.float32(k_scale)).astype(np.float16)
    v = (rng.standard_normal(shape, dtype=np.float32) * np.float32(v_scale)).astype(np.float16)
    want = oracle.linattn_fwd(q, k, v)
    for out_dtype, kind in ((torch.float32, False), (torch.float16, "f16")):
        got = run_hip(q, k, v, out_dtype=out_dtype)
        compare(got, want, v, kind, f"k{k_scale}_v{v_scale}/{kind}")


@pytest.mark.parametrize("in_dt", [workloads.DT_BF16, workloads.DT_F16])
def test_16bit_out_is_the_fp32_out_rounded_to_nearest_even(in_dt):
    """The bf16 and fp16 outputs are the fp32 output rounded once to nearest
    even (torch's conversion on the host), bit for bit."""
    w = workloads.Workload("round_B2_N3000_H5", 2, 3000, 5, 32, in_dt, seed=47, v_scale=3.0)
    q, k, v = (to_device(x) for x in workloads.make_inputs(w))
    import diffusion_transformer_relu_amd as sana
    f32 = sana.linattn_fwd(q, k, v, out_dtype=torch.float32).cpu()
    for t in (torch.bfloat16, torch.float16):
        got = sana.linattn_fwd(q, k, v, out_dtype=t).cpu()
        assert torch.equal(got.view(torch.int16), f32.to(t).view(torch.int16)), t


HEAD_DIMS = [
    workloads.Workload("d16_B2_N1000_H8_bf16", 2, 1000, 8, 16, workloads.DT_BF16, seed=121),
    workloads.Workload("d16_B1_N4096_H72_L1024_f16", 1, 4096, 72, 16, workloads.DT_F16, seed=122, block_len=1024),
    workloads.Workload("d64_B2_N1000_H5_f32", 2, 1000, 5, 64, workloads.DT_F32, seed=123, block_len=300),
    workloads.Workload("d64_B1_N4096_H18_bf16", 1, 4096, 18, 64, workloads.DT_BF16, seed=124),
    workloads.Workload("d64_B3_N1000_H7_L100_f16", 3, 1000, 7, 64, workloads.DT_F16, seed=127, block_len=100),
    workloads.Workload("d64_B2_N33_H1_bf16", 2, 33, 1, 64, workloads.DT_BF16, seed=128),
    workloads.Workload("d64_B1_N4097_H3_L1_bf16", 1, 4097, 3, 64, workloads.DT_BF16, seed=129, block_len=1),
    workloads.Workload("d64_B1_N16384_H35_bf16", 1, 16384, 35, 64, workloads.DT_BF16, seed=130),
    workloads.Workload("d16_B3_N1000_H7_L100_bf16", 3, 1000, 7, 16, workloads.DT_BF16, seed=131, block_len=100),
    workloads.Workload("d16_B2_N33_H1_f16", 2, 33, 1, 16, workloads.DT_F16, seed=132),
    workloads.Workload("d16_B1_N4097_H5_L1_bf16", 1, 4097, 5, 16, workloads.DT_BF16, seed=133, block_len=1),
    workloads.Workload("d16_B2_N1000_H3_f32", 2, 1000, 3, 16, workloads.DT_F32, seed=134),
    workloads.Workload("d16_B1_N16384_H140_bf16", 1, 16384, 140, 16, workloads.DT_BF16, seed=135),
    workloads.Workload("d16_B1_N777_H7_L256_f32", 1, 777, 7, 16, workloads.DT_F32, seed=136, block_len=256),
    workloads.Workload("d64_B1_N16384_H35_f32", 1, 16384, 35, 64, workloads.DT_F32, seed=137),
    workloads.Workload("d16_B1_N16384_H140_f32", 1, 16384, 140, 16, workloads.DT_F32, seed=138),
]


@pytest.mark.parametrize("w", HEAD_DIMS, ids=lambda w: w.name)
@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16], ids=["f32out", "bf16out"])
def test_other_head_dims(w, out_dtype):
    """Head dims 16 and 64 against the oracle (matrix cores; fp32 inputs as
    three-term splits); 16384 tokens x 35 heads of 64 and x 140 heads of 16
    are the headline's token-head-feature count; odd and single heads of 16
    leave a 32-feature group half empty."""
    (q, k, v), want = inputs_and_oracle(w)
    got = run_hip(q, k, v, block_len=w.block_len, eps=w.eps, out_dtype=out_dtype)
    compare(got, want, v, out_dtype == torch.bfloat16, w.name)


@pytest.mark.parametrize("w", [w for w in HEAD_DIMS if w.N < 16384], ids=lambda w: w.name)
def test_other_head_dims_vector_path(monkeypatch, w):
    """The vector-unit kernels (SANA_LINATTN_PATH=valu) for the same cases."""
    monkeypatch.setenv("SANA_LINATTN_PATH", "valu")
    (q, k, v), want = inputs_and_oracle(w)
    got = run_hip(q, k, v, block_len=w.block_len, eps=w.eps, out_dtype=torch.float32)
    compare(got, want, v, False, w.name + "/valu")


def test_other_head_dims_streaming_and_strided():
    """D = 64 streamed with a carried state; D = 16 from a fused qkv buffer."""
    import diffusion_transformer_relu_amd as sana
    w = workloads.Workload("d64_stream", 2, 2048, 3, 64, workloads.DT_BF16, seed=125, block_len=256)
    (q, k, v), want = inputs_and_oracle(w)
    _, st_want = oracle.linattn_fwd(q, k, v, block_len=256, return_states=True)
    qd, kd, vd = to_device(q), to_device(k), to_device(v)
    out = torch.empty((2, 2048, 3, 64), dtype=torch.float32, device="cuda:0")
    state = torch.empty((2, 3, 64, 65), dtype=torch.float32, device="cuda:0")
    for c, (a, b) in enumerate(((0, 768), (768, 2048))):
        ws = torch.empty(sana.sana_linattn_workspace_bytes(2, 3, b - a, 64, 256), dtype=torch.uint8, device="cuda:0")
        o = torch.empty((2, b - a, 3, 64), dtype=torch.float32, device="cuda:0")
        sana.sana_linattn_blockcausal_stream_fwd(qd[:, a:b].contiguous(), kd[:, a:b].contiguous(),
                                                 vd[:, a:b].contiguous(), o, ws, 256,
                                                 state_in=state if c else None, state_out=state)
        out[:, a:b] = o
    torch.cuda.synchronize()
    compare(out.cpu().double().numpy(), want, v, False, w.name)
    fin = st_want[:, :, -1]
    assert np.max(np.abs(state.cpu().double().numpy() - fin)) <= 1e-5 * np.max(np.abs(fin))

    w2 = workloads.Workload("d16_qkv", 2, 777, 6, 16, workloads.DT_BF16, seed=126)
    (q, k, v), want = inputs_and_oracle(w2)
    qkv = to_device(np.stack([q, k, v], axis=2))
    out = torch.empty((2, 777, 6, 16), dtype=torch.float32, device="cuda:0")
    ws = torch.empty(sana.sana_linattn_workspace_bytes(2, 6, 777, 16, 0), dtype=torch.uint8, device="cuda:0")
    sana.sana_linattn_fwd_strided(qkv[:, :, 0], qkv[:, :, 1], qkv[:, :, 2], out, ws)
    torch.cuda.synchronize()
    compare(out.cpu().double().numpy(), want, v, False, w2.name)


def test_offsets_beyond_2_31_elements():
    """q, k, v and out of 2^31 + elements each (B=1, N=4M+, H=16, D=32; 20 GB on
    the device): every offset past 2^31 is computed in 64 bits.  The inputs are
    drawn on the device from a seeded generator; one head's slice is copied back
    and checked against the oracle at the last tokens (the largest offsets)."""
    import diffusion_transformer_relu_amd as sana
    B, N, H, D = 1, (1 << 22) + 1000, 16, 32
    gen = torch.Generator(device="cuda:0").manual_seed(2024)
    q, k, v = (torch.randn((B, N, H, D), device="cuda:0", generator=gen).to(torch.bfloat16) for _ in range(3))
    assert q.numel() > (1 << 31)
    out = sana.linattn_fwd(q, k, v)
    h = H - 1
    sl = [x[:, :, h:h + 1].contiguous().cpu().view(torch.int16).numpy().view(np.uint16) for x in (q, k, v)]
    tail = out[:, -64:, h:h + 1].cpu().double().numpy()
    del q, k, v, out
    torch.cuda.empty_cache()
    want = oracle.linattn_fwd(*sl)[:, -64:]
    compare(tail, want, sl[2], False, "offsets>2^31")


def test_concurrent_calls_from_two_threads_on_two_streams():
    """Calls are re-entrant: two host threads, each with its own stream and
    workspace, interleave many calls; every result equals the single-threaded one."""
    import threading

    import diffusion_transformer_relu_amd as sana
    ws_ = [workloads.Workload(f"thr{t}", 2, 3000, 7, 32, workloads.DT_BF16, seed=130 + t, block_len=512 * t)
           for t in range(2)]
    ins = [[to_device(x) for x in workloads.make_inputs(w)] for w in ws_]
    ref = [sana.linattn_fwd(*ins[t], block_len=ws_[t].block_len or None) for t in range(2)]
    torch.cuda.synchronize()
    results, errors = [[], []], []

    def worker(t):
        try:
            st = torch.cuda.Stream()
            with torch.cuda.stream(st):
                for _ in range(20):
                    results[t].append(sana.linattn_fwd(*ins[t], block_len=ws_[t].block_len or None, stream=st))
            st.synchronize()
        except Exception as e:   # noqa: BLE001 - reported below
            errors.append(e)

    threads = [threading.Thread(target=worker, args=(t,)) for t in range(2)]
    for th in threads:
        th.start()
    for th in threads:
        th.join()
    assert not errors, errors
    for t in range(2):
        assert len(results[t]) == 20 and all(torch.equal(r, ref[t]) for r in results[t])
