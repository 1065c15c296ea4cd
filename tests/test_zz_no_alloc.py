"""The no-allocation forward (sana_linattn_fwd_noalloc, the library's static
device scratch in place of a workspace) against sana_linattn_fwd on the same
inputs: two calls in a row, the second smaller, so the second runs on the
scratch contents the first left behind.  Same kernels and decomposition, so
the outputs must be the same bytes; both also meet the oracle bar."""
import numpy as np
import pytest
import torch

import workloads
from hip_helpers import compare, inputs_and_oracle, to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _announce(request):
    print(f"\n[gpu] {request.node.name}", flush=True)


@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16], ids=["f32out", "bf16out"])
def test_noalloc_matches_workspace_forward(out_dtype):
    import diffusion_transformer_relu_amd as sana
    cases = [workloads.HEADLINE,   # 4.4 MB of scratch
             workloads.with_shape(workloads.S600M_1024, B=1, N=777, H=5, name="noalloc_small")]
    for w in cases:
        (q, k, v), want = inputs_and_oracle(w)
        qd, kd, vd = to_device(q), to_device(k), to_device(v)
        B, N, H, D = qd.shape
        ref = torch.empty((B, N, H, D), dtype=out_dtype, device="cuda:0")
        ws = torch.empty(sana.sana_linattn_workspace_bytes(B, H, N, D, 0), dtype=torch.uint8, device="cuda:0")
        sana.sana_linattn_fwd(qd, kd, vd, ref, ws, eps=w.eps)
        got = torch.full((B, N, H, D), float("nan"), dtype=out_dtype, device="cuda:0")
        sana.sana_linattn_fwd_noalloc(qd, kd, vd, got, eps=w.eps)
        torch.cuda.synchronize()
        assert torch.equal(got.view(torch.uint8), ref.view(torch.uint8)), w.name
        compare(got.float().cpu().double().numpy(), want, v, out_dtype == torch.bfloat16, w.name)


def test_noalloc_on_a_side_stream_and_empty_problem():
    import diffusion_transformer_relu_amd as sana
    w = workloads.with_shape(workloads.BLOCK_CAUSAL, N=1500, H=3, block_len=0, name="noalloc_stream")
    (q, k, v), want = inputs_and_oracle(w)
    qd, kd, vd = to_device(q), to_device(k), to_device(v)
    out = torch.empty(qd.shape, dtype=torch.float32, device="cuda:0")
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        sana.sana_linattn_fwd_noalloc(qd, kd, vd, out, eps=w.eps, stream=s)
    s.synchronize()
    compare(out.double().cpu().numpy(), want, v, False, w.name)
    empty = torch.empty((1, 0, 3, 32), dtype=torch.bfloat16, device="cuda:0")
    sana.sana_linattn_fwd_noalloc(empty, empty, empty, torch.empty((1, 0, 3, 32), device="cuda:0"))
