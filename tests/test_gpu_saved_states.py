"""GPU tests of the training-step pair sana_linattn_fwd_save_states /
sana_linattn_bwd_from_states: the forward's output is bitwise the plain
forward's, its saved per-block states match the fp64 oracle's states, and the
backward from those states is bitwise the backward that rebuilds them (and so
meets the oracle's backward bar, checked at full size too)."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from hip_helpers import compare, to_device
from test_gpu_backward import case, check

pytestmark = pytest.mark.gpu

DT = {workloads.DT_F32: torch.float32, workloads.DT_BF16: torch.bfloat16, workloads.DT_F16: torch.float16}


@pytest.fixture(autouse=True)
def _announce(request):
    print(f"\n[gpu] {request.node.name}", flush=True)


def step(q, k, v, g, block_len, eps, grad_t, out_t=torch.float32):
    """Forward with saved states, then the backward from them; also the plain
    forward and the rebuilding backward on the same device inputs."""
    import diffusion_transformer_relu_amd as sana
    B, N, H, D = q.shape
    L = block_len or 0
    states = torch.empty(sana.sana_linattn_states_bytes(B, H, N, D, L) // 4, dtype=torch.float32, device="cuda:0")
    ws = torch.empty(max(sana.sana_linattn_workspace_bytes(B, H, N, D, L),
                         sana.sana_linattn_bwd_workspace_bytes(B, H, N, D, L), 1), dtype=torch.uint8, device="cuda:0")
    out = torch.empty(q.shape, dtype=out_t, device="cuda:0")
    sana.sana_linattn_fwd_save_states(q, k, v, out, states, ws, block_len=L, eps=eps)
    grads = [torch.empty(q.shape, dtype=grad_t, device="cuda:0") for _ in range(3)]
    sana.sana_linattn_bwd_from_states(q, k, v, g, states, *grads, ws, block_len=L, eps=eps)
    plain = sana.linattn_fwd(q, k, v, eps=eps, out_dtype=out_t, block_len=block_len or None)
    rebuilt = sana.linattn_bwd(q, k, v, g, eps=eps, grad_dtype=grad_t, block_len=block_len or None)
    torch.cuda.synchronize()
    return out, states, grads, plain, rebuilt


def bits(t):
    return t.view(torch.int16) if t.element_size() == 2 else t.view(torch.int32)


CASES = [
    workloads.Workload("ss_B2_N1000_H3_bf16", 2, 1000, 3, 32, workloads.DT_BF16, seed=401),
    workloads.Workload("ss_B2_N1000_H3_L128_bf16", 2, 1000, 3, 32, workloads.DT_BF16, seed=402, block_len=128),
    workloads.Workload("ss_B1_N777_H5_L100_f32", 1, 777, 5, 32, workloads.DT_F32, seed=403, block_len=100),
    workloads.Workload("ss_B1_N1024_H4_L256_f16", 1, 1024, 4, 32, workloads.DT_F16, seed=404, block_len=256),
    workloads.Workload("ss_d16_B2_N1000_H7_L300_bf16", 2, 1000, 7, 16, workloads.DT_BF16, seed=405, block_len=300),
    workloads.Workload("ss_d64_B1_N4097_H3_L1024_bf16", 1, 4097, 3, 64, workloads.DT_BF16, seed=406, block_len=1024),
    workloads.Workload("ss_B1_N1_H1_bf16", 1, 1, 1, 32, workloads.DT_BF16, seed=407),
]


@pytest.mark.parametrize("w", CASES, ids=lambda w: w.name)
def test_saved_states_match_oracle_and_give_the_same_bits(w):
    q_np, k_np, v_np = workloads.make_inputs(w)
    g_np = workloads.make_dout(w)
    want, st_want = oracle.linattn_fwd(q_np, k_np, v_np, block_len=w.block_len, eps=w.eps, return_states=True)
    q, k, v, g = (to_device(a) for a in (q_np, k_np, v_np, g_np))
    grad_t = DT[w.in_dtype]
    out, states, grads, plain, rebuilt = step(q, k, v, g, w.block_len, w.eps, grad_t)
    compare(out.cpu().double().numpy(), want, v_np, False, w.name)
    assert torch.equal(bits(out), bits(plain))
    got_st = states.view(st_want.shape).cpu().double().numpy()
    assert np.max(np.abs(got_st - st_want)) <= 1e-5 * max(np.max(np.abs(st_want)), 1e-30), w.name
    for a, b in zip(grads, rebuilt):
        assert torch.equal(bits(a), bits(b)), w.name


@pytest.mark.parametrize("w", [workloads.HEADLINE, workloads.BLOCK_CAUSAL], ids=lambda w: w.name)
def test_full_size_training_step(w):
    """The 4096px shape and the 16 x 1024 video shape: the backward from saved
    states against the oracle's backward (bf16 gradients), bitwise the
    rebuilding backward."""
    (q_np, k_np, v_np, g_np), want = case(w, workloads.DT_BF16)
    q, k, v, g = (to_device(a) for a in (q_np, k_np, v_np, g_np))
    out, states, grads, plain, rebuilt = step(q, k, v, g, w.block_len, w.eps, torch.bfloat16)
    assert torch.equal(bits(out), bits(plain))
    check(grads, want, torch.bfloat16, w.name + "/from_states")
    for a, b in zip(grads, rebuilt):
        assert torch.equal(bits(a), bits(b)), w.name
