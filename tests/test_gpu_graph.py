"""Graph capture: every entry point enqueues kernels only (no allocation,
memset or synchronisation, the workspace is the caller's), so a caller can
record the calls in a HIP graph.  Each replay, with new inputs copied into the
recorded buffers and unrelated eager work in between, must give the bytes of
the same calls made eagerly."""
import pytest
import torch

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _announce(request):
    print(f"\n[gpu] {request.node.name}", flush=True)


def test_graph_replays_match_eager():
    import diffusion_transformer_relu_amd as sana
    dev = "cuda:0"
    B, N, H, D, L = 1, 3000, 6, 32, 512
    gen = torch.Generator(device=dev).manual_seed(7)

    def rnd():
        return torch.randn(B, N, H, D, device=dev, generator=gen).to(torch.bfloat16)

    ins = [rnd() for _ in range(7)]            # q, k, v, dout, q_t, k_t, v_t (recorded buffers)
    ws_bytes = max(sana.sana_linattn_workspace_bytes(B, H, N, D, 0),
                   sana.sana_linattn_workspace_bytes(B, H, N, D, L),
                   sana.sana_linattn_bwd_workspace_bytes(B, H, N, D, 0),
                   sana.sana_linattn_jvp_workspace_bytes(B, H, N, D, 0))

    def buffers():
        f32 = lambda: torch.empty(B, N, H, D, dtype=torch.float32, device=dev)   # noqa: E731
        b16 = lambda: torch.empty(B, N, H, D, dtype=torch.bfloat16, device=dev)  # noqa: E731
        return {"fwd": f32(), "fwd_bf16": b16(), "bc": f32(), "dq": b16(), "dk": b16(), "dv": b16(),
                "jo": f32(), "jt": f32(), "ws": torch.empty(ws_bytes, dtype=torch.uint8, device=dev)}

    def run(o):
        q, k, v, g, qt, kt, vt = ins
        sana.sana_linattn_fwd(q, k, v, o["fwd"], o["ws"])
        sana.sana_linattn_fwd(q, k, v, o["fwd_bf16"], o["ws"])
        sana.sana_linattn_blockcausal_fwd(q, k, v, o["bc"], o["ws"], L)
        sana.sana_linattn_bwd(q, k, v, g, o["dq"], o["dk"], o["dv"], o["ws"])
        sana.sana_linattn_jvp(q, k, v, qt, kt, vt, o["jo"], o["jt"], o["ws"])

    rec, ref = buffers(), buffers()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):   # warm-up outside the capture
        run(rec)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()

    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        run(rec)

    for rep in range(3):
        for t in ins:                # new inputs in the recorded buffers
            t.copy_(rnd())
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        x = torch.randn(512, 512, device=dev, generator=gen)   # unrelated eager work
        _ = (x @ x).sum().item()
        run(ref)                     # the same calls, eagerly, into other buffers
        torch.cuda.synchronize()
        for name in ("fwd", "fwd_bf16", "bc", "dq", "dk", "dv", "jo", "jt"):
            a, b = rec[name], ref[name]
            assert torch.equal(a.view(torch.int16) if a.dtype == torch.bfloat16 else a.view(torch.int32),
                               b.view(torch.int16) if b.dtype == torch.bfloat16 else b.view(torch.int32)), (rep, name)
        assert torch.isfinite(rec["fwd"]).all()
