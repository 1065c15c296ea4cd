"""C-ABI checks that need no GPU: the library loads, exports every entry point
include/sana_linattn.h declares, and rejects bad arguments before it touches
the device (no call here reaches a kernel launch)."""
import ctypes
import os
import re

import pytest

import diffusion_transformer_relu_amd as sana

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = [os.path.join(ROOT, "include", f) for f in os.listdir(os.path.join(ROOT, "include")) if f.endswith(".h")]


def declared_functions():
    names = []
    for h in HEADERS:
        src = open(h).read()
        names += re.findall(r"SANA_API\s+[\w\s\*]+?\b(sana_\w+)\s*\(", src)
    return names


def test_every_declared_symbol_is_exported_and_bound():
    names = declared_functions()
    assert len(names) == 18, names
    for n in names:
        assert hasattr(sana.lib, n), n           # resolves in the shared library
        assert n in sana._SIGNATURES, n          # and the binding declares its signature
        assert hasattr(sana, n), n               # and exposes a function of the same name


def test_version_and_status_strings():
    assert sana.sana_linattn_abi_version() == 1
    for s in range(8):
        assert sana.sana_linattn_status_string(s) not in ("", "unknown status")
    assert sana.sana_linattn_status_string(99) == "unknown status"
    assert sana.sana_linattn_status_string(-1) == "unknown status"


def test_other_head_dims():
    assert sana.sana_linattn_plan_info(sana.SANA_DT_BF16, 1, 8, 256, 64, 0)["mfma"] == 1   # pairs of 32-feature halves
    assert sana.sana_linattn_plan_info(sana.SANA_DT_F16, 1, 8, 256, 64, 0)["mfma"] == 1
    assert sana.sana_linattn_plan_info(sana.SANA_DT_BF16, 1, 8, 256, 16, 0)["mfma"] == 1   # two heads per 32 features
    assert sana.sana_linattn_plan_info(sana.SANA_DT_F32, 1, 8, 256, 16, 0)["mfma"] == 1
    w16, w32, w64 = (sana.sana_linattn_workspace_bytes(1, 8, 4096, d, 0) for d in (16, 32, 64))
    assert w16 < w32 < w64
    for d in (8, 48, 128):
        assert sana.lib.sana_linattn_workspace_bytes(1, 8, 4096, d, 0, ctypes.byref(ctypes.c_size_t())) == \
            sana.SANA_ERR_UNSUPPORTED
    for d in (16, 64):   # the backward and the forward-mode derivative take every head dim
        jw = sana.sana_linattn_jvp_workspace_bytes(1, 8, 4096, d, 0)
        assert jw >= 2 * 8 * d * (d + 1) * 4   # one state and one tangent state per head
        bw = sana.sana_linattn_bwd_workspace_bytes(1, 8, 4096, d, 0)
        assert bw >= 2 * 8 * d * (d + 1) * 4   # the forward's state and one gradient state per head
    for f in (sana.lib.sana_linattn_bwd_workspace_bytes, sana.lib.sana_linattn_jvp_workspace_bytes):
        assert f(1, 8, 4096, 48, 0, ctypes.byref(ctypes.c_size_t())) == sana.SANA_ERR_UNSUPPORTED


def test_workspace_and_plan_queries():
    ws = sana.sana_linattn_workspace_bytes(1, 70, 16384, 32, 0)
    assert ws > 0 and ws % 256 == 0
    assert sana.sana_linattn_workspace_bytes(1, 70, 16384, 32, 1024) > ws   # one state per block
    assert sana.sana_linattn_workspace_bytes(1, 70, 16384, 32, 16384) == ws  # block_len >= N
    assert sana.sana_linattn_workspace_bytes(0, 70, 16384, 32, 0) == 0
    assert sana.sana_linattn_workspace_bytes(1, 70, 0, 32, 0) == 0
    info = sana.sana_linattn_plan_info(sana.SANA_DT_BF16, 1, 70, 16384, 32, 0)
    assert info["mfma"] == 1 and info["chunk_tokens"] % 64 == 0 and info["apply_tokens"] % 64 == 0
    assert info["num_chunks"] * info["chunk_tokens"] >= 16384
    assert sana.sana_linattn_plan_info(sana.SANA_DT_F32, 1, 2, 256, 32, 0)["mfma"] == 1   # fp32 in: split terms
    assert sana.sana_linattn_plan_info(sana.SANA_DT_F32, 1, 2, 256, 64, 0)["mfma"] == 1
    f16 = sana.sana_linattn_plan_info(sana.SANA_DT_F16, 1, 70, 16384, 32, 0)
    assert f16["mfma"] == 1 and f16["apply_tokens"] >= info["apply_tokens"]   # fp16 apply: 4 work-groups per CU
    bc = sana.sana_linattn_plan_info(sana.SANA_DT_BF16, 1, 70, 16384, 32, 1000)
    assert bc["chunk_tokens"] <= 1024 and bc["num_chunks"] % 17 == 0        # chunks never cross blocks


def test_tuning_environment(monkeypatch):
    monkeypatch.setenv("SANA_LINATTN_CHUNK", "300")
    monkeypatch.setenv("SANA_LINATTN_APPLY_TILE", "100")
    info = sana.sana_linattn_plan_info(sana.SANA_DT_BF16, 1, 70, 16384, 32, 0)
    assert info["chunk_tokens"] == 320 and info["apply_tokens"] == 128
    monkeypatch.setenv("SANA_LINATTN_PATH", "valu")
    assert sana.sana_linattn_plan_info(sana.SANA_DT_BF16, 1, 70, 16384, 32, 0)["mfma"] == 0
    monkeypatch.setenv("SANA_LINATTN_CHUNK", "junk")
    assert sana.sana_linattn_plan_info(sana.SANA_DT_BF16, 1, 70, 16384, 32, 0)["chunk_tokens"] % 64 == 0


@pytest.mark.parametrize("args,code", [
    ((1, 70, 16384, 31, 0), sana.SANA_ERR_UNSUPPORTED),
    ((1, 70, 16384, 128, 0), sana.SANA_ERR_UNSUPPORTED),
    ((1, 70, 16384, 0, 0), sana.SANA_ERR_INVALID_ARG),
    ((-1, 70, 16384, 32, 0), sana.SANA_ERR_INVALID_ARG),
    ((1, -70, 16384, 32, 0), sana.SANA_ERR_INVALID_ARG),
    ((1, 70, -5, 32, 0), sana.SANA_ERR_INVALID_ARG),
    ((1, 70, 16384, 32, -1), sana.SANA_ERR_INVALID_ARG),
    ((1, 70, (1 << 30) + 1, 32, 0), sana.SANA_ERR_UNSUPPORTED),
])
def test_workspace_query_errors(args, code):
    out = ctypes.c_size_t(0)
    assert sana.lib.sana_linattn_workspace_bytes(*args, ctypes.byref(out)) == code
    assert sana.lib.sana_linattn_workspace_bytes(1, 1, 1, 32, 0, None) == sana.SANA_ERR_INVALID_ARG


# Fake, never-dereferenced addresses: every call below fails a check before any launch.
A = 1 << 32                 # 16- and 256-byte aligned
MB = 1 << 20


def fwd(q=A, k=A + 64 * MB, v=A + 128 * MB, out=A + 192 * MB, in_dt=1, out_dt=0, B=1, H=2, N=256,
        D=32, eps=1e-15, ws=A + 512 * MB, ws_bytes=1 << 30, stream=None):
    return sana.lib.sana_linattn_fwd(q, k, v, out, in_dt, out_dt, B, H, N, D, eps, ws, ws_bytes, stream)


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), sana.SANA_ERR_INVALID_ARG),
    (dict(k=None), sana.SANA_ERR_INVALID_ARG),
    (dict(v=None), sana.SANA_ERR_INVALID_ARG),
    (dict(out=None), sana.SANA_ERR_INVALID_ARG),
    (dict(ws=None), sana.SANA_ERR_INVALID_ARG),
    (dict(in_dt=3), sana.SANA_ERR_INVALID_ARG),
    (dict(out_dt=-1), sana.SANA_ERR_INVALID_ARG),
    (dict(out_dt=3), sana.SANA_ERR_INVALID_ARG),
    (dict(D=48), sana.SANA_ERR_UNSUPPORTED),
    (dict(D=16, ws_bytes=1024), sana.SANA_ERR_WORKSPACE),   # head dims 16 and 64: their own workspace sizes
    (dict(D=64, ws_bytes=1024), sana.SANA_ERR_WORKSPACE),
    (dict(B=-1), sana.SANA_ERR_INVALID_ARG),
    (dict(eps=float("nan")), sana.SANA_ERR_INVALID_ARG),
    (dict(eps=float("inf")), sana.SANA_ERR_INVALID_ARG),
    (dict(eps=-1e-6), sana.SANA_ERR_INVALID_ARG),
    (dict(q=A + 2), sana.SANA_ERR_ALIGNMENT),
    (dict(out=A + 192 * MB + 8), sana.SANA_ERR_ALIGNMENT),
    (dict(ws=A + 512 * MB + 16), sana.SANA_ERR_ALIGNMENT),
    (dict(out=A), sana.SANA_ERR_ALIAS),                         # out == q
    (dict(out=A + 64 * MB + 16 * 1024), sana.SANA_ERR_ALIAS),   # out overlaps k's tail
    (dict(ws=A + 128 * MB), sana.SANA_ERR_ALIAS),               # workspace == v
    (dict(ws_bytes=1024), sana.SANA_ERR_WORKSPACE),
])
def test_forward_argument_errors(kw, code):
    assert fwd(**kw) == code


def test_empty_problems_succeed_without_touching_pointers():
    for B, H, N in ((0, 2, 256), (1, 0, 256), (1, 2, 0)):
        assert fwd(q=None, k=None, v=None, out=None, ws=None, ws_bytes=0, B=B, H=H, N=N) == sana.SANA_OK


def test_blockcausal_and_stage_argument_errors():
    args = (A, A + 64 * MB, A + 128 * MB, A + 192 * MB, 1, 0, 1, 2, 256, 32)
    tail = (1e-15, A + 512 * MB, 1 << 30, None)
    for L in (0, -3):
        assert sana.lib.sana_linattn_blockcausal_fwd(*args, L, *tail) == sana.SANA_ERR_INVALID_ARG
    assert sana.lib.sana_linattn_blockcausal_fwd(*args, 64, 1e-15, A + 512 * MB, 16, None) == \
        sana.SANA_ERR_WORKSPACE
    for stages in (0, 8, -1, 15):
        assert sana.lib.sana_linattn_fwd_stages(*args, 0, *tail, stages) == sana.SANA_ERR_INVALID_ARG
    assert sana.lib.sana_linattn_fwd_stages(*args, -1, *tail, 7) == sana.SANA_ERR_INVALID_ARG


def test_one_hip_runtime_in_the_process():
    # The library must bind to the HIP runtime torch brings in, whatever the
    # import order: with two runtimes (or torch on the system one) torch's GPU
    # calls fail.
    import subprocess
    import sys
    code = ("import diffusion_transformer_relu_amd, torch, os\n"
            "maps = open('/proc/self/maps').read().split('\\n')\n"
            "paths = sorted({l.split()[-1] for l in maps if 'libamdhip64' in l})\n"
            "bundled = os.path.join(os.path.dirname(torch.__file__), 'lib', 'libamdhip64.so')\n"
            "print(len(paths), int(not os.path.exists(bundled) or paths == [bundled]), paths)\n")
    res = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, cwd=ROOT, timeout=300)
    assert res.returncode == 0, res.stderr
    n, is_torch_runtime = res.stdout.split()[:2]
    assert n == "1" and is_torch_runtime == "1", res.stdout


def test_stream_argument_errors():
    S0 = A + 700 * MB
    args = (A, A + 64 * MB, A + 128 * MB, A + 192 * MB, 1, 0, 1, 2, 256, 32)
    ws = (A + 512 * MB, 1 << 30, None)
    f = sana.lib.sana_linattn_blockcausal_stream_fwd
    assert f(*args, 0, 1e-15, S0, S0, *ws) == sana.SANA_ERR_INVALID_ARG          # block_len < 1
    assert f(*args, 64, 1e-15, S0 + 2, None, *ws) == sana.SANA_ERR_ALIGNMENT
    assert f(*args, 64, 1e-15, None, S0 + 1, *ws) == sana.SANA_ERR_ALIGNMENT
    assert f(*args, 64, 1e-15, None, A, *ws) == sana.SANA_ERR_ALIAS               # state_out = q
    assert f(*args, 64, 1e-15, A + 192 * MB, None, *ws) == sana.SANA_ERR_ALIAS    # state_in = out
    assert f(*args, 64, 1e-15, S0, S0 + 64, *ws) == sana.SANA_ERR_ALIAS           # partly overlapping states
    # in place (state_out == state_in) is allowed: the call gets as far as the workspace check
    assert f(*args, 64, 1e-15, S0, S0, A + 512 * MB, 16, None) == sana.SANA_ERR_WORKSPACE


def test_strided_argument_errors():
    H, N, D = 2, 256, 32
    dense = [N * H * D, H * D] * 4
    f = sana.lib.sana_linattn_fwd_strided
    args = (A, A + 64 * MB, A + 128 * MB, A + 192 * MB, 1, 0, 1, H, N, D, 0, 1e-15)
    tail = (A + 512 * MB, 16, None)     # workspace too small: a passing call stops there, never launches
    st = lambda xs: (ctypes.c_int64 * 8)(*xs)
    assert f(*args, st(dense), *tail) == sana.SANA_ERR_WORKSPACE
    assert f(*args, None, *tail) == sana.SANA_ERR_INVALID_ARG
    assert f(*args[:10], -1, 1e-15, st(dense), *tail) == sana.SANA_ERR_INVALID_ARG
    assert f(*args, st([-64] + dense[1:]), *tail) == sana.SANA_ERR_INVALID_ARG
    assert f(*args, st(dense[:1] + [H * D + 4] + dense[2:]), *tail) == sana.SANA_ERR_ALIGNMENT   # 8-byte rows
    # fused qkv slices: token stride 3*H*D for q, k, v is fine
    fused = [N * 3 * H * D, 3 * H * D] * 3 + [N * H * D, H * D]
    assert f(*args, st(fused), *tail) == sana.SANA_ERR_WORKSPACE
    # output rows overlapping each other
    assert f(*args, st(dense[:6] + [N * H * D, H * D // 2]), *tail) == sana.SANA_ERR_ALIAS
    # [N, B, H, D] output layout (batch stride H*D, token stride B*H*D) is disjoint
    args2 = args[:6] + (2,) + args[7:]
    assert f(*args2, st(dense[:6] + [H * D, 2 * H * D]), *tail) == sana.SANA_ERR_WORKSPACE
    assert f(*args2, st(dense[:6] + [H * D, H * D]), *tail) == sana.SANA_ERR_ALIAS


def bwd(q=A, k=A + 64 * MB, v=A + 128 * MB, g=A + 192 * MB, dq=A + 256 * MB, dk=A + 320 * MB, dv=A + 384 * MB,
        in_dt=1, g_dt=1, gr_dt=1, B=1, H=2, N=256, D=32, L=0, eps=1e-15, ws=A + 512 * MB, ws_bytes=16):
    # ws_bytes 16 is too small: a call whose other checks pass stops with WORKSPACE, never launching
    return sana.lib.sana_linattn_bwd(q, k, v, g, dq, dk, dv, in_dt, g_dt, gr_dt, B, H, N, D, L, eps, ws,
                                     ws_bytes, None)


@pytest.mark.parametrize("kw,code", [
    ({}, sana.SANA_ERR_WORKSPACE),
    (dict(L=64), sana.SANA_ERR_WORKSPACE),
    (dict(in_dt=0, g_dt=0, gr_dt=0), sana.SANA_ERR_WORKSPACE),
    (dict(in_dt=2, g_dt=2, gr_dt=2), sana.SANA_ERR_WORKSPACE),
    (dict(L=-1), sana.SANA_ERR_INVALID_ARG),
    (dict(g=None), sana.SANA_ERR_INVALID_ARG),
    (dict(dv=None), sana.SANA_ERR_INVALID_ARG),
    (dict(ws=None), sana.SANA_ERR_INVALID_ARG),
    (dict(g_dt=3), sana.SANA_ERR_INVALID_ARG),
    (dict(gr_dt=-1), sana.SANA_ERR_INVALID_ARG),
    (dict(in_dt=5), sana.SANA_ERR_INVALID_ARG),
    (dict(D=48), sana.SANA_ERR_UNSUPPORTED),
    (dict(eps=float("nan")), sana.SANA_ERR_INVALID_ARG),
    (dict(dk=A + 320 * MB + 8), sana.SANA_ERR_ALIGNMENT),
    (dict(g=A + 192 * MB + 2), sana.SANA_ERR_ALIGNMENT),
    (dict(dq=A), sana.SANA_ERR_ALIAS),                  # dq == q
    (dict(dk=A + 192 * MB), sana.SANA_ERR_ALIAS),       # dk == dout
    (dict(dv=A + 256 * MB), sana.SANA_ERR_ALIAS),       # dv == dq
    (dict(ws=A + 384 * MB), sana.SANA_ERR_ALIAS),       # workspace == dv
    (dict(B=0), sana.SANA_OK),
    (dict(N=0, q=None, ws=None), sana.SANA_OK),
])
def test_backward_argument_errors(kw, code):
    assert bwd(**kw) == code


def test_backward_workspace_query():
    fw = sana.sana_linattn_workspace_bytes(1, 70, 16384, 32, 0)
    bw = sana.sana_linattn_bwd_workspace_bytes(1, 70, 16384, 32, 0)
    assert bw > fw and bw % 256 == 0
    assert sana.sana_linattn_bwd_workspace_bytes(1, 70, 16384, 32, 1024) > bw
    assert sana.sana_linattn_bwd_workspace_bytes(0, 70, 16384, 32, 0) == 0
    assert sana.lib.sana_linattn_bwd_workspace_bytes(1, 1, 1, 32, 0, None) == sana.SANA_ERR_INVALID_ARG


def jvp(q=A, k=A + 64 * MB, v=A + 128 * MB, qt=A + 192 * MB, kt=A + 256 * MB, vt=A + 320 * MB, out=A + 384 * MB,
        outt=A + 448 * MB, in_dt=1, out_dt=0, B=1, H=2, N=256, D=32, L=0, eps=1e-15, ws=A + 512 * MB, ws_bytes=16):
    return sana.lib.sana_linattn_jvp(q, k, v, qt, kt, vt, out, outt, in_dt, out_dt, B, H, N, D, L, eps, ws,
                                     ws_bytes, None)


@pytest.mark.parametrize("kw,code", [
    ({}, sana.SANA_ERR_WORKSPACE),
    (dict(L=64, in_dt=2, out_dt=2), sana.SANA_ERR_WORKSPACE),
    (dict(in_dt=0), sana.SANA_ERR_WORKSPACE),
    (dict(L=-1), sana.SANA_ERR_INVALID_ARG),
    (dict(kt=None), sana.SANA_ERR_INVALID_ARG),
    (dict(outt=None), sana.SANA_ERR_INVALID_ARG),
    (dict(in_dt=3), sana.SANA_ERR_INVALID_ARG),
    (dict(D=48), sana.SANA_ERR_UNSUPPORTED),
    (dict(eps=-1.0), sana.SANA_ERR_INVALID_ARG),
    (dict(vt=A + 320 * MB + 4), sana.SANA_ERR_ALIGNMENT),
    (dict(outt=A + 384 * MB), sana.SANA_ERR_ALIAS),     # out_t == out
    (dict(out=A + 256 * MB), sana.SANA_ERR_ALIAS),      # out == k_t
    (dict(ws=A + 448 * MB), sana.SANA_ERR_ALIAS),       # workspace == out_t
    (dict(H=0), sana.SANA_OK),
])
def test_jvp_argument_errors(kw, code):
    assert jvp(**kw) == code


def test_jvp_workspace_query():
    # a state and a tangent state per head: twice the partials and states of
    # the bf16 forward's decomposition (16 chunks of 4224 B per head, one state)
    jw = sana.sana_linattn_jvp_workspace_bytes(1, 70, 16384, 32, 0)
    assert jw >= 2 * 70 * (16 + 1) * 4224 and jw % 256 == 0
    assert jw > sana.sana_linattn_workspace_bytes(1, 70, 16384, 32, 0)
    assert sana.lib.sana_linattn_jvp_workspace_bytes(1, 1, 1, 32, 0, None) == sana.SANA_ERR_INVALID_ARG


def test_noalloc_entry_point_rejects_problems_beyond_its_scratch():
    """The no-allocation forward checks its sizes before any HIP call: a problem
    whose workspace exceeds the static scratch is refused with SCRATCH, bad
    arguments with the usual codes, an empty problem succeeds (fake, never
    dereferenced pointers)."""
    fake = ctypes.c_void_p(1 << 20)
    f = sana.lib.sana_linattn_fwd_noalloc
    B, H, N, D = 64, 70, 1024, 32
    assert sana.sana_linattn_workspace_bytes(B, H, N, D, 0) > sana.SANA_LINATTN_SCRATCH_BYTES
    assert f(fake, fake, fake, fake, sana.SANA_DT_BF16, sana.SANA_DT_F32, B, H, N, D, 1e-15, None) == \
        sana.SANA_ERR_SCRATCH
    assert "scratch" in sana.sana_linattn_status_string(sana.SANA_ERR_SCRATCH)
    assert f(fake, fake, fake, fake, sana.SANA_DT_BF16, sana.SANA_DT_F32, 1, 70, 16384, 48, 1e-15, None) == \
        sana.SANA_ERR_UNSUPPORTED
    assert f(fake, fake, fake, fake, 9, sana.SANA_DT_F32, 1, 70, 16384, 32, 1e-15, None) == sana.SANA_ERR_INVALID_ARG
    assert f(None, None, None, None, sana.SANA_DT_BF16, sana.SANA_DT_F32, 1, 0, 16384, 32, 1e-15, None) == \
        sana.SANA_OK
    # the headline shape fits
    assert sana.sana_linattn_workspace_bytes(1, 70, 16384, 32, 0) <= sana.SANA_LINATTN_SCRATCH_BYTES


def test_qknorm_argument_errors():
    """sana_linattn_fwd_qknorm checks norm_eps (finite, > 0 whenever a gamma is
    given), the gammas' alignment and overlap, and the usual arguments, before
    anything is enqueued (fake, never dereferenced pointers)."""
    f = sana.lib.sana_linattn_fwd_qknorm
    base = 1 << 30
    q, k, v, out, ws = (ctypes.c_void_p(base + i * (1 << 26)) for i in range(5))
    gq, gk = ctypes.c_void_p(base + 5 * (1 << 26)), ctypes.c_void_p(base + 6 * (1 << 26))
    B, H, N, D = 1, 4, 1024, 32
    wsb = sana.sana_linattn_workspace_bytes(B, H, N, D, 0)

    def call(gamma_q=gq, gamma_k=gk, norm_eps=1e-6, o=out, block_len=0, eps=1e-15, dt=sana.SANA_DT_BF16, d=D,
             nbytes=wsb):
        return f(q, k, v, o, dt, sana.SANA_DT_F32, B, H, N, d, block_len, eps, gamma_q, gamma_k, norm_eps, None,
                 ws, nbytes, None)

    for bad in (0.0, -1e-6, float("nan"), float("inf")):
        assert call(norm_eps=bad) == sana.SANA_ERR_INVALID_ARG
        assert call(gamma_q=None, norm_eps=bad) == sana.SANA_ERR_INVALID_ARG
    assert call(norm_eps=0.0, gamma_q=None, gamma_k=None, nbytes=0) == sana.SANA_ERR_WORKSPACE   # no gamma: eps unused
    assert call(block_len=-1) == sana.SANA_ERR_INVALID_ARG
    assert call(eps=float("nan")) == sana.SANA_ERR_INVALID_ARG
    assert call(d=48) == sana.SANA_ERR_UNSUPPORTED
    assert call(gamma_k=ctypes.c_void_p(base + 6 * (1 << 26) + 2)) == sana.SANA_ERR_ALIGNMENT
    assert call(gamma_q=ctypes.c_void_p(out.value + 64)) == sana.SANA_ERR_ALIAS
    assert call(gamma_k=ctypes.c_void_p(ws.value)) == sana.SANA_ERR_ALIAS
    assert call(nbytes=wsb - 1) == sana.SANA_ERR_WORKSPACE
    # an empty problem succeeds without touching any pointer
    assert f(None, None, None, None, sana.SANA_DT_BF16, sana.SANA_DT_F32, 0, H, N, D, 0, 1e-15, None, None, 1e-6,
             None, None, 0, None) == sana.SANA_OK


def test_saved_states_size_and_argument_errors():
    """sana_linattn_states_bytes is B H NB D (D+1) 4; the save / from-states
    entry points reject a missing, misaligned or overlapping states buffer
    before anything is enqueued (fake, never dereferenced pointers)."""
    assert sana.sana_linattn_states_bytes(1, 70, 16384, 32, 0) == 70 * 32 * 33 * 4
    assert sana.sana_linattn_states_bytes(1, 70, 16384, 32, 1024) == 16 * 70 * 32 * 33 * 4
    assert sana.sana_linattn_states_bytes(2, 3, 1000, 64, 300) == 2 * 3 * 4 * 64 * 65 * 4
    assert sana.sana_linattn_states_bytes(0, 3, 1000, 16, 0) == 0
    assert sana.lib.sana_linattn_states_bytes(1, 3, 1000, 48, 0, ctypes.byref(ctypes.c_size_t())) == \
        sana.SANA_ERR_UNSUPPORTED
    base = 1 << 32
    q, k, v, out, ws, st = (base + i * (1 << 26) for i in range(6))
    B, H, N, D = 1, 4, 1024, 32
    wsb = sana.sana_linattn_workspace_bytes(B, H, N, D, 256)
    save = sana.lib.sana_linattn_fwd_save_states

    def fwd(states=st, o=out, L=256):
        return save(q, k, v, o, sana.SANA_DT_BF16, sana.SANA_DT_F32, B, H, N, D, L, 1e-15, states, ws, wsb, None)

    assert fwd(states=None) == sana.SANA_ERR_INVALID_ARG
    assert fwd(states=st + 2) == sana.SANA_ERR_ALIGNMENT
    assert fwd(states=out + 64) == sana.SANA_ERR_ALIAS
    assert fwd(states=ws) == sana.SANA_ERR_ALIAS
    assert fwd(L=-1) == sana.SANA_ERR_INVALID_ARG
    assert save(None, None, None, None, 1, 0, 0, H, N, D, 0, 1e-15, None, None, 0, None) == sana.SANA_OK
    bw = sana.lib.sana_linattn_bwd_from_states
    bwb = sana.sana_linattn_bwd_workspace_bytes(B, H, N, D, 256)
    dq, dk, dv, dout = (base + (6 + i) * (1 << 26) for i in range(4))

    def bwd(states=st, L=256, nbytes=bwb):
        return bw(q, k, v, dout, states, dq, dk, dv, 1, 1, 1, B, H, N, D, L, 1e-15, ws, nbytes, None)

    assert bwd(states=None) == sana.SANA_ERR_INVALID_ARG
    assert bwd(states=st + 1) == sana.SANA_ERR_ALIGNMENT
    assert bwd(states=dk + 128) == sana.SANA_ERR_ALIAS
    assert bwd(states=ws + 256) == sana.SANA_ERR_ALIAS
    assert bwd(nbytes=bwb - 1) == sana.SANA_ERR_WORKSPACE
