"""Python binding of the gfx950 LiteLA forward library (libsana_linattn.so).

Argument marshalling only: every step of the forward runs in the HIP kernels of
the shared library; PyTorch provides device memory and the stream.  The
functions below carry the names of the C entry points declared in
include/sana_linattn.h and raise SanaError on a non-zero status.  If the
library has not been built, importing this package raises ImportError: there
is no fallback implementation.
"""
from __future__ import annotations

import ctypes
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
# SANA_LINATTN_LIB selects another build of the same sources (the host
# sanitizer build, lib_san/)
LIB_PATH = os.environ.get("SANA_LINATTN_LIB") or os.path.join(_PKG, "lib", "libsana_linattn.so")

SANA_DT_F32 = 0
SANA_DT_BF16 = 1
SANA_DT_F16 = 2
SANA_OK = 0
SANA_ERR_INVALID_ARG = 1
SANA_ERR_UNSUPPORTED = 2
SANA_ERR_ALIGNMENT = 3
SANA_ERR_ALIAS = 4
SANA_ERR_WORKSPACE = 5
SANA_ERR_HIP = 6
SANA_ERR_SCRATCH = 7
SANA_LINATTN_SCRATCH_BYTES = 16 << 20
SANA_STAGE_STATE = 1
SANA_STAGE_MERGE = 2
SANA_STAGE_APPLY = 4
SANA_STAGE_ALL = 7

# name -> (restype, argtypes) of every exported C entry point
_P = ctypes.c_void_p
_I = ctypes.c_int
_SIGNATURES = {
    "sana_linattn_abi_version": (_I, []),
    "sana_linattn_status_string": (ctypes.c_char_p, [_I]),
    "sana_linattn_workspace_bytes": (_I, [_I, _I, _I, _I, _I, ctypes.POINTER(ctypes.c_size_t)]),
    "sana_linattn_plan_info": (_I, [_I, _I, _I, _I, _I, _I, ctypes.POINTER(_I), ctypes.POINTER(_I),
                                    ctypes.POINTER(_I), ctypes.POINTER(_I)]),
    "sana_linattn_fwd": (_I, [_P, _P, _P, _P, _I, _I, _I, _I, _I, _I, ctypes.c_float, _P,
                              ctypes.c_size_t, _P]),
    "sana_linattn_blockcausal_fwd": (_I, [_P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, ctypes.c_float,
                                          _P, ctypes.c_size_t, _P]),
    "sana_linattn_blockcausal_stream_fwd": (_I, [_P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, ctypes.c_float,
                                                 _P, _P, _P, ctypes.c_size_t, _P]),
    "sana_linattn_fwd_strided": (_I, [_P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, ctypes.c_float,
                                      ctypes.POINTER(ctypes.c_int64), _P, ctypes.c_size_t, _P]),
    "sana_linattn_fwd_qknorm": (_I, [_P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, ctypes.c_float, _P, _P,
                                     ctypes.c_float, ctypes.POINTER(ctypes.c_int64), _P, ctypes.c_size_t, _P]),
    "sana_linattn_fwd_stages": (_I, [_P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, ctypes.c_float, _P,
                                     ctypes.c_size_t, _P, _I]),
    "sana_linattn_bwd_workspace_bytes": (_I, [_I, _I, _I, _I, _I, ctypes.POINTER(ctypes.c_size_t)]),
    "sana_linattn_jvp_workspace_bytes": (_I, [_I, _I, _I, _I, _I, ctypes.POINTER(ctypes.c_size_t)]),
    "sana_linattn_jvp": (_I, [_P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, ctypes.c_float, _P,
                              ctypes.c_size_t, _P]),
    "sana_linattn_fwd_noalloc": (_I, [_P, _P, _P, _P, _I, _I, _I, _I, _I, _I, ctypes.c_float, _P]),
    "sana_linattn_states_bytes": (_I, [_I, _I, _I, _I, _I, ctypes.POINTER(ctypes.c_size_t)]),
    "sana_linattn_fwd_save_states": (_I, [_P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, ctypes.c_float, _P, _P,
                                          ctypes.c_size_t, _P]),
    "sana_linattn_bwd_from_states": (_I, [_P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _I,
                                          ctypes.c_float, _P, ctypes.c_size_t, _P]),
    "sana_linattn_bwd": (_I, [_P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _I, ctypes.c_float, _P,
                              ctypes.c_size_t, _P]),
}

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is missing: build it with `python -c 'import __graft_entry__ as g; "
                      f"g.build()'` (hipcc, gfx950)")

# torch ships its own HIP runtime under the same soname as the system one
# (libamdhip64.so.7).  Importing torch first makes this library bind to that
# already-loaded runtime, so device pointers and streams are shared with
# torch; loading the library first would pull in the system runtime and leave
# torch running on a mix of the two.
import torch  # noqa: E402,F401

lib = ctypes.CDLL(LIB_PATH)
for _name, (_res, _args) in _SIGNATURES.items():
    _fn = getattr(lib, _name)
    _fn.restype = _res
    _fn.argtypes = _args


class SanaError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {sana_linattn_status_string(status)} (status {status})")


def _check(status: int, where: str):
    if status != SANA_OK:
        raise SanaError(status, where)


def sana_linattn_abi_version() -> int:
    return lib.sana_linattn_abi_version()


def sana_linattn_status_string(status: int) -> str:
    return lib.sana_linattn_status_string(status).decode()


def sana_linattn_workspace_bytes(B: int, H: int, N: int, D: int, block_len: int = 0) -> int:
    out = ctypes.c_size_t(0)
    _check(lib.sana_linattn_workspace_bytes(B, H, N, D, block_len, ctypes.byref(out)),
           "sana_linattn_workspace_bytes")
    return out.value


def sana_linattn_plan_info(in_dtype: int, B: int, H: int, N: int, D: int, block_len: int = 0) -> dict:
    vals = [ctypes.c_int(0) for _ in range(4)]
    _check(lib.sana_linattn_plan_info(in_dtype, B, H, N, D, block_len, *[ctypes.byref(x) for x in vals]),
           "sana_linattn_plan_info")
    return dict(zip(("chunk_tokens", "num_chunks", "apply_tokens", "mfma"), (x.value for x in vals)))


# ------------------------------------------------------------------ torch marshalling
def _torch():
    import torch
    return torch


def dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.bfloat16:
        return SANA_DT_BF16
    if t.dtype == torch.float32:
        return SANA_DT_F32
    if t.dtype == torch.float16:
        return SANA_DT_F16
    raise TypeError(f"LiteLA tensors are bfloat16, float16 or float32, got {t.dtype}")


def _shape(q, k, v, out):
    for name, t in (("q", q), ("k", k), ("v", v), ("out", out)):
        if t.dim() != 4 or not t.is_contiguous() or not t.is_cuda:
            raise ValueError(f"{name} must be a contiguous 4-d [B, N, H, D] GPU tensor")
    if not (q.shape == k.shape == v.shape == out.shape):
        raise ValueError("q, k, v and out must share one [B, N, H, D] shape")
    if not (q.dtype == k.dtype == v.dtype):
        raise TypeError("q, k and v must share one dtype")
    B, N, H, D = q.shape
    return B, N, H, D


def _stream_handle(stream):
    torch = _torch()
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _torch_stream(stream):
    """The torch stream object for `stream` (None = the current stream, an int
    = a raw hipStream_t)."""
    torch = _torch()
    if stream is None:
        return torch.cuda.current_stream()
    if isinstance(stream, int):
        return torch.cuda.ExternalStream(stream)
    return stream


def sana_linattn_fwd(q, k, v, out, workspace, *, eps: float = 1e-15, stream=None):
    """Non-causal forward into `out` (torch tensors on the GPU; `workspace` a
    uint8 GPU tensor of at least sana_linattn_workspace_bytes bytes)."""
    B, N, H, D = _shape(q, k, v, out)
    _check(lib.sana_linattn_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), dtype_code(q),
                                dtype_code(out), B, H, N, D, eps, workspace.data_ptr(),
                                workspace.numel() * workspace.element_size(), _stream_handle(stream)),
           "sana_linattn_fwd")


def sana_linattn_fwd_noalloc(q, k, v, out, *, eps: float = 1e-15, stream=None):
    """Non-causal forward into `out` with the library's static device scratch
    (no workspace argument, nothing allocated)."""
    B, N, H, D = _shape(q, k, v, out)
    _check(lib.sana_linattn_fwd_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), dtype_code(q),
                                        dtype_code(out), B, H, N, D, eps, _stream_handle(stream)),
           "sana_linattn_fwd_noalloc")


def sana_linattn_blockcausal_fwd(q, k, v, out, workspace, block_len: int, *, eps: float = 1e-15,
                                 stream=None):
    """Block-causal forward into `out`; block_len >= 1 tokens per block."""
    B, N, H, D = _shape(q, k, v, out)
    _check(lib.sana_linattn_blockcausal_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                                            dtype_code(q), dtype_code(out), B, H, N, D, block_len, eps,
                                            workspace.data_ptr(),
                                            workspace.numel() * workspace.element_size(),
                                            _stream_handle(stream)),
           "sana_linattn_blockcausal_fwd")


def sana_linattn_blockcausal_stream_fwd(q, k, v, out, workspace, block_len: int, state_in=None,
                                        state_out=None, *, eps: float = 1e-15, stream=None):
    """Block-causal forward continuing a sequence: state_in / state_out are
    float32 [B, H, D, D+1] GPU tensors (or None) holding the carried state."""
    B, N, H, D = _shape(q, k, v, out)
    for name, t in (("state_in", state_in), ("state_out", state_out)):
        if t is not None and (not t.is_cuda or not t.is_contiguous() or t.dtype != _torch().float32
                              or tuple(t.shape) != (B, H, D, D + 1)):
            raise ValueError(f"{name} must be a contiguous float32 [B, H, D, D+1] GPU tensor")
    _check(lib.sana_linattn_blockcausal_stream_fwd(
        q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), dtype_code(q), dtype_code(out), B, H, N, D,
        block_len, eps, state_in.data_ptr() if state_in is not None else None,
        state_out.data_ptr() if state_out is not None else None, workspace.data_ptr(),
        workspace.numel() * workspace.element_size(), _stream_handle(stream)),
        "sana_linattn_blockcausal_stream_fwd")


def _view_shape(q, k, v, out):
    for name, t in (("q", q), ("k", k), ("v", v), ("out", out)):
        if t.dim() != 4 or not t.is_cuda or t.stride(3) != 1 or t.stride(2) != t.shape[3]:
            raise ValueError(f"{name} must be a 4-d [B, N, H, D] GPU view with contiguous heads")
    if not (q.shape == k.shape == v.shape == out.shape):
        raise ValueError("q, k, v and out must share one [B, N, H, D] shape")
    if not (q.dtype == k.dtype == v.dtype):
        raise TypeError("q, k and v must share one dtype")
    return tuple(q.shape)


def sana_linattn_fwd_strided(q, k, v, out, workspace, *, block_len: int = 0, eps: float = 1e-15,
                             stream=None):
    """Forward on [B, N, H, D] views with free batch/token strides (e.g. the
    q, k, v slices of one fused qkv projection), read in place."""
    B, N, H, D = _view_shape(q, k, v, out)
    st = (ctypes.c_int64 * 8)(q.stride(0), q.stride(1), k.stride(0), k.stride(1), v.stride(0), v.stride(1),
                              out.stride(0), out.stride(1))
    _check(lib.sana_linattn_fwd_strided(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), dtype_code(q),
                                        dtype_code(out), B, H, N, D, block_len, eps, st, workspace.data_ptr(),
                                        workspace.numel() * workspace.element_size(), _stream_handle(stream)),
           "sana_linattn_fwd_strided")


def sana_linattn_fwd_qknorm(q, k, v, out, workspace, gamma_q=None, gamma_k=None, *, norm_eps: float = 1e-6,
                            block_len: int = 0, eps: float = 1e-15, stream=None):
    """Forward with the qk_norm prologue on [B, N, H, D] views (free batch and
    token strides): gamma_q / gamma_k are contiguous float32 [H, D] GPU tensors,
    or None for no normalisation of that side."""
    B, N, H, D = _view_shape(q, k, v, out)
    for name, t in (("gamma_q", gamma_q), ("gamma_k", gamma_k)):
        if t is not None and (not t.is_cuda or not t.is_contiguous() or t.dtype != _torch().float32
                              or tuple(t.shape) != (H, D)):
            raise ValueError(f"{name} must be a contiguous float32 [H, D] GPU tensor")
    st = (ctypes.c_int64 * 8)(q.stride(0), q.stride(1), k.stride(0), k.stride(1), v.stride(0), v.stride(1),
                              out.stride(0), out.stride(1))
    _check(lib.sana_linattn_fwd_qknorm(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), dtype_code(q),
                                       dtype_code(out), B, H, N, D, block_len, eps,
                                       gamma_q.data_ptr() if gamma_q is not None else None,
                                       gamma_k.data_ptr() if gamma_k is not None else None, norm_eps, st,
                                       workspace.data_ptr(), workspace.numel() * workspace.element_size(),
                                       _stream_handle(stream)),
           "sana_linattn_fwd_qknorm")


def sana_linattn_fwd_stages(q, k, v, out, workspace, stages: int, *, block_len: int = 0,
                            eps: float = 1e-15, stream=None):
    """Runs the selected kernels (SANA_STAGE_* bits) of the forward."""
    B, N, H, D = _shape(q, k, v, out)
    _check(lib.sana_linattn_fwd_stages(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                                       dtype_code(q), dtype_code(out), B, H, N, D, block_len, eps,
                                       workspace.data_ptr(), workspace.numel() * workspace.element_size(),
                                       _stream_handle(stream), stages),
           "sana_linattn_fwd_stages")


def linattn_fwd(q, k, v, *, eps: float = 1e-15, out_dtype=None, block_len: int | None = None,
                gamma_q=None, gamma_k=None, norm_eps: float = 1e-6, stream=None):
    """Allocates `out` (float32 unless out_dtype is given) and the workspace with
    torch, then runs the non-causal (block_len None) or block-causal forward,
    with the qk_norm prologue when gamma_q or gamma_k is given.  Both buffers
    are allocated on the stream the kernels run on."""
    torch = _torch()
    s = _torch_stream(stream)
    with torch.cuda.stream(s):
        out = torch.empty(q.shape, dtype=out_dtype or torch.float32, device=q.device)
        B, N, H, D = q.shape
        ws = torch.empty(max(sana_linattn_workspace_bytes(B, H, N, D, block_len or 0), 1),
                         dtype=torch.uint8, device=q.device)
        if gamma_q is not None or gamma_k is not None:
            sana_linattn_fwd_qknorm(q, k, v, out, ws, gamma_q, gamma_k, norm_eps=norm_eps,
                                    block_len=block_len or 0, eps=eps, stream=s)
        elif not (q.is_contiguous() and k.is_contiguous() and v.is_contiguous()):
            sana_linattn_fwd_strided(q, k, v, out, ws, block_len=block_len or 0, eps=eps, stream=s)
        elif block_len is None:
            sana_linattn_fwd(q, k, v, out, ws, eps=eps, stream=s)
        else:
            sana_linattn_blockcausal_fwd(q, k, v, out, ws, block_len, eps=eps, stream=s)
    return out


def sana_linattn_bwd_workspace_bytes(B: int, H: int, N: int, D: int, block_len: int = 0) -> int:
    out = ctypes.c_size_t(0)
    _check(lib.sana_linattn_bwd_workspace_bytes(B, H, N, D, block_len, ctypes.byref(out)),
           "sana_linattn_bwd_workspace_bytes")
    return out.value


def sana_linattn_bwd(q, k, v, dout, dq, dk, dv, workspace, *, block_len: int = 0, eps: float = 1e-15,
                     stream=None):
    """Gradients dq, dk, dv (written in place) of the forward for upstream gradient dout."""
    B, N, H, D = _shape(q, k, v, dout)
    for name, t in (("dq", dq), ("dk", dk), ("dv", dv)):
        if tuple(t.shape) != (B, N, H, D) or not t.is_contiguous() or not t.is_cuda:
            raise ValueError(f"{name} must be a contiguous GPU tensor of shape {(B, N, H, D)}")
    if not (dq.dtype == dk.dtype == dv.dtype):
        raise TypeError("dq, dk and dv must share one dtype")
    _check(lib.sana_linattn_bwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), dout.data_ptr(), dq.data_ptr(),
                                dk.data_ptr(), dv.data_ptr(), dtype_code(q), dtype_code(dout), dtype_code(dq),
                                B, H, N, D, block_len, eps, workspace.data_ptr(),
                                workspace.numel() * workspace.element_size(), _stream_handle(stream)),
           "sana_linattn_bwd")


def sana_linattn_states_bytes(B: int, H: int, N: int, D: int, block_len: int = 0) -> int:
    out = ctypes.c_size_t(0)
    _check(lib.sana_linattn_states_bytes(B, H, N, D, block_len, ctypes.byref(out)), "sana_linattn_states_bytes")
    return out.value


def sana_linattn_fwd_save_states(q, k, v, out, states, workspace, *, block_len: int = 0, eps: float = 1e-15,
                                 stream=None):
    """Forward into `out` that also writes the per-block prefix states into
    `states` (float32 GPU tensor of at least sana_linattn_states_bytes bytes,
    viewed as [B, H, NB, D, D+1])."""
    B, N, H, D = _shape(q, k, v, out)
    if not states.is_cuda or not states.is_contiguous() or states.dtype != _torch().float32 or \
            states.numel() * 4 < sana_linattn_states_bytes(B, H, N, D, block_len):
        raise ValueError("states must be a contiguous float32 GPU tensor of sana_linattn_states_bytes bytes")
    _check(lib.sana_linattn_fwd_save_states(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), dtype_code(q),
                                            dtype_code(out), B, H, N, D, block_len, eps, states.data_ptr(),
                                            workspace.data_ptr(), workspace.numel() * workspace.element_size(),
                                            _stream_handle(stream)),
           "sana_linattn_fwd_save_states")


def sana_linattn_bwd_from_states(q, k, v, dout, states, dq, dk, dv, workspace, *, block_len: int = 0,
                                 eps: float = 1e-15, stream=None):
    """Gradients dq, dk, dv (written in place) from the states a
    sana_linattn_fwd_save_states call wrote for the same q, k, v."""
    B, N, H, D = _shape(q, k, v, dout)
    for name, t in (("dq", dq), ("dk", dk), ("dv", dv)):
        if tuple(t.shape) != (B, N, H, D) or not t.is_contiguous() or not t.is_cuda:
            raise ValueError(f"{name} must be a contiguous GPU tensor of shape {(B, N, H, D)}")
    if not (dq.dtype == dk.dtype == dv.dtype):
        raise TypeError("dq, dk and dv must share one dtype")
    if not states.is_cuda or not states.is_contiguous() or states.dtype != _torch().float32 or \
            states.numel() * 4 < sana_linattn_states_bytes(B, H, N, D, block_len):
        raise ValueError("states must be a contiguous float32 GPU tensor of sana_linattn_states_bytes bytes")
    _check(lib.sana_linattn_bwd_from_states(q.data_ptr(), k.data_ptr(), v.data_ptr(), dout.data_ptr(),
                                            states.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(),
                                            dtype_code(q), dtype_code(dout), dtype_code(dq), B, H, N, D, block_len,
                                            eps, workspace.data_ptr(), workspace.numel() * workspace.element_size(),
                                            _stream_handle(stream)),
           "sana_linattn_bwd_from_states")


def linattn_bwd(q, k, v, dout, *, eps: float = 1e-15, grad_dtype=None, block_len: int | None = None,
                stream=None):
    """Allocates dq, dk, dv (q's dtype unless grad_dtype is given) and the
    workspace with torch, runs the backward and returns (dq, dk, dv)."""
    torch = _torch()
    s = _torch_stream(stream)
    with torch.cuda.stream(s):   # allocated on the stream the kernels run on
        gt = grad_dtype or q.dtype
        dq, dk, dv = (torch.empty(q.shape, dtype=gt, device=q.device) for _ in range(3))
        B, N, H, D = q.shape
        ws = torch.empty(max(sana_linattn_bwd_workspace_bytes(B, H, N, D, block_len or 0), 1),
                         dtype=torch.uint8, device=q.device)
        sana_linattn_bwd(q, k, v, dout, dq, dk, dv, ws, block_len=block_len or 0, eps=eps, stream=s)
    return dq, dk, dv


def sana_linattn_jvp_workspace_bytes(B: int, H: int, N: int, D: int, block_len: int = 0) -> int:
    out = ctypes.c_size_t(0)
    _check(lib.sana_linattn_jvp_workspace_bytes(B, H, N, D, block_len, ctypes.byref(out)),
           "sana_linattn_jvp_workspace_bytes")
    return out.value


def sana_linattn_jvp(q, k, v, q_t, k_t, v_t, out, out_t, workspace, *, block_len: int = 0, eps: float = 1e-15,
                     stream=None):
    """Output and its tangent along (q_t, k_t, v_t), written into out and out_t."""
    B, N, H, D = _shape(q, k, v, out)
    for name, t in (("q_t", q_t), ("k_t", k_t), ("v_t", v_t), ("out_t", out_t)):
        if tuple(t.shape) != (B, N, H, D) or not t.is_contiguous() or not t.is_cuda:
            raise ValueError(f"{name} must be a contiguous GPU tensor of shape {(B, N, H, D)}")
    if not (q.dtype == q_t.dtype == k_t.dtype == v_t.dtype) or out.dtype != out_t.dtype:
        raise TypeError("tangents must share the inputs' dtype, out_t the output's")
    _check(lib.sana_linattn_jvp(q.data_ptr(), k.data_ptr(), v.data_ptr(), q_t.data_ptr(), k_t.data_ptr(),
                                v_t.data_ptr(), out.data_ptr(), out_t.data_ptr(), dtype_code(q), dtype_code(out),
                                B, H, N, D, block_len, eps, workspace.data_ptr(),
                                workspace.numel() * workspace.element_size(), _stream_handle(stream)),
           "sana_linattn_jvp")


def linattn_jvp(q, k, v, q_t, k_t, v_t, *, eps: float = 1e-15, out_dtype=None, block_len: int | None = None,
                stream=None):
    """Allocates out, out_t (float32 unless out_dtype is given) and the
    workspace with torch and returns (out, out_t)."""
    torch = _torch()
    s = _torch_stream(stream)
    with torch.cuda.stream(s):   # allocated on the stream the kernels run on
        ot = out_dtype or torch.float32
        out = torch.empty(q.shape, dtype=ot, device=q.device)
        out_t = torch.empty(q.shape, dtype=ot, device=q.device)
        B, N, H, D = q.shape
        ws = torch.empty(max(sana_linattn_jvp_workspace_bytes(B, H, N, D, block_len or 0), 1),
                         dtype=torch.uint8, device=q.device)
        sana_linattn_jvp(q, k, v, q_t, k_t, v_t, out, out_t, ws, block_len=block_len or 0, eps=eps, stream=s)
    return out, out_t
