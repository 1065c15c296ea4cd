"""fp64 CPU oracle for the LiteLA forward.

TEST INFRASTRUCTURE ONLY: imported by the tests, the smoke check and the
CPU-baseline leg of the benchmark.  The HIP product path never imports it.

* ``linattn_fwd``  -- the linear (state) form in C, fp64, OpenMP over (b, h);
  see ``linattn_oracle.c`` for the definition and the pages it follows.
* ``linattn_bwd``  -- its gradients (dq, dk, dv) in C, fp64, same structure.
* ``linattn_jvp``  -- its forward-mode derivative (out, d out) in C, fp64.
* ``brute``        -- the quadratic form in numpy (its pin).
* ``exact``        -- the quadratic form in exact rational arithmetic (tiny sizes).
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
# SANA_ORACLE_LIB selects another build of the same source (the sanitizer build)
_LIB_PATH = os.environ.get("SANA_ORACLE_LIB") or os.path.join(_HERE, "liblinattn_oracle.so")
_lib = None

F32 = 0
BF16 = 1
F16 = 2


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            from . import build as _b
            _b.build()
        lib = ctypes.CDLL(_LIB_PATH)
        lib.oracle_linattn_fwd.restype = ctypes.c_int
        lib.oracle_linattn_fwd.argtypes = [
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int,
            ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
            ctypes.c_double, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int]
        lib.oracle_linattn_fwd_qknorm.restype = ctypes.c_int
        lib.oracle_linattn_fwd_qknorm.argtypes = [
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int,
            ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
            ctypes.c_double, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_double,
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int]
        lib.oracle_max_threads.restype = ctypes.c_int
        lib.oracle_linattn_bwd.restype = ctypes.c_int
        lib.oracle_linattn_bwd.argtypes = [
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_int,
            ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_double,
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int]
        lib.oracle_linattn_jvp.restype = ctypes.c_int
        lib.oracle_linattn_jvp.argtypes = [
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
            ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_double,
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int]
        lib.oracle_decode.restype = ctypes.c_int
        lib.oracle_decode.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t, ctypes.c_void_p]
        _lib = lib
    return _lib


def _dtype_code(a: np.ndarray) -> int:
    if a.dtype == np.uint16:
        return BF16
    if a.dtype == np.float32:
        return F32
    if a.dtype == np.float16:
        return F16
    raise TypeError(f"oracle inputs are float32, float16 or uint16 (bf16 bits), got {a.dtype}")


def decode(a: np.ndarray) -> np.ndarray:
    """The oracle's own decoding of its inputs to float64 (for pinning it)."""
    a = np.ascontiguousarray(a)
    out = np.empty(a.shape, dtype=np.float64)
    if _load().oracle_decode(a.ctypes.data, _dtype_code(a), a.size, out.ctypes.data) != 0:
        raise RuntimeError("oracle_decode failed")
    return out


def max_threads() -> int:
    return int(_load().oracle_max_threads())


def num_blocks(N: int, block_len: int | None) -> int:
    L = N if (not block_len or block_len <= 0 or block_len >= N) else block_len
    return (N + L - 1) // L if N > 0 else 0


def linattn_fwd(q, k, v, *, block_len: int | None = None, eps: float = 1e-15,
                nthreads: int = 0, return_states: bool = False, state_in=None,
                gamma_q=None, gamma_k=None, norm_eps: float = 0.0):
    """fp64 LiteLA forward on host arrays of shape [B, N, H, D].

    q, k, v: float32, float16, or uint16 holding bfloat16 bits (all three the same).
    block_len: None/0 for non-causal, else the frame-block length in tokens.
    state_in: optional float64 [B, H, D, D+1], the state before the first token
    (a carried state from an earlier call over the preceding tokens).
    gamma_q, gamma_k: optional [H, D] per-channel scales of the qk_norm prologue
    (each head's q or k row RMS-normalised over its D features, with norm_eps
    under the root, then scaled, before phi); None leaves that side as it is.
    Returns out as float64 [B, N, H, D]; with return_states also the inclusive
    per-block states, float64 [B, H, NB, D, D+1] (the last one is the final state).
    """
    q = np.ascontiguousarray(q)
    k = np.ascontiguousarray(k)
    v = np.ascontiguousarray(v)
    if not (q.shape == k.shape == v.shape) or q.ndim != 4:
        raise ValueError("q, k, v must share one [B, N, H, D] shape")
    code = _dtype_code(q)
    if _dtype_code(k) != code or _dtype_code(v) != code:
        raise TypeError("q, k, v must share one dtype")
    B, N, H, D = q.shape
    out = np.empty((B, N, H, D), dtype=np.float64)
    states = None
    if return_states:
        states = np.empty((B, H, max(num_blocks(N, block_len), 1), D, D + 1), dtype=np.float64)
    if state_in is not None:
        state_in = np.ascontiguousarray(state_in, dtype=np.float64)
        if state_in.shape != (B, H, D, D + 1):
            raise ValueError(f"state_in must be [B, H, D, D+1] = {(B, H, D, D + 1)}")
    gq = gk = None
    if gamma_q is not None:
        gq = np.ascontiguousarray(gamma_q, dtype=np.float64).reshape(H, D)
    if gamma_k is not None:
        gk = np.ascontiguousarray(gamma_k, dtype=np.float64).reshape(H, D)
    rc = _load().oracle_linattn_fwd_qknorm(
        q.ctypes.data, k.ctypes.data, v.ctypes.data, code, B, H, N, D,
        int(block_len or 0), float(eps), gq.ctypes.data if gq is not None else None,
        gk.ctypes.data if gk is not None else None, float(norm_eps), out.ctypes.data,
        states.ctypes.data if states is not None else None,
        state_in.ctypes.data if state_in is not None else None, int(nthreads))
    if rc != 0:
        raise RuntimeError(f"oracle_linattn_fwd failed ({rc})")
    return (out, states) if return_states else out


def linattn_bwd(q, k, v, dout, *, block_len: int | None = None, eps: float = 1e-15, nthreads: int = 0):
    """fp64 gradients (dq, dk, dv) of the LiteLA forward for dL/dout = dout.

    q, k, v as for linattn_fwd; dout float32, float16 or uint16 bf16 bits,
    [B, N, H, D].  Returns three float64 [B, N, H, D] arrays."""
    q, k, v, dout = (np.ascontiguousarray(x) for x in (q, k, v, dout))
    if not (q.shape == k.shape == v.shape == dout.shape) or q.ndim != 4:
        raise ValueError("q, k, v, dout must share one [B, N, H, D] shape")
    code = _dtype_code(q)
    if _dtype_code(k) != code or _dtype_code(v) != code:
        raise TypeError("q, k, v must share one dtype")
    B, N, H, D = q.shape
    dq, dk, dv = (np.empty((B, N, H, D), dtype=np.float64) for _ in range(3))
    rc = _load().oracle_linattn_bwd(q.ctypes.data, k.ctypes.data, v.ctypes.data, dout.ctypes.data, code,
                                    _dtype_code(dout), B, H, N, D, int(block_len or 0), float(eps),
                                    dq.ctypes.data, dk.ctypes.data, dv.ctypes.data, int(nthreads))
    if rc != 0:
        raise RuntimeError(f"oracle_linattn_bwd failed ({rc})")
    return dq, dk, dv


def linattn_jvp(q, k, v, qt, kt, vt, *, block_len: int | None = None, eps: float = 1e-15, nthreads: int = 0):
    """fp64 (out, tangent of out) of the LiteLA forward at (q, k, v) along the
    tangents (qt, kt, vt), which share the inputs' dtype and shape."""
    arrs = [np.ascontiguousarray(x) for x in (q, k, v, qt, kt, vt)]
    if any(a.shape != arrs[0].shape for a in arrs) or arrs[0].ndim != 4:
        raise ValueError("q, k, v and the tangents must share one [B, N, H, D] shape")
    code = _dtype_code(arrs[0])
    if any(_dtype_code(a) != code for a in arrs):
        raise TypeError("q, k, v and the tangents must share one dtype")
    B, N, H, D = arrs[0].shape
    out, outt = (np.empty((B, N, H, D), dtype=np.float64) for _ in range(2))
    rc = _load().oracle_linattn_jvp(*[a.ctypes.data for a in arrs], code, B, H, N, D, int(block_len or 0),
                                    float(eps), out.ctypes.data, outt.ctypes.data, int(nthreads))
    if rc != 0:
        raise RuntimeError(f"oracle_linattn_jvp failed ({rc})")
    return out, outt
