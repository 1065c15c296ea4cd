"""Compile the gfx950 LiteLA library into diffusion_transformer_relu_amd/lib/libsana_linattn.so.

hipcc builds the kernels and the C-ABI layer for gfx950 only.  Packed-fp32
instruction selection is switched off for device code; the host pass of hipcc
prints that it does not know this target feature, which is harmless.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIBDIR = os.path.join(PKG, "lib")
LIB = os.path.join(LIBDIR, "libsana_linattn.so")
SOURCES = [os.path.join(CSRC, "linattn_kernels.hip"), os.path.join(CSRC, "linattn_bwd_kernels.hip"),
           os.path.join(CSRC, "linattn_jvp_kernels.hip"), os.path.join(CSRC, "linattn_noalloc.hip"),
           os.path.join(CSRC, "linattn_api.cpp")]

HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-Wall", "-Wextra", "-Wno-unused-parameter",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-fvisibility=hidden",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (set HIPCC or install ROCm)")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    msgs = [l for l in (res.stdout + res.stderr).splitlines() if noise not in l]
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + "\n".join(msgs))
    if msgs and verbose:
        print("\n".join(msgs))


# Host-only AddressSanitizer + UndefinedBehaviorSanitizer for the sanitizer
# build (each flag applies to the host pass only; device code is built as
# usual).
SAN_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer", "-g"]


def build(verbose: bool = False, extra_flags=(), sanitize: bool = False) -> str:
    """Compiles every source to an object file in parallel (each kernel file
    holds its own launchers, so no device code crosses files), then links.
    sanitize: the host code (the C-ABI layer and the launchers) with
    AddressSanitizer and UndefinedBehaviorSanitizer, into lib_san/ (load it
    with SANA_LINATTN_LIB and the sanitizer runtime preloaded)."""
    from concurrent.futures import ThreadPoolExecutor

    libdir = LIBDIR + "_san" if sanitize else LIBDIR
    lib = os.path.join(libdir, os.path.basename(LIB))
    extra = [*extra_flags, *(SAN_FLAGS if sanitize else [])]
    os.makedirs(libdir, exist_ok=True)
    objdir = os.path.join(libdir, "obj")
    os.makedirs(objdir, exist_ok=True)
    inc = ["-I", os.path.join(ROOT, "include"), "-I", CSRC]
    compile_flags = [f for f in HIPCC_FLAGS if f != "-shared"]
    objs = [os.path.join(objdir, os.path.basename(s) + ".o") for s in SOURCES]
    with ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        jobs = [ex.submit(_run, [hipcc(), *compile_flags, *extra, *inc, "-c", s, "-o", o], verbose)
                for s, o in zip(SOURCES, objs)]
        for j in jobs:
            j.result()
    tmp = lib + ".tmp"
    _run([hipcc(), *HIPCC_FLAGS, *extra, *objs, "-o", tmp], verbose)
    os.replace(tmp, lib)
    return lib


if __name__ == "__main__":
    print(build(verbose=True, sanitize="--sanitize" in sys.argv))
