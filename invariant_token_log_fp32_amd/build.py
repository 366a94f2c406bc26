"""Ahead-of-time build of the HIP library for gfx950.

Produces ``librlk_logp.so`` next to this file from ``csrc/rlk_logp.hip``
(token logprobs, their backward), ``csrc/rlk_norm.hip`` (gradient L2 norm) and
``csrc/rlk_linear.hip`` (LM-head linear, fused linear + logprob):
    python -m invariant_token_log_fp32_amd.build
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
SRCS = [os.path.join(PKG, "csrc", n) for n in ("rlk_logp.hip", "rlk_norm.hip", "rlk_linear.hip")]
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "librlk_logp.so")
ARCH = "gfx950"

HIP_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    # every intended fused multiply-add is written explicitly
    "-ffp-contract=off",
    # no packed fp32 instructions in the device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]


def hipcc() -> str:
    exe = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(exe):
        raise RuntimeError("hipcc not found: the ROCm toolchain is required to build librlk_logp.so")
    return exe


# Host-side sanitizer build (CPU tests only): AddressSanitizer and
# UndefinedBehaviorSanitizer on the host code, i.e. the C ABI's argument
# validation; the GPU code is built as usual.
HOST_SANITIZER_FLAGS = [
    "-O1", "-g",
    "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
    "-Xarch_host", "-fno-omit-frame-pointer",
]


def asan_runtime() -> str:
    """Path of the compiler's AddressSanitizer runtime (preloaded into a Python
    process that loads the sanitized library), or '' when it is not found."""
    clang = os.path.join(os.path.dirname(os.path.realpath(hipcc())), "..", "llvm", "bin", "clang")
    for exe in (clang, "/opt/rocm/llvm/bin/clang", shutil.which("clang") or ""):
        if exe and os.path.exists(exe):
            res = subprocess.run([exe, "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True, text=True)
            path = res.stdout.strip()
            if res.returncode == 0 and os.path.isabs(path) and os.path.exists(path):
                return path
    return ""


def build_host_sanitized(out: str, verbose: bool = False) -> str:
    """The library with HOST_SANITIZER_FLAGS, written to `out` (outside the package)."""
    return build(HOST_SANITIZER_FLAGS, out=out, verbose=verbose)


def build(extra_flags=(), out: str = LIB, verbose: bool = False) -> str:
    tmp = out + ".tmp"
    cmd = [hipcc(), *HIP_FLAGS, *extra_flags, "-I", INCLUDE, "-I", os.path.join(PKG, "csrc"), "-o", tmp, *SRCS]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"hipcc failed with status {res.returncode}")
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
