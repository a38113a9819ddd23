"""Builds libmoe_ffn.so for gfx950 with hipcc, in the package directory.

Usage: python -m mixture_experts_ffn_align_amd.build   (or build() from Python)
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libmoe_ffn.so")
SOURCES = ["api.hip", "align.hip", "decode.hip", "grouped.hip"]
# Measurement kernels (streaming-read floor, copy peak) for bench.py.
BENCH_LIB = os.path.join(PKG, "libmoe_bench.so")
BENCH_SOURCES = ["bench_kernels.hip"]
ARCH = "gfx950"

FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-Wall", "-Wno-unused-result",
    # Keep the compiler from emitting packed-fp32 VALU ops.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-fvisibility=hidden",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def _compile(sources, out, verbose, extra=()):
    tmp = out + ".tmp"
    cmd = [hipcc(), *FLAGS, *extra, f"-I{INCLUDE}", f"-I{CSRC}",
           *[os.path.join(CSRC, s) for s in sources], "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    text = "\n".join(l for l in (res.stdout + res.stderr).splitlines()
                     if "packed-fp32-ops" not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{text}")
    if text.strip() and verbose:
        print(text)
    os.replace(tmp, out)


def build(verbose: bool = False) -> str:
    """Compile the layer library and the measurement library; returns the
    layer library's path."""
    _compile(SOURCES, LIB, verbose)
    _compile(BENCH_SOURCES, BENCH_LIB, verbose)
    return LIB


# Host-side AddressSanitizer and UndefinedBehaviorSanitizer (each -fsanitize=
# applies to the host pass only; the device code is built as usual).
SANITIZE_HOST = [
    "-O1", "-g",
    "-Xarch_host", "-fsanitize=address",
    "-Xarch_host", "-fsanitize=undefined",
    "-Xarch_host", "-fno-sanitize-recover=undefined",
    "-Xarch_host", "-fno-omit-frame-pointer",
]


def build_host_sanitized(out: str, verbose: bool = False) -> str:
    """The layer library with instrumented host code, written to `out` (not
    the in-tree library). Loading it needs the sanitizer runtime preloaded
    (asan_runtime())."""
    _compile(SOURCES, out, verbose, SANITIZE_HOST)
    return out


def asan_runtime() -> str | None:
    """Path of the compiler's shared AddressSanitizer runtime, or None."""
    clang = os.path.join(os.path.dirname(os.path.realpath(hipcc())), "..", "llvm", "bin", "clang")
    for cand in (clang, "/opt/rocm/llvm/bin/clang"):
        if os.path.exists(cand):
            res = subprocess.run([cand, "-print-file-name=libclang_rt.asan-x86_64.so"],
                                 capture_output=True, text=True)
            path = res.stdout.strip()
            if res.returncode == 0 and os.path.isabs(path) and os.path.exists(path):
                return path
    return None


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
