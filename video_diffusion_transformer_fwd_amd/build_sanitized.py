"""Builds a copy of libh3dit.so whose host code runs under AddressSanitizer and
UndefinedBehaviorSanitizer, for CPU-only tests of the host logic and argument validation.

    python -m video_diffusion_transformer_fwd_amd.build_sanitized

The host-side sources (h3_host.cpp, h3_api.cpp, h3_profile.cpp) are compiled with the
sanitizers applied to their host pass only; the kernel objects of the regular build are
linked unchanged (GPU code is never instrumented).  The result is csrc/_build/libh3dit_san.so.
Load it with the sanitizer runtime preloaded (``sanitizer_env()``) and point the binding at
it through H3DIT_LIB.  It is for CPU runs: no kernel is launched through it.
"""
from __future__ import annotations

import glob
import os
import subprocess
import sys

from . import build as B

LIB = os.path.join(B.BUILD, "libh3dit_san.so")
HOST_SOURCES = ["h3_host.cpp", "h3_api.cpp", "h3_profile.cpp"]
# each sanitizer flag applies to the host compilation only
SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
       "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer",
       "-Xarch_host", "-g"]


def runtime_path() -> str:
    """The clang AddressSanitizer runtime matching hipcc's compiler."""
    hits = sorted(glob.glob("/opt/rocm/lib/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not hits:
        raise RuntimeError("clang AddressSanitizer runtime not found under /opt/rocm/lib/llvm")
    return hits[-1]


def sanitizer_env(env=None) -> dict:
    """Environment for a process that loads the sanitized library."""
    e = dict(os.environ if env is None else env)
    e["LD_PRELOAD"] = runtime_path()
    e["H3DIT_LIB"] = LIB
    # Python itself is not instrumented and keeps objects alive until exit
    e["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=0:halt_on_error=1:exitcode=86"
    e["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1:exitcode=87"
    return e


def build(verbose: bool = False) -> str:
    os.makedirs(B.BUILD, exist_ok=True)
    kernel_objs = []
    for src in B.SOURCES:
        if src in HOST_SOURCES:
            continue
        obj = os.path.join(B.BUILD, os.path.splitext(src)[0] + ".o")
        if not os.path.exists(obj):
            B._compile(src, verbose)
        kernel_objs.append(obj)
    host_objs = []
    for src in HOST_SOURCES:
        obj = os.path.join(B.BUILD, os.path.splitext(src)[0] + "_san.o")
        cmd = [B.HIPCC, *B.COMMON, *SAN, "-x", "hip", "-c", os.path.join(B.CSRC, src), "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"sanitized compile of {src} failed:\n{r.stdout}{r.stderr}")
        host_objs.append(obj)
    cmd = [B.HIPCC, f"--offload-arch={B.ARCH}", "-shared", "-fPIC", "-shared-libasan",
           "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           *host_objs, *kernel_objs, "-o", LIB]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"sanitized link failed:\n{r.stdout}{r.stderr}")
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
