"""Host-sanitizer build of libsvg2 (CPU side only).

Compiles the same sources as build.py, with AddressSanitizer and
UndefinedBehaviorSanitizer on the host code (argument validation, workspace
carving, launch set-up); the device code is built as usual.  The result goes
to _build/sanitized/libsvg2.so, outside the package, and is loaded by setting
SVG2_LIBRARY to it with clang's ASan runtime preloaded (see
tests/test_host_sanitizers_cpu.py).  It is a test build: GPU runs use the
regular library.

Usage: ``python -m sparse_attention_video_head_amd.build_sanitized``.
"""
from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import subprocess
import sys

from .build import ARCH, BUILD_DIR, CSRC, SOURCES, _flags, hipcc

OUT_DIR = os.path.join(BUILD_DIR, "sanitized")
LIB_PATH = os.path.join(OUT_DIR, "libsvg2.so")
# each sanitizer flag applies to the host compilation only
HOST_SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer",
            "-Xarch_host", "-g"]


def asan_runtime() -> str:
    """clang's shared ASan runtime matching hipcc's host compiler."""
    found = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not found:
        raise RuntimeError("clang's ASan runtime (libclang_rt.asan-x86_64.so) was not found")
    return found[-1]


def _compile(src: str) -> str:
    obj = os.path.join(OUT_DIR, os.path.basename(src) + ".o")
    cmd = [hipcc(), *_flags(), *HOST_SAN, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def build() -> str:
    os.makedirs(OUT_DIR, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(len(SOURCES), 8)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    cmd = [hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", "-shared-libsan",
           "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined", "-o", LIB_PATH, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return LIB_PATH


if __name__ == "__main__":
    print(build())
    sys.exit(0)
