"""Host-side AddressSanitizer / UndefinedBehaviorSanitizer build of the C ABI.

    python -m fixed_cost_drafter_amd.sanitize

Builds ``_build/sanitize/liblongspark_san.so``: the host code that validates
and marshals every call (``abi.cpp``, and ``noalloc.hip``'s host part) is
instrumented with ASan and UBSan; the kernels' device code is not (GPU
sanitizers are not used).  The other translation units are the objects of the
regular build.  Load it with the clang ASan runtime preloaded and
``LONGSPARK_LIB`` pointing at it (tests/test_abi_sanitized.py does this for
the host-side ABI tests, on a machine without a GPU).
"""
from __future__ import annotations

import glob
import os
import subprocess
import sys

from . import build as B

OUT = os.path.join(B.BUILD, "sanitize")
LIB = os.path.join(OUT, "liblongspark_san.so")
HOST_CHECKED = ("abi.cpp", "noalloc.hip")
SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
       "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host", "-fno-sanitize-recover=all"]


def asan_runtime() -> str | None:
    """The clang ASan runtime that hipcc's host compiler links against."""
    hits = sorted(glob.glob("/opt/rocm/lib/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return hits[-1] if hits else None


def build() -> str:
    os.makedirs(OUT, exist_ok=True)
    B.build()  # regular objects for the kernels' translation units
    objs = []
    for src in B.SOURCES:
        if src in HOST_CHECKED:
            obj = os.path.join(OUT, os.path.splitext(src)[0] + ".o")
            cmd = [B.hipcc(), *B.flags(), *SAN, "-g", "-c", os.path.join(B.CSRC, src), "-o", obj]
            r = subprocess.run(cmd, capture_output=True, text=True)
            if r.returncode != 0:
                raise RuntimeError(f"sanitized build of {src} failed:\n{r.stderr}")
        else:
            obj = os.path.join(B.BUILD, os.path.splitext(src)[0] + ".o")
        objs.append(obj)
    cmd = [B.hipcc(), f"--offload-arch={B.ARCH}", "-shared", "-fPIC", *SAN, "-shared-libsan",
           "-o", LIB, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"sanitized link failed:\n{r.stderr}")
    return LIB


if __name__ == "__main__":
    print(build())
    sys.exit(0)
