"""Build liblongspark.so (gfx950) in-tree with hipcc.

    python -m fixed_cost_drafter_amd.build [--resource-usage]

Each source is compiled to an object under ``fixed_cost_drafter_amd/_build``
in parallel, then linked into ``fixed_cost_drafter_amd/liblongspark.so``.
Every HIP translation unit is built with packed-fp32 instructions disabled.
"""
from __future__ import annotations

import argparse
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "liblongspark.so")
SOURCES = ["abi.cpp", "verify.hip", "append.hip", "init.hip", "draft.hip", "boundary.hip",
           "verify_attn.hip", "sampling.hip", "noalloc.hip", "round.hip"]
ARCH = "gfx950"


def hipcc() -> str:
    for p in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc"):
        if p and os.path.exists(p):
            return p
    return "hipcc"


def flags(resource_usage: bool = False) -> list[str]:
    f = ["-x", "hip", f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-I", os.path.join(ROOT, "include"), "-Wno-unused-command-line-argument"]
    if resource_usage:
        f += ["-Rpass-analysis=kernel-resource-usage"]
    return f


def compile_one(src: str, resource_usage: bool) -> tuple[str, str]:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), *flags(resource_usage), "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    return obj, r.stderr


def build(resource_usage: bool = False, verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with ThreadPoolExecutor(max_workers=min(len(SOURCES), os.cpu_count() or 4)) as ex:
        results = list(ex.map(lambda s: compile_one(s, resource_usage), SOURCES))
    if verbose or resource_usage:
        for (obj, err), src in zip(results, SOURCES):
            lines = [l for l in err.splitlines() if "target-feature" not in l and
                     "packed-fp32-ops" not in l]
            if lines:
                print(f"--- {src}\n" + "\n".join(lines))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp,
           *[o for o, _ in results]]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


def main(argv=None) -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--resource-usage", action="store_true")
    a = ap.parse_args(argv)
    print(build(resource_usage=a.resource_usage, verbose=True))
    return 0


if __name__ == "__main__":
    sys.exit(main())
