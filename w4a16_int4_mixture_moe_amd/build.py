"""Build the HIP library libw4a16moe.so for gfx950 (in-tree).

    python -m w4a16_int4_mixture_moe_amd.build [--jobs N] [--debug]

Compiles every source under csrc/ with hipcc (packed FP32 instructions
disabled), links one shared library into lib/, and returns its path.  Object
files go to _build/ at the repository root.
"""
from __future__ import annotations

import argparse
import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIBDIR = os.path.join(PKG, "lib")
LIBNAME = "libw4a16moe.so"
OBJDIR = os.path.join(ROOT, "_build", "w4a16moe")
ARCH = "gfx950"

SOURCES = ["api.cpp", "align.hip", "pack.hip", "gemm.hip", "prefill.hip", "mx.hip"]

COMMON = [
    f"--offload-arch={ARCH}", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-result",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # MFMA accumulators in ordinary VGPRs: with accumulation registers the
    # allocator rotates the GEMM accumulators between registers inside the
    # main loop, and every such move waits for an MFMA
    "-mllvm", "-amdgpu-mfma-vgpr-form=true",
    "-I", INCLUDE, "-I", CSRC,
]


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found (need ROCm)")


def lib_path() -> str:
    return os.path.join(LIBDIR, LIBNAME)


def _compile(src: str, opt: list[str]) -> str:
    obj = os.path.join(OBJDIR, os.path.splitext(src)[0] + ".o")
    lang = ["-x", "hip"] if src.endswith(".cpp") else []
    cmd = [hipcc()] + COMMON + opt + lang + ["-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in (r.stderr or "").splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{' '.join(cmd)}\n{err}")
    if err.strip():
        sys.stderr.write(err + "\n")
    return obj


def build(jobs: int = 4, debug: bool = False) -> str:
    os.makedirs(OBJDIR, exist_ok=True)
    os.makedirs(LIBDIR, exist_ok=True)
    opt = ["-O1", "-g"] if debug else ["-O3"]
    with cf.ThreadPoolExecutor(max_workers=max(1, jobs)) as ex:
        objs = list(ex.map(lambda s: _compile(s, opt), SOURCES))
    out = lib_path()
    tmp = out + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{r.stderr}")
    os.replace(tmp, out)
    return out


def main() -> None:
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=4)
    ap.add_argument("--debug", action="store_true")
    a = ap.parse_args()
    print(build(a.jobs, a.debug))


if __name__ == "__main__":
    main()
