"""Builds libdsa.so (the HIP kernels + C ABI) for gfx950 with hipcc, in-tree.

Each .hip file is compiled to an object in parallel, then linked into one shared library.
Packed-FP32 instruction selection is disabled (-packed-fp32-ops off) for all device code.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
ROOT = os.path.dirname(PKG)
LIB = os.path.join(PKG, "libdsa.so")
BUILD_DIR = os.path.join(ROOT, "_build")

SOURCES = ["dsa_abi.hip", "k_store.hip", "k_indexer.hip", "k_topk.hip", "k_mla.hip", "k_probe.hip"]
HIPCC_FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-result",
               "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
               "-mllvm", "-amdgpu-mfma-vgpr-form=1",     # MFMA results in VGPRs: no AGPR read-back
               "-I", os.path.join(ROOT, "include")]


def _compile(src: str, extra: list[str]) -> str:
    obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
    cmd = ["hipcc", *HIPCC_FLAGS, *extra, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{out}")
    if out.strip():
        sys.stderr.write(out + "\n")
    return obj


def build(extra: list[str] | None = None, jobs: int = 8) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    extra = extra or []
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(lambda s: _compile(s, extra), SOURCES))
    tmp = LIB + ".tmp"
    subprocess.check_call(["hipcc", "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp])
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(sys.argv[1:]))
