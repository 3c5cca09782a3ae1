"""Builds libzn.so in-tree with hipcc for gfx950 (no JIT cache, no pip install)."""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
OBJ = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libzn.so")
SOURCES = ["zn_api.hip", "zn_encode.hip", "zn_decode.hip", "zn_setup.hip"]
ARCH = os.environ.get("ZN_OFFLOAD_ARCH", "gfx950")
FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
         # packed FP32 instructions are kept out of every kernel
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Wall", "-Wno-unused-function", "-I", os.path.join(HERE, "..", "include")]


def _compile(src: str) -> str:
    obj = os.path.join(OBJ, src.replace(".hip", ".o"))
    cmd = ["hipcc", *FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    errs = "\n".join(l for l in (r.stdout + r.stderr).splitlines()
                     if "packed-fp32-ops" not in l and l.strip())
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{errs}")
    if errs:
        print(errs, file=sys.stderr)
    return obj


def build() -> str:
    """Compiles every HIP source and links libzn.so; always rebuilds."""
    os.makedirs(OBJ, exist_ok=True)
    with cf.ThreadPoolExecutor(len(SOURCES)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    r = subprocess.run(["hipcc", "-shared", f"--offload-arch={ARCH}", "-o", tmp, *objs],
                       capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stdout + r.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build())
