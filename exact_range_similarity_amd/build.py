"""Compile the HIP sources into ``libersj.so`` (gfx950) inside the package.

Every device translation unit is built with packed-FP32 instruction
selection turned off (``-Xclang -target-feature -Xclang -packed-fp32-ops``):
the kernels use plain fp32 vector instructions only.  Objects go to
``_build/`` at the repository root; the library lands next to this file.
"""
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
OBJ = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "libersj.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

SOURCES = ["k_index.hip", "k_refine.hip", "k_refine_mfma.hip", "k_refine_m16.hip", "k_refine_g16.hip", "k_expand.hip", "k_knn.hip", "k_scratch.hip",
           "ersj_api.cpp"]

COMMON = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-I", INCLUDE, "-I", CSRC,
          "-Wall", "-Wno-unused-result", "-Wno-unused-command-line-argument"]
DEVICE = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-ffp-contract=fast-honor-pragmas"]


def _compile(src: str, verbose: bool) -> str:
    out = os.path.join(OBJ, os.path.splitext(src)[0] + ".o")
    lang = ["-x", "hip"] if src.endswith(".hip") else []
    cmd = [HIPCC, *COMMON, *lang, *(DEVICE if src.endswith(".hip") else []), "-c",
           os.path.join(CSRC, src), "-o", out]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    return out


def build(verbose: bool = False) -> str:
    os.makedirs(OBJ, exist_ok=True)
    with ThreadPoolExecutor(max_workers=4) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), SOURCES))
    cmd = [HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", LIB + ".tmp"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
