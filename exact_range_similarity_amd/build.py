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


# Host-side AddressSanitizer and UndefinedBehaviorSanitizer build of the
# API layer (argument validation, handle state, planning and the host
# bookkeeping of every entry point), linked with the ordinary kernel
# objects.  Load it through ERSJ_LIBRARY with the clang ASan runtime
# preloaded into the interpreter (SANITIZER_RUNTIME).
SAN_LIB = os.path.join(OBJ, "libersj_san.so")
SAN_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer",
             "-shared-libsan", "-g", "-O1"]
SANITIZER_RUNTIME = os.path.join(os.path.dirname(os.path.dirname(HIPCC)), "llvm", "lib", "clang")


def sanitizer_runtime() -> str:
    """Path of the clang ASan runtime that a sanitized library needs preloaded."""
    for ver in sorted(os.listdir(SANITIZER_RUNTIME), reverse=True):
        p = os.path.join(SANITIZER_RUNTIME, ver, "lib", "linux", "libclang_rt.asan-x86_64.so")
        if os.path.exists(p):
            return p
    raise FileNotFoundError("clang ASan runtime not found under " + SANITIZER_RUNTIME)


def build_sanitized(verbose: bool = False) -> str:
    os.makedirs(OBJ, exist_ok=True)
    objs = [os.path.join(OBJ, os.path.splitext(s)[0] + ".o") for s in SOURCES if s.endswith(".hip")]
    if not all(os.path.exists(o) for o in objs):
        build(verbose)
    api = os.path.join(OBJ, "ersj_api_san.o")
    cmd = [HIPCC, *COMMON, *SAN_FLAGS, "-c", os.path.join(CSRC, "ersj_api.cpp"), "-o", api]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    cmd = [HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", "-shared-libsan", "-Xarch_host",
           "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined", *objs, api, "-o", SAN_LIB]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    return SAN_LIB


if __name__ == "__main__":
    if "--sanitize" in sys.argv:
        print(build_sanitized(verbose="-v" in sys.argv))
    else:
        print(build(verbose="-v" in sys.argv))
