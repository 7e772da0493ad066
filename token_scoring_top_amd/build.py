"""Build libhubkv.so (the gfx950 kernels and the C ABI) in-tree with hipcc.

    python -m token_scoring_top_amd.build

Every source is compiled for gfx950 only, with packed-fp32 instruction
selection turned off, and linked into token_scoring_top_amd/libhubkv.so.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
OUT = os.path.join(HERE, "libhubkv.so")
BUILD_DIR = os.path.join(HERE, "_build")
SOURCES = ["abi.cpp", "score.hip", "refine_select.hip", "compact.hip", "h2o_step.hip",
           "select_layer.hip", "nestedkv.hip"]
ARCH = "gfx950"
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-fPIC", "-std=c++17", "-Wall", "-Wno-unused-function",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def _compile(src: str, verbose: bool) -> str:
    obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, "-x", "hip", *FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass warns that it does not know the packed-fp32 feature; drop that line
    err = "\n".join(x for x in r.stderr.splitlines() if "packed-fp32-ops" not in x)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{err}")
    if verbose and err.strip():
        print(err, file=sys.stderr)
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    with ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), SOURCES))
    tmp = OUT + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stderr)
    os.replace(tmp, OUT)
    return OUT


SAN_OUT = os.path.join(BUILD_DIR, "libhubkv_san.so")
# host-side sanitizers only: every -fsanitize applies to the host pass
SAN_FLAGS = ["-O1", "-g", "-fno-omit-frame-pointer",
             "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-sanitize-recover=all"]


def build_sanitized() -> str:
    """libhubkv_san.so: the C ABI layer (abi.cpp: validation, workspace sizing,
    dispatch) compiled with AddressSanitizer and UndefinedBehaviorSanitizer on
    its host code, linked with the kernels of the regular build.  For the test
    suite's host-side memory-safety run; the GPU code is not instrumented."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    objs = [os.path.join(BUILD_DIR, os.path.splitext(x)[0] + ".o") for x in SOURCES if x != "abi.cpp"]
    if not all(os.path.exists(o) for o in objs):
        build()
    obj = os.path.join(BUILD_DIR, "abi_san.o")
    flags = [f for f in FLAGS if f != "-O3"]
    cmd = [HIPCC, "-x", "hip", *flags, *SAN_FLAGS, "-c", os.path.join(CSRC, "abi.cpp"), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed on abi.cpp (sanitized):\n" + r.stderr)
    tmp = SAN_OUT + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", obj, *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed (sanitized):\n" + r.stderr)
    os.replace(tmp, SAN_OUT)
    return SAN_OUT


if __name__ == "__main__":
    print(build(verbose=True))
