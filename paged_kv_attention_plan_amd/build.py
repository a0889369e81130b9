"""Build libpkv.so (host planner + C ABI + gfx950 kernels) in-tree with hipcc,
and libpkv_ceilings.so, the benchmark's measurement probes (a bf16 MFMA loop
and a streaming read), which nothing on the attention path uses.

    python -m paged_kv_attention_plan_amd.build

Every HIP source is compiled for gfx950 only, with packed-FP32 VALU
instructions disabled (-Xclang -target-feature -Xclang -packed-fp32-ops).
Objects go to paged_kv_attention_plan_amd/_build/, the library next to this
file.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libpkv.so")
CEIL_LIB = os.path.join(PKG, "libpkv_ceilings.so")
ARCH = "gfx950"

SOURCES = ["plan.cpp", "capi.cpp", "decode.hip", "merge_append.hip", "prefill.hip", "mixed.hip",
           "noalloc.hip"]
CEIL_SOURCES = ["ceilings.hip"]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build the library)")


def common_flags():
    return [
        f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
        "-I", os.path.join(ROOT, "include"), "-I", CSRC,
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-Wno-unused-command-line-argument",
    ]


def _compile(src: str, verbose: bool) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    path = os.path.join(CSRC, src)
    # Kernels: no NaN inputs are supported, so fmaxf need not quiet signalling
    # NaNs first (saves a v_max_f32 x, x, x per operand in the softmax).
    lang = ["-x", "hip", "-fno-honor-nans"] if src.endswith(".hip") else []
    cmd = [hipcc()] + common_flags() + lang + ["-c", path, "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"compiling {src} failed:\n{res.stdout}\n{res.stderr}")
    return obj


def _link(objs, lib: str, verbose: bool) -> None:
    tmp = lib + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"linking {os.path.basename(lib)} failed:\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, lib)


def build(verbose: bool = False) -> str:
    """Compile every source, link libpkv.so and libpkv_ceilings.so.  Returns
    the path of libpkv.so."""
    os.makedirs(BUILD, exist_ok=True)
    srcs = SOURCES + CEIL_SOURCES
    with cf.ThreadPoolExecutor(max_workers=min(len(srcs), os.cpu_count() or 4)) as ex:
        objs = dict(zip(srcs, ex.map(lambda s: _compile(s, verbose), srcs)))
    _link([objs[s] for s in SOURCES], LIB, verbose)
    _link([objs[s] for s in CEIL_SOURCES], CEIL_LIB, verbose)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
