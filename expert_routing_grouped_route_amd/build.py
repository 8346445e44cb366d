"""Build libmoe.so, the gfx950 HIP library behind the MoE-layer C ABI.

Each HIP source is compiled to an object for gfx950 (in parallel), then the
objects are linked into ``libmoe.so`` next to this file.  Every call compiles.
"""
from __future__ import annotations

import os
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG_DIR)
CSRC = os.path.join(PKG_DIR, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB_PATH = os.path.join(PKG_DIR, "libmoe.so")
SOURCES = ("route.hip", "dispatch.hip", "gemm_bf16.hip", "gemm_f32.hip", "combine.hip",
           "condense.hip", "backward.hip", "moe_api.hip")
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the gfx950 library cannot be built")


def compile_flags() -> list:
    return [
        f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden",
        # no packed-fp32 instructions in any generated code
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-I", INCLUDE, "-I", CSRC,
    ]


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    noise = "is not a recognized feature for this target"
    out = "\n".join(l for l in r.stdout.splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{out}")
    return out


def build_library(verbose: bool = False, jobs: int = 8) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    cc = hipcc()
    flags = compile_flags()

    def one(src):
        obj = os.path.join(BUILD_DIR, src.replace(".hip", ".o"))
        out = _run([cc, *flags, "-c", os.path.join(CSRC, src), "-o", obj])
        if verbose and out.strip():
            print(out)
        return obj

    with ThreadPoolExecutor(max(1, min(jobs, len(SOURCES)))) as ex:
        objs = list(ex.map(one, SOURCES))
    tmp = LIB_PATH + ".tmp"
    # --no-undefined: a kernel whose host-side launch stub went missing fails
    # here rather than when the library is loaded
    _run([cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-Wl,--no-undefined", *objs, "-o", tmp])
    os.replace(tmp, LIB_PATH)
    if verbose:
        print(f"built {LIB_PATH}")
    return LIB_PATH


if __name__ == "__main__":
    build_library(verbose=True)
