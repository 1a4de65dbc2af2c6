"""Build libdag_attn.so in-tree for gfx950.

    python dag_packed_attention_amd/build_lib.py      (or call build())

The host compactor (plan.cpp, gdn_plan.cpp, logprob_map.cpp, conv_plan.cpp, harts_plan.cpp) is plain C++ and is compiled with g++; the ABI
glue and the kernels are compiled with hipcc for gfx950.  Packed-fp32 code
generation is switched off for the device code.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "libdag_attn.so")
LIB_DEBUG = os.path.join(HERE, "libdag_attn_debug.so")  # DAG_DEBUG: device checks of the plan tables
ARCH = os.environ.get("DAG_ATTN_ARCH", "gfx950")

HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
_HIP_FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-Wall",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             f"-I{os.path.join(ROOT, 'include')}"]
_CXX_FLAGS = ["-O2", "-std=c++17", "-fPIC", "-Wall", "-Wextra", f"-I{os.path.join(ROOT, 'include')}"]


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"build step failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return r


OBJS = ("plan.o", "pack_plan.o", "gdn_plan.o", "logprob_map.o", "conv_plan.o", "harts_plan.o", "abi.o", "kernels.o", "gdn.o", "logprob.o",
        "conv.o", "noalloc.o")


def build(verbose: bool = False, debug: bool = False) -> str:
    """Compile every source and link libdag_attn.so (debug: libdag_attn_debug.so, every
    file compiled with DAG_DEBUG, objects in their own folder)."""
    obj_dir = os.path.join(HERE, "_build_debug" if debug else "_build")
    os.makedirs(obj_dir, exist_ok=True)
    HIP_FLAGS = _HIP_FLAGS + (["-DDAG_DEBUG"] if debug else [])
    CXX_FLAGS = _CXX_FLAGS + (["-DDAG_DEBUG"] if debug else [])
    lib = LIB_DEBUG if debug else LIB
    steps = [
        ["g++", *CXX_FLAGS, "-c", os.path.join(CSRC, "plan.cpp"), "-o", os.path.join(obj_dir, "plan.o")],
        ["g++", *CXX_FLAGS, "-c", os.path.join(CSRC, "pack_plan.cpp"), "-o", os.path.join(obj_dir, "pack_plan.o")],
        ["g++", *CXX_FLAGS, "-c", os.path.join(CSRC, "gdn_plan.cpp"), "-o", os.path.join(obj_dir, "gdn_plan.o")],
        ["g++", *CXX_FLAGS, "-c", os.path.join(CSRC, "logprob_map.cpp"),
         "-o", os.path.join(obj_dir, "logprob_map.o")],
        [HIPCC, *HIP_FLAGS, "-c", os.path.join(CSRC, "logprob.hip"), "-o", os.path.join(obj_dir, "logprob.o")],
        ["g++", *CXX_FLAGS, "-c", os.path.join(CSRC, "conv_plan.cpp"), "-o", os.path.join(obj_dir, "conv_plan.o")],
        ["g++", *CXX_FLAGS, "-c", os.path.join(CSRC, "harts_plan.cpp"), "-o", os.path.join(obj_dir, "harts_plan.o")],
        [HIPCC, *HIP_FLAGS, "-c", os.path.join(CSRC, "conv.hip"), "-o", os.path.join(obj_dir, "conv.o")],
        [HIPCC, *HIP_FLAGS, "-c", os.path.join(CSRC, "abi.cpp"), "-o", os.path.join(obj_dir, "abi.o")],
        [HIPCC, *HIP_FLAGS, "-c", os.path.join(CSRC, "kernels.hip"), "-o", os.path.join(obj_dir, "kernels.o")],
        [HIPCC, *HIP_FLAGS, "-c", os.path.join(CSRC, "gdn.hip"), "-o", os.path.join(obj_dir, "gdn.o")],
        [HIPCC, *HIP_FLAGS, "-c", os.path.join(CSRC, "noalloc.hip"), "-o", os.path.join(obj_dir, "noalloc.o")],
    ]
    with ThreadPoolExecutor(len(steps)) as ex:
        for r in ex.map(_run, steps):
            if verbose and r.stderr:
                sys.stderr.write(r.stderr)
    tmp = lib + ".tmp"
    _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-o", tmp,
          *(os.path.join(obj_dir, f) for f in OBJS)])
    os.replace(tmp, lib)
    return lib


if __name__ == "__main__":
    print(build(verbose=True, debug="--debug" in sys.argv[1:]))
