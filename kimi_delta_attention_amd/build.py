"""Builds libkda.so (the C-ABI library and its gfx950 kernels) in place with hipcc."""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libkda.so")
SOURCES = ["kda_api.cpp", "kda_decode.hip", "kda_layer.hip", "kda_prefill.hip",
           "kda_prefill_prep.hip",
           "kda_prefill_state.hip", "kda_prefill_f32.hip", "kda_noalloc.hip"]
ARCH = os.environ.get("KDA_OFFLOAD_ARCH", "gfx950")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
    f"--offload-arch={ARCH}",
    # keep packed-fp32 VALU instructions out of the generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def build(verbose: bool = False) -> str:
    """Compiles every source (always) and links libkda.so next to this file."""
    objs = []
    bdir = os.path.join(HERE, "_build")
    os.makedirs(bdir, exist_ok=True)
    cmds = []
    for src in SOURCES:
        obj = os.path.join(bdir, os.path.splitext(src)[0] + ".o")
        lang = ["-x", "hip"] if src.endswith(".hip") else []
        cmds.append([HIPCC, *FLAGS, *lang, "-c", os.path.join(CSRC, src), "-o", obj])
        objs.append(obj)
    # the sources compile independently: run them side by side (bounded by the
    # host's cores and the job limit the environment sets)
    jobs = max(1, min(len(cmds), os.cpu_count() or 1, int(os.environ.get("MAX_JOBS", "16"))))
    running = []
    for cmd in cmds:
        if verbose:
            print(" ".join(cmd), flush=True)
        running.append(subprocess.Popen(cmd))
        if len(running) >= jobs:
            if running.pop(0).wait() != 0:
                raise subprocess.CalledProcessError(1, "hipcc")
    for pr in running:
        if pr.wait() != 0:
            raise subprocess.CalledProcessError(1, "hipcc")
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.check_call(cmd)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
