"""Build libmoe.so (the HIP kernels and the C ABI) in-tree for gfx950.

``python -m gemm_gate_softmax_amd.build`` compiles the library's ``csrc/*.hip`` with hipcc and
links them into ``gemm_gate_softmax_amd/libmoe.so``; ``csrc/probe.hip`` (memory-path ceilings
for ``bench.py --memory-ceilings``, not part of the library) becomes ``libmoe_probe.so``.
Compilation runs in parallel; objects go to ``gemm_gate_softmax_amd/_build``.

``python -m gemm_gate_softmax_amd.build --variant NAME -DMOE_...=V ...`` builds the library
with the given compile-time switches into ``gemm_gate_softmax_amd/_variants/libmoe_NAME.so``,
for ``bench.py --ab`` comparisons of the alternatives the sources keep behind switches.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libmoe.so")
SOURCES = ["api.hip", "gemm.hip", "gate.hip", "pft.hip", "move.hip", "backward.hip"]
PROBE_SOURCE = "probe.hip"
PROBE_LIB = os.path.join(HERE, "libmoe_probe.so")
VARIANTS = os.path.join(HERE, "_variants")
ARCH = "gfx950"

# Packed fp32 vector ops are switched off for all device code (the compiler otherwise
# forms them from plain float arithmetic).
FLAGS = [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden",
         "-Wall", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libmoe.so)")


def _compile(src: str, out_dir: str = BUILD, defines=()) -> str:
    obj = os.path.join(out_dir, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), *FLAGS, *defines, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def _link(objs, lib: str) -> None:
    tmp = lib + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, lib)


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = SOURCES + [PROBE_SOURCE]
    with ThreadPoolExecutor(max_workers=min(len(srcs), os.cpu_count() or 1)) as ex:
        objs = list(ex.map(_compile, srcs))
    _link(objs[:-1], LIB)
    _link(objs[-1:], PROBE_LIB)
    if verbose:
        print(f"built {LIB} and {PROBE_LIB}")
    return LIB


def build_variant(name: str, defines) -> str:
    """libmoe.so built with extra -D switches into _variants/libmoe_NAME.so."""
    defines = list(defines)
    if not name.isidentifier() or any(not d.startswith("-DMOE_") for d in defines):
        raise ValueError("variant: a plain name and -DMOE_... switches only")
    out_dir = os.path.join(VARIANTS, name + ".objs")
    os.makedirs(out_dir, exist_ok=True)
    with ThreadPoolExecutor(max_workers=min(len(SOURCES), os.cpu_count() or 1)) as ex:
        objs = list(ex.map(lambda src: _compile(src, out_dir, defines), SOURCES))
    lib = os.path.join(VARIANTS, f"libmoe_{name}.so")
    _link(objs, lib)
    return lib


if __name__ == "__main__":
    if len(sys.argv) > 2 and sys.argv[1] == "--variant":
        print(f"built {build_variant(sys.argv[2], sys.argv[3:])}")
    else:
        build(verbose=True)
    sys.exit(0)
