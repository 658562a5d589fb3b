"""Build libpagedattn.so in-tree for gfx950.

Device sources are compiled with hipcc for gfx950 only; the host-only source
with g++.  The shared library is linked against the HIP runtime that PyTorch
ships (the copy inside ``torch/lib``), so one process holds one HIP runtime
and the stream and device pointers PyTorch hands over are valid in our calls.

Usage: ``python -m paged_kv_cache_reshape_amd.build`` (or ``build()``).
"""
from __future__ import annotations

import importlib.util
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(PKG, "_build")
LIB_NAME = "libpagedattn.so"
LIB_PATH = os.path.join(PKG, LIB_NAME)

ARCH = "gfx950"
HIP_SOURCES = ["decode_api.hip", "decode_partition.hip", "decode_mfma.hip", "decode_stream.hip",
               "decode_stream_mfma.hip", "prefill_mfma.hip", "kv_write.hip"]
HOST_SOURCES = ["status.cpp"]

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall",
    # never emit packed fp32 arithmetic (v_pk_*_f32)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def _hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def torch_lib_dir() -> str:
    spec = importlib.util.find_spec("torch")
    if spec is None or spec.origin is None:
        raise RuntimeError("torch is not importable; it provides the HIP runtime")
    return os.path.join(os.path.dirname(spec.origin), "lib")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"command failed ({res.returncode}): {' '.join(cmd)}\n"
                           f"{res.stdout}\n{res.stderr}")
    return res


def build(verbose: bool = False, jobs: int = 4, defines=(), out: str | None = None) -> str:
    """Compile every source and link ``libpagedattn.so``; returns its path.

    ``defines`` (``NAME=VALUE`` strings) and ``out`` build a variant of the
    library elsewhere, in its own object folder, for tuning experiments.
    """
    lib_path = out or LIB_PATH
    build_dir = BUILD_DIR if out is None else os.path.splitext(out)[0] + "_build"
    os.makedirs(build_dir, exist_ok=True)
    dflags = [f"-D{d}" for d in defines]
    hipcc = _hipcc()
    cmds = []
    objs = []
    for src in HIP_SOURCES:
        obj = os.path.join(build_dir, src + ".o")
        objs.append(obj)
        cmds.append([hipcc, "-x", "hip", *HIPCC_FLAGS, *dflags, f"-I{INCLUDE}", f"-I{CSRC}",
                     "-c", os.path.join(CSRC, src), "-o", obj])
    for src in HOST_SOURCES:
        obj = os.path.join(build_dir, src + ".o")
        objs.append(obj)
        cmds.append(["g++", "-O2", "-std=c++17", "-fPIC", "-Wall", f"-I{INCLUDE}", f"-I{CSRC}",
                     "-c", os.path.join(CSRC, src), "-o", obj])
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        list(ex.map(lambda c: _run(c, verbose), cmds))
    tlib = torch_lib_dir()
    tmp = lib_path + ".tmp"
    _run(["g++", "-shared", "-o", tmp, *objs, os.path.join(tlib, "libamdhip64.so"),
          f"-Wl,-rpath,{tlib}", "-Wl,--no-undefined", "-Wl,-z,defs"], verbose)
    os.replace(tmp, lib_path)
    return lib_path


# The benchmark's read-ceiling kernels (pure reads of the decode's access
# patterns), a library of their own beside bench.py: measurement, not part
# of libpagedattn.
CEILING_SRC = os.path.join(ROOT, "read_ceiling.hip")
CEILING_LIB = os.path.join(ROOT, "libreadceiling.so")


def build_read_ceiling(verbose: bool = False) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    obj = os.path.join(BUILD_DIR, "read_ceiling.hip.o")
    _run([_hipcc(), "-x", "hip", *HIPCC_FLAGS, "-c", CEILING_SRC, "-o", obj], verbose)
    tlib = torch_lib_dir()
    tmp = CEILING_LIB + ".tmp"
    _run(["g++", "-shared", "-o", tmp, obj, os.path.join(tlib, "libamdhip64.so"),
          f"-Wl,-rpath,{tlib}", "-Wl,--no-undefined"], verbose)
    os.replace(tmp, CEILING_LIB)
    return CEILING_LIB


if __name__ == "__main__":
    path = build(verbose="-v" in sys.argv)
    print(path)
    print(build_read_ceiling(verbose="-v" in sys.argv))
