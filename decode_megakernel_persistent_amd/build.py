"""Build libmk.so (the C-ABI library) for gfx950, in-tree.

    python -m decode_megakernel_persistent_amd.build

Every call compiles from scratch: hipcc for ``runtime.hip``, once per kernel
batch variant (``-DMK_UNIT_NB=v``: that variant's worker and launch-per-task
kernels, the dispatch kernel with v = 1) and once for its host side
(``-DMK_UNIT_HOST``: the C ABI), all in parallel; g++ for the host-only
compiler / simulator / checker; linked by hipcc into
``decode_megakernel_persistent_amd/libmk.so``.
Also builds a host-only protocol simulator executable under ThreadSanitizer
(``_build/mk_sim_tsan``) when requested.
"""

from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libmk.so")
ARCH = os.environ.get("MK_OFFLOAD_ARCH", "gfx950")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
HIP_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    # packed fp32 instructions are disabled for all device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]
HOST_FLAGS = ["-O2", "-std=c++17", "-fPIC", "-pthread", "-Wall"]
HOST_SRCS = ["graph.cpp", "sim.cpp"]
KERNEL_VARIANTS = [1, 2, 3, 4, 16, 17]  # VALU batches 1..4, the MFMA variant (kMfmaVariant), batch 1 with the LDS ring (kRingVariant)


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"build step failed ({r.returncode}): {' '.join(cmd)}\n{out}")
    if verbose and out.strip():
        print(out)


def build(verbose: bool = False, tsan: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    inc = ["-I", INCLUDE, "-I", CSRC]
    jobs = []
    objs = []
    for src in HOST_SRCS:
        obj = os.path.join(BUILD, src.replace(".cpp", ".o"))
        jobs.append(["g++", *HOST_FLAGS, *inc, "-c", os.path.join(CSRC, src), "-o", obj])
        objs.append(obj)
    for unit in [f"-DMK_UNIT_NB={v}" for v in KERNEL_VARIANTS] + ["-DMK_UNIT_HOST"]:
        obj = os.path.join(BUILD, "runtime_" + unit.split("-D")[1].replace("=", "") + ".o")
        jobs.append([HIPCC, *HIP_FLAGS, unit, *inc, "-c", os.path.join(CSRC, "runtime.hip"), "-o", obj])
        objs.append(obj)
    with ThreadPoolExecutor(max_workers=min(len(jobs), os.cpu_count() or 1, 16)) as ex:
        list(ex.map(lambda c: _run(c, verbose), jobs))
    tmp = LIB + ".tmp"
    _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs, "-pthread", "-ldl"], verbose)
    os.replace(tmp, LIB)
    if tsan:
        build_tsan(verbose)
    return LIB


def build_tsan(verbose: bool = False) -> str:
    """Host-only simulator + checker executable built with ThreadSanitizer."""
    os.makedirs(BUILD, exist_ok=True)
    exe = os.path.join(BUILD, "mk_sim_tsan")
    srcs = [os.path.join(CSRC, s) for s in HOST_SRCS] + [os.path.join(CSRC, "sim_main.cpp")]
    _run(["g++", "-O1", "-g", "-std=c++17", "-pthread", "-fsanitize=thread", "-I", INCLUDE, "-I", CSRC, *srcs,
          "-o", exe], verbose)
    return exe


def build_asan(verbose: bool = False) -> str:
    """The same host driver built with AddressSanitizer and
    UndefinedBehaviorSanitizer (graph compiler, simulator, trace checker)."""
    os.makedirs(BUILD, exist_ok=True)
    exe = os.path.join(BUILD, "mk_sim_asan")
    srcs = [os.path.join(CSRC, s) for s in HOST_SRCS] + [os.path.join(CSRC, "sim_main.cpp")]
    _run(["g++", "-O1", "-g", "-std=c++17", "-pthread", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
          "-fno-omit-frame-pointer", "-I", INCLUDE, "-I", CSRC, *srcs, "-o", exe], verbose)
    return exe


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv, tsan="--tsan" in sys.argv))
