"""Build the drafter's native libraries in-tree.

* ``libdflash.so``       the product: C ABI + HIP backend, kernels for gfx950.
* ``libdflash_host.so``  the same C ABI over the trace backend, host only; it
  lets the session state machine be tested on a machine without a GPU.

Run ``python -m block_diffusion_drafter_fwd_amd.build``.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
ROOT = os.path.dirname(HERE)

HIP_SOURCES = ["engine_hip.hip", "kern_gemm.hip", "kern_attn.hip", "kern_misc.hip"]
HOST_SOURCES = ["api.cpp"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
HIP_FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             # MFMA accumulators in ordinary VGPRs: no copies through AGPRs
             # where an accumulator is rescaled between products
             "-mllvm", "-amdgpu-mfma-vgpr-form",
             "-I", os.path.join(ROOT, "include"), "-Wno-unused-result"]
CXX_FLAGS = ["-O2", "-std=c++17", "-fPIC", "-Wall", "-I", os.path.join(ROOT, "include")]


def _run(cmd):
    p = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in p.stdout.splitlines() if "packed-fp32-ops" not in l)
    if p.returncode != 0:
        raise RuntimeError(f"command failed ({p.returncode}): {' '.join(cmd)}\n{out}")
    return out


def build_hip(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    jobs = []
    for src in HIP_SOURCES:
        obj = os.path.join(BUILD, src + ".o")
        jobs.append([HIPCC, *HIP_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj])
    for src in HOST_SOURCES:
        obj = os.path.join(BUILD, src + ".o")
        jobs.append(["g++", *CXX_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj])
    with cf.ThreadPoolExecutor(max_workers=min(8, len(jobs))) as ex:
        for out in ex.map(_run, jobs):
            if verbose and out.strip():
                print(out)
    objs = [os.path.join(BUILD, s + ".o") for s in HIP_SOURCES + HOST_SOURCES]
    lib = os.path.join(HERE, "libdflash.so")
    tmp = lib + f".tmp{os.getpid()}"
    # -z defs: an unresolved symbol (say, a kernel stub the host pass failed to
    # emit) fails the build instead of the first dlopen
    _run([HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", "-Wl,-z,defs", *objs, "-o", tmp])
    os.replace(tmp, lib)
    return lib


def build_host(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    lib = os.path.join(HERE, "libdflash_host.so")
    tmp = lib + f".tmp{os.getpid()}"
    out = _run(["g++", *CXX_FLAGS, "-shared", os.path.join(CSRC, "api.cpp"),
                os.path.join(CSRC, "engine_trace.cpp"), "-o", tmp])
    if verbose and out.strip():
        print(out)
    os.replace(tmp, lib)
    return lib


def build_all(verbose: bool = False):
    return build_hip(verbose), build_host(verbose)


if __name__ == "__main__":
    for p in build_all(verbose="-v" in sys.argv):
        print("built", p)
