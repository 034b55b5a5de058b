"""Build the native libraries in-tree.

  libff.so            C ABI + gfx950 HIP kernels (hipcc, --offload-arch=gfx950):
                      ff_kernels.hip (renderer / planner attention, bank
                      copies), ff_bc_kernels.hip (block-causal backward),
                      ff_static_scratch.hip (the fixed device scratch of the
                      call that allocates nothing) and ff_prof.hip (settings
                      of the per-launch timing)
  libff_hostcheck.so  the same host bookkeeping linked against a recording stub
                      instead of the kernels (g++); CPU tests use it to drive the
                      ABI's success paths without a GPU.

Run ``python -m chunked_kv_cache_amd.build`` (``__graft_entry__.build()`` calls it).
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libff.so")
HOSTCHECK = os.path.join(PKG, "libff_hostcheck.so")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
# Packed fp32 VALU forms are kept out of every HIP object.  The kernels never
# produce or consume NaN on valid inputs (infinities are still honoured), so
# max/min need no NaN-quieting instructions.
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-fno-honor-nans"]


def _run(cmd):
    print("+", " ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)


def build(verbose_resources: bool = False) -> None:
    os.makedirs(BUILD, exist_ok=True)
    inc = ["-I", os.path.join(ROOT, "include")]
    host_src = os.path.join(CSRC, "host", "ff_host.cpp")
    host_obj = os.path.join(BUILD, "ff_host.o")
    _run(["g++", "-O2", "-std=c++17", "-fPIC", "-Wall", "-Wextra", *inc, "-c", host_src, "-o", host_obj])

    extra = ["-Rpass-analysis=kernel-resource-usage"] if verbose_resources else []
    kern_objs = []
    for name in ("ff_kernels", "ff_bc_kernels", "ff_static_scratch", "ff_prof"):
        src = os.path.join(CSRC, "hip", name + ".hip")
        obj = os.path.join(BUILD, name + ".o")
        _run([HIPCC, f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", *DEVICE_FLAGS, *extra, *inc,
              "-c", src, "-o", obj])
        kern_objs.append(obj)
    tmp = LIB + ".tmp"
    # -z defs: every symbol the host code calls must be defined by the kernels.
    _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-Wl,-z,defs", host_obj, *kern_objs, "-o", tmp])
    os.replace(tmp, LIB)

    stub_src = os.path.join(CSRC, "host", "device_stub.cpp")
    tmp = HOSTCHECK + ".tmp"
    _run(["g++", "-O2", "-std=c++17", "-fPIC", "-shared", "-Wall", *inc, host_src, stub_src, "-o", tmp])
    os.replace(tmp, HOSTCHECK)


if __name__ == "__main__":
    build(verbose_resources="-v" in sys.argv)
