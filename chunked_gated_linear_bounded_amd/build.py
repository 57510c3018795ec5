"""Builds libkda.so (HIP kernels for gfx950 + the host C ABI) in-tree with hipcc.

    python -m chunked_gated_linear_bounded_amd.build

Flags: -O3 for gfx950 only; packed-fp32 instruction selection is disabled
(-target-feature -packed-fp32-ops) for every device compile.  MFMA results
are kept in ordinary VGPRs (-amdgpu-mfma-vgpr-form): a kernel whose LDS use
already limits it to one work-group per CU otherwise gets the accumulator-
register form, and every accumulator is copied out with v_accvgpr_read
before VALU code can use it.  The machine scheduler favours instruction-level
parallelism over occupancy (-amdgpu-sched-strategy=max-ilp): the chunk kernel's
occupancy is set by its LDS and the state kernel runs one work-group per CU, so
latency hiding inside a wave is what pays (about 1 % and 3 % faster, same results).
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
LIB = os.path.join(PKG, "libkda.so")
ARCH = "gfx950"

HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
COMMON = ["-O3", "-std=c++17", "-fPIC", "-I", os.path.join(ROOT, "include"), "-I", CSRC]
DEVICE = ["--offload-arch=" + ARCH, "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-munsafe-fp-atomics", "-mllvm", "-amdgpu-mfma-vgpr-form",
          "-mllvm", "-amdgpu-sched-strategy=max-ilp"]

# (source, output object, extra defines)
UNITS = [
    ("kda_kernels.hip", "kda_kernels.o", []),
    ("kda_kernels_lowrank.hip", "kda_kernels_lowrank.o", []),
    ("kda_kernels_bwd.hip", "kda_kernels_bwd.o", []),
    ("kda_abi.cpp", "kda_abi.o", []),
]


def _compile(src, obj, defs):
    cmd = [HIPCC] + COMMON + defs + ["-c", os.path.join(CSRC, src), "-o", os.path.join(BUILD, obj)]
    if src.endswith(".hip"):
        cmd[1:1] = DEVICE
    else:
        cmd[1:1] = ["-x", "c++", "-D__HIP_PLATFORM_AMD__", "-I", "/opt/rocm/include"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("compile failed: %s\n%s\n%s" % (" ".join(cmd), r.stdout, r.stderr))
    return obj


def build(verbose: bool = True) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(8, len(UNITS))) as ex:
        list(ex.map(lambda u: _compile(*u), UNITS))
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [HIPCC, "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp] + \
          [os.path.join(BUILD, u[1]) for u in UNITS]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed: %s\n%s" % (r.stdout, r.stderr))
    os.replace(tmp, LIB)
    if verbose:
        print("built", LIB)
    return LIB


if __name__ == "__main__":
    build()
    sys.exit(0)
