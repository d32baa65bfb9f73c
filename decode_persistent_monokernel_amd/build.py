"""Compile the HIP library in-tree for gfx950.

libkie.so = the persistent decode kernel (kie_kernel.hip) + the batched
prefill kernels (kie_prefill.hip) + the host C ABI (kie_api.cpp).  Built with hipcc; packed fp32 vector instructions are turned
off for the device code (-packed-fp32-ops).
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libkie.so")
ARCH = os.environ.get("KIE_OFFLOAD_ARCH", "gfx950")


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError(f"build failed: {' '.join(cmd[:3])} ...")


def build(verbose: bool = False) -> str:
    cc = hipcc()
    common = ["-O3", "-std=c++17", "-fPIC", f"-I{INCLUDE}", f"-I{CSRC}"]
    dev = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
    objs = []
    tmp = os.path.join(PKG, "_build")
    os.makedirs(tmp, exist_ok=True)
    k_o = os.path.join(tmp, "kie_kernel.o")
    _run([cc, f"--offload-arch={ARCH}", *common, *dev, "-c", os.path.join(CSRC, "kie_kernel.hip"), "-o", k_o], verbose)
    objs.append(k_o)
    p_o = os.path.join(tmp, "kie_prefill.o")
    _run([cc, f"--offload-arch={ARCH}", *common, *dev, "-c", os.path.join(CSRC, "kie_prefill.hip"), "-o", p_o], verbose)
    objs.append(p_o)
    a_o = os.path.join(tmp, "kie_api.o")
    _run([cc, *common, "-c", os.path.join(CSRC, "kie_api.cpp"), "-o", a_o], verbose)
    objs.append(a_o)
    out_tmp = LIB + ".tmp"
    _run([cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", out_tmp], verbose)
    os.replace(out_tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
