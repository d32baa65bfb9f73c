"""Compile the HIP library in-tree for gfx950.

libkie.so = the persistent decode kernel (kie_kernel.hip, built for two ring
depths) + the batched prefill kernels (kie_prefill.hip) + the host C ABI
(kie_api.cpp).  Built with hipcc; packed fp32 vector instructions are turned
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
    # the decode kernel once per ring depth (kRingBase, kRingDeep in kie_layout.h)
    for depth in (8, 10):
        k_o = os.path.join(tmp, f"kie_kernel_ring{depth}.o")
        _run([cc, f"--offload-arch={ARCH}", *common, *dev, f"-DKIE_RING_DEPTH={depth}", "-c",
              os.path.join(CSRC, "kie_kernel.hip"), "-o", k_o], verbose)
        objs.append(k_o)
    p_o = os.path.join(tmp, "kie_prefill.o")
    _run([cc, f"--offload-arch={ARCH}", *common, *dev, "-c", os.path.join(CSRC, "kie_prefill.hip"), "-o", p_o], verbose)
    objs.append(p_o)
    a_o = os.path.join(tmp, "kie_api.o")
    # host code keeps its debug info, so a native stack names its frames
    _run([cc, *common, "-g", "-c", os.path.join(CSRC, "kie_api.cpp"), "-o", a_o], verbose)
    objs.append(a_o)
    out_tmp = LIB + ".tmp"
    _run([cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", out_tmp], verbose)
    os.replace(out_tmp, LIB)
    return LIB


SANITIZED_LIB = os.path.join(PKG, "_build", "libkie_host_sanitized.so")


def build_host_sanitized(verbose: bool = False) -> str:
    """The host library alone (kie_api.cpp, no device code: the launch
    helpers are stand-ins that report no device binary), compiled with g++
    under AddressSanitizer and UndefinedBehaviorSanitizer, for the CPU tests
    of the C ABI.  Load it with the sanitizer runtime preloaded
    (sanitizer_env())."""
    os.makedirs(os.path.dirname(SANITIZED_LIB), exist_ok=True)
    cxx = shutil.which("g++") or "g++"
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    out_tmp = SANITIZED_LIB + ".tmp"
    _run([cxx, "-std=c++17", "-O1", "-g", "-fPIC", "-shared", "-fsanitize=address,undefined",
          "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer", "-D__HIP_PLATFORM_AMD__",
          f"-I{rocm}/include", f"-I{INCLUDE}", f"-I{CSRC}", os.path.join(CSRC, "kie_api.cpp"),
          os.path.join(CSRC, "kie_host_stubs.cpp"), f"-L{rocm}/lib", "-lamdhip64", f"-Wl,-rpath,{rocm}/lib",
          "-o", out_tmp], verbose)
    os.replace(out_tmp, SANITIZED_LIB)
    return SANITIZED_LIB


def sanitizer_env() -> dict:
    """environment for a process that loads the sanitized host library: the
    sanitizer runtime first in the link order, leak checks off (the Python
    interpreter's own allocations are never freed), any error fatal"""
    cxx = shutil.which("g++") or "g++"
    asan = subprocess.run([cxx, "-print-file-name=libasan.so"], capture_output=True, text=True).stdout.strip()
    env = dict(os.environ)
    env["LD_PRELOAD"] = asan
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=1:halt_on_error=1"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    env["KIE_LIBRARY"] = SANITIZED_LIB
    return env


if __name__ == "__main__":
    if len(sys.argv) > 1 and sys.argv[1] == "sanitized":
        print(build_host_sanitized(verbose=True))
    else:
        print(build(verbose=True))
