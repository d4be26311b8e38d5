"""Builds libspb.so in-tree for gfx950 with hipcc.

    python -m shared_prefix_branch_amd.build

One shared library: the host planner and C ABI (spb_host.cpp) and the
kernel sources (attention, lm head, decoder-stack layers, slot decoding).  Packed-FP32 instruction selection is switched off for the GPU
code (-packed-fp32-ops).
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libspb.so")
SOURCES = ["spb_host.cpp", "spb_attention.hip", "spb_score.hip", "spb_layer.hip", "spb_decode.hip"]
ARCH = "gfx950"


def hipcc() -> str:
    for c in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found")


def build(verbose: bool = False) -> str:
    """Compiles the library (always) and returns its path."""
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-Wno-unused-command-line-argument", "-I", os.path.join(HERE, "..", "include")]
    cmd += [os.path.join(CSRC, s) for s in SOURCES] + ["-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    errs = "\n".join(l for l in (r.stdout + r.stderr).splitlines()
                     if "packed-fp32-ops" not in l and l.strip())
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed ({r.returncode}):\n{errs}")
    if verbose and errs:
        print(errs)
    os.replace(tmp, LIB)
    return LIB


# The host-only sanitizer build: the planner, plan accessors and validations
# of spb_host.cpp under AddressSanitizer and UndefinedBehaviorSanitizer, built
# by g++ (no GPU code; the kernel launchers are spb_host_nogpu.cpp, which
# refuse every launch).  Loaded in place of libspb.so through SPB_LIBRARY by
# the host tests, in a process started with the ASan runtime preloaded.
SAN_LIB = os.path.join(HERE, "_build", "libspb_host_san.so")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def build_host_sanitized() -> str:
    os.makedirs(os.path.dirname(SAN_LIB), exist_ok=True)
    tmp = SAN_LIB + ".tmp"
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", "-fPIC", "-shared",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(ROCM, "include"), "-I", os.path.join(HERE, "..", "include"),
           os.path.join(CSRC, "spb_host.cpp"), os.path.join(CSRC, "spb_host_nogpu.cpp"),
           "-L", os.path.join(ROCM, "lib"), "-lamdhip64", "-Wl,-rpath," + os.path.join(ROCM, "lib"), "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"g++ failed ({r.returncode}):\n{r.stdout}{r.stderr}")
    os.replace(tmp, SAN_LIB)
    return SAN_LIB


if __name__ == "__main__":
    if "--host-sanitized" in sys.argv:
        print(build_host_sanitized())
    else:
        print(build(verbose="-v" in sys.argv))
