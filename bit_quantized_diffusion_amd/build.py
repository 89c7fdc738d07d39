"""Build libsvdq.so in-tree with hipcc for gfx950.

    python bit_quantized_diffusion_amd/build.py [-v]

(run as a file: importing the package needs a library that is already
built)

The kernels are compiled for gfx950 only.  Packed-FP32 VALU instructions are
disabled (-packed-fp32-ops) and no fast-math flag is used: the quantizer
needs IEEE division and round-to-nearest-even conversions on both the host
(offline pack) and the device.  Host-side files are compiled with
-ffp-contract=off so that no multiply-add is fused behind the pack's back.
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys
import tempfile

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libsvdq.so")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
HIPCC = os.path.join(ROCM, "bin", "hipcc")
CLANGXX = os.path.join(ROCM, "llvm", "bin", "clang++")

ARCH = "gfx950"
DEVICE_FLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-fvisibility=hidden",
]
HOST_FLAGS = ["-O3", "-std=c++17", "-fPIC", "-ffp-contract=off", "-pthread",
              "-Wall", "-fvisibility=hidden", "-D__HIP_PLATFORM_AMD__", f"-I{ROCM}/include"]

KERNEL_SOURCES = ["svdq_kernels.hip"]
HOST_SOURCES = ["svdq_abi.cpp", "svdq_pack.cpp"]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError(f"build step failed: {' '.join(cmd)}")
    # hipcc's host pass does not know the packed-fp32 target feature and
    # says so; that note is expected and not shown.
    noise = "'-packed-fp32-ops' is not a recognized feature"
    rest = "\n".join(ln for ln in (r.stdout + r.stderr).splitlines() if noise not in ln)
    if verbose and rest.strip():
        sys.stderr.write(rest + "\n")


def build(verbose: bool = False) -> str:
    """Compile every source and link libsvdq.so; returns the library path."""
    tmp = tempfile.mkdtemp(prefix="svdq_build_")
    try:
        objs = []
        procs = []
        for src in KERNEL_SOURCES:
            obj = os.path.join(tmp, src + ".o")
            procs.append(([HIPCC, *DEVICE_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj], obj))
        compiler = CLANGXX if os.path.exists(CLANGXX) else "g++"
        for src in HOST_SOURCES:
            obj = os.path.join(tmp, src + ".o")
            procs.append(([compiler, "-x", "c++", *HOST_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj], obj))
        running = [(subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True), cmd, obj)
                   for cmd, obj in procs]
        for p, cmd, obj in running:
            out, err = p.communicate()
            if p.returncode != 0:
                sys.stderr.write(out + err)
                raise RuntimeError(f"build step failed: {' '.join(cmd)}")
            if verbose:
                print(" ".join(cmd), flush=True)
            objs.append(obj)
        tmp_lib = os.path.join(tmp, "libsvdq.so")
        _run([HIPCC, "-shared", f"--offload-arch={ARCH}", "-fPIC", "-pthread", "-o", tmp_lib, *objs], verbose)
        staged = LIB + ".tmp"
        shutil.copyfile(tmp_lib, staged)
        os.replace(staged, LIB)
        return LIB
    finally:
        shutil.rmtree(tmp, ignore_errors=True)


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
