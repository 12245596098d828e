"""Build the Conv3D HIP library for gfx950 in-tree.

Produces convolution_video_vae_amd/libconv3d_mi355x.so from csrc/ with hipcc
(cross-compiles without a GPU). Packed-fp32 instructions are disabled for all
device code.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
OUT = os.path.join(HERE, "libconv3d_mi355x.so")
BUILD = os.path.join(HERE, "_build")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
IGEMM_PARTS = 8


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), file=sys.stderr)
    subprocess.run(cmd, check=True)


def build(verbose: bool = False) -> str:
    """Compile every source (in parallel: the implicit-GEMM file dominates)
    and link the shared library."""
    os.makedirs(BUILD, exist_ok=True)
    jobs, objs = [], []
    # The implicit-GEMM configurations compile as IGEMM_PARTS units of one
    # source (each instantiates every IGEMM_PARTS-th configuration).
    units = [("conv3d_igemm", [f"-DCONV3D_PART={k}", f"-DCONV3D_NPARTS={IGEMM_PARTS}"],
              f"conv3d_igemm_{k}") for k in range(IGEMM_PARTS)]
    units += [("conv3d_kernels", [], "conv3d_kernels"), ("conv3d_norm", [], "conv3d_norm")]
    for name, defs, oname in units:
        obj = os.path.join(BUILD, oname + ".o")
        jobs.append([HIPCC, "-O3", "-std=c++17", f"--offload-arch={ARCH}", "-fPIC", "-c",
                     *DEVICE_FLAGS, *defs, "-Wall", os.path.join(CSRC, name + ".hip"), "-o", obj])
        objs.append(obj)
    aobj = os.path.join(BUILD, "conv3d_api.o")
    jobs.append(["g++", "-O2", "-std=c++17", "-fPIC", "-c", "-Wall", "-Wextra",
                 os.path.join(CSRC, "conv3d_api.cpp"), "-o", aobj])
    procs = []
    for cmd in jobs:
        if verbose:
            print(" ".join(cmd), file=sys.stderr)
        procs.append((cmd, subprocess.Popen(cmd)))
    failed = [cmd for cmd, p in procs if p.wait() != 0]
    if failed:
        raise subprocess.CalledProcessError(1, failed[0])
    _run([HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, aobj, "-o", OUT + ".tmp"],
         verbose)
    os.replace(OUT + ".tmp", OUT)
    return OUT


if __name__ == "__main__":
    print(build(verbose=True))
