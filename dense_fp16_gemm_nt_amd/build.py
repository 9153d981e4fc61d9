"""Build the HIP library (gfx950) in-tree: dense_fp16_gemm_nt_amd/libgemm_f16_nt.so, and the
matrix-core calibration kernel the profiling tools use (libmfma_calib.so)."""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
SRC = os.path.join(PKG, "csrc", "gemm_f16_nt.hip")
LIB = os.path.join(PKG, "libgemm_f16_nt.so")
ARCH = "gfx950"

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
    # packed fp32 VALU forms stay off (the accumulators live in MFMA
    # registers; nothing here needs them)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    return "hipcc"


CALIB_SRC = os.path.join(PKG, "csrc", "mfma_calib.hip")
CALIB_LIB = os.path.join(PKG, "libmfma_calib.so")


def _compile(src: str, lib: str, verbose: bool) -> None:
    tmp = lib + ".tmp"
    cmd = [hipcc(), *HIPCC_FLAGS, "-o", tmp, src]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, lib)


CLIENT_SRC = os.path.join(ROOT, "tests", "c_client", "gemm_client.c")
CLIENT = os.path.join(ROOT, "tests", "c_client", "gemm_client")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def build_client(verbose: bool = False) -> str:
    """The plain C caller of the C-ABI that a GPU test runs: host code only,
    built with the system C compiler against the HIP runtime's C API."""
    cmd = ["gcc", "-O2", "-std=c11", "-Wall", "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROCM, "include"),
           "-I", os.path.join(ROOT, "include"), "-o", CLIENT + ".tmp", CLIENT_SRC, "-L", PKG, "-lgemm_f16_nt",
           "-L", os.path.join(ROCM, "lib"), "-lamdhip64", "-Wl,-rpath,$ORIGIN/../../dense_fp16_gemm_nt_amd",
           "-Wl,-rpath," + os.path.join(ROCM, "lib")]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(CLIENT + ".tmp", CLIENT)
    return CLIENT


def build(verbose: bool = False) -> str:
    """Compile the library, the matrix-core calibration kernel of the
    profiling tools and the C client of the tests (always recompiles);
    return the library's path."""
    _compile(SRC, LIB, verbose)
    _compile(CALIB_SRC, CALIB_LIB, verbose)
    build_client(verbose)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
