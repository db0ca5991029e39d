"""Build libpa.so (the HIP kernels and the C ABI of include/pa.h, and the
host-side block manager of include/pa_block_manager.h) for gfx950.

Each ``csrc/*.hip`` file is compiled by hipcc and each host-only
``csrc/*.cpp`` file by the host C++ compiler, in parallel, then linked into
``paged_kv_cache_400_amd/libpa.so`` next to this file.  Packed-FP32 VALU
instructions are disabled for all device code.
"""
import glob
import os
import subprocess
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
OBJ = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libpa.so")
ARCH = "gfx950"
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

CFLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # MFMA accumulators in ordinary VGPRs: the softmax rescales them with VALU
    # ops, which cannot read the accumulation registers directly
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    "-I", INCLUDE, "-I", CSRC,
]


HOST_CXX = os.environ.get("CXX", "g++")
HOST_FLAGS = ["-O2", "-std=c++17", "-fPIC", "-Wall", "-I", INCLUDE, "-I", "/opt/rocm/include",
              "-D__HIP_PLATFORM_AMD__"]


def sources():
    """HIP sources (device + host code, hipcc) and host-only C++ sources (g++)."""
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")) + glob.glob(os.path.join(CSRC, "*.cpp")))


def _compile(src):
    obj = os.path.join(OBJ, os.path.basename(src) + ".o")
    if src.endswith(".cpp"):
        subprocess.run([HOST_CXX, *HOST_FLAGS, "-c", src, "-o", obj], check=True)
    else:
        subprocess.run([HIPCC, *CFLAGS, "-c", src, "-o", obj], check=True)
    return obj


def build(verbose: bool = False) -> str:
    """Compile every HIP source and link libpa.so; returns its path."""
    os.makedirs(OBJ, exist_ok=True)
    srcs = sources()
    with ThreadPoolExecutor(max(1, min(len(srcs), os.cpu_count() or 1))) as ex:
        objs = list(ex.map(_compile, srcs))
    tmp = LIB + ".tmp"
    subprocess.run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp],
                   check=True)
    os.replace(tmp, LIB)
    if verbose:
        print(LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
