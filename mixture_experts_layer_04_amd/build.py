"""Build libmoe.so (all HIP kernels + the C ABI) for gfx950 with hipcc.

Usage: python -m mixture_experts_layer_04_amd.build   (or build() from Python)

Every .hip file under csrc/ is compiled to an object in parallel and linked
into mixture_experts_layer_04_amd/libmoe.so next to this file.
"""

import concurrent.futures
import glob
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(os.path.dirname(HERE), "include")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libmoe.so")
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", shutil.which("hipcc") or "/opt/rocm/bin/hipcc")

COMMON = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-munsafe-fp-atomics",
    # matrix-core accumulators in VGPRs: in the AGPR form the register
    # allocator copies the tiled GEMMs' accumulators between the two files on
    # every K step
    "-mllvm", "-amdgpu-mfma-vgpr-form=1",
    "-I", INCLUDE, "-I", CSRC,
]


def _source_hash():
    sys.path.insert(0, os.path.dirname(HERE))
    try:
        from mixture_experts_layer_04_amd._lib import source_hash
    finally:
        sys.path.pop(0)
    return source_hash()


def _compile(src, defines=()):
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [HIPCC, *COMMON, *defines, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    return obj


def build(verbose=False):
    os.makedirs(BUILD, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    jobs = min(len(srcs), int(os.environ.get("MAX_JOBS", "8")))
    # the library reports the hash of the sources it was built from
    # (moe_source_hash); the loader refuses a library whose hash differs
    defines = [f'-DMOE_SOURCE_HASH="{_source_hash()}"']
    with concurrent.futures.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(lambda s: _compile(s, defines), srcs))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
