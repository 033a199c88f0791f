"""Build liblscd.so in-tree with hipcc for gfx950.

    python unstructured_sparse_skinny_amd/build.py

Every source is compiled to an object under _build/ (in parallel), then linked into
unstructured_sparse_skinny_amd/liblscd.so.  The packed-fp32 target feature is switched
off for all device code; the host pass warns that it does not know the feature, which is
harmless.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "liblscd.so")
BUILD_DIR = os.path.join(HERE, "_build")
# The kernel families are separate translation units so that they compile in parallel.
SOURCES = ["csrc/lscd_skinny64.hip", "csrc/lscd_skinny32.hip", "csrc/lscd_skinny16.hip", "csrc/lscd_three_level.hip",
           "csrc/lscd_bitmap.hip", "csrc/lscd_wide.hip", "csrc/lscd_kernels.hip", "csrc/lscd_encode_dev.hip",
           "csrc/lscd_api.cpp", "csrc/lscd_linear.cpp", "csrc/lscd_pack.cpp"]
# Device sources of each format's product (their hash identifies the kernels behind a committed
# measurement of that format; the split-K reduction and the shared helpers belong to all).
_COMMON_DEVICE = ["csrc/lscd_internal.h", "csrc/lscd_device.h", "csrc/lscd_kernels.hip"]
DEVICE_SOURCES_BY_FORMAT = {
    "tiled-csl": _COMMON_DEVICE + ["csrc/lscd_skinny.h", "csrc/lscd_skinny16.hip", "csrc/lscd_skinny32.hip",
                                   "csrc/lscd_skinny64.hip", "csrc/lscd_wide.hip"],
    "bitmap": _COMMON_DEVICE + ["csrc/lscd_bitmap.hip"],
    "three-level": _COMMON_DEVICE + ["csrc/lscd_three_level.hip"],
}
DEVICE_SOURCES = sorted({f for v in DEVICE_SOURCES_BY_FORMAT.values() for f in v})
ARCH = os.environ.get("LSCD_OFFLOAD_ARCH", "gfx950")


def _hipcc() -> str:
    for cand in (os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc"), shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build liblscd.so)")


def _flags():
    return [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-pthread",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            # MFMA results stay in ordinary VGPRs (no copies through the accumulator registers)
            "-mllvm", "-amdgpu-mfma-vgpr-form",
                "-I", os.path.join(ROOT, "include")]


def build(verbose: bool = False, pkg_dir: str = HERE) -> str:
    """Compile the sources of `pkg_dir` (default: this package) into `pkg_dir`/liblscd.so."""
    hipcc = _hipcc()
    build_dir = os.path.join(pkg_dir, "_build")
    lib = os.path.join(pkg_dir, "liblscd.so")
    os.makedirs(build_dir, exist_ok=True)

    def compile_one(src):
        obj = os.path.join(build_dir, os.path.basename(src) + ".o")
        cmd = [hipcc, *_flags(), "-I", os.path.join(pkg_dir, "csrc"), "-c", os.path.join(pkg_dir, src),
               "-o", obj]
        if src.endswith(".cpp"):
            cmd[1:1] = ["-x", "hip"]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}\n{r.stderr}")
        if verbose:
            print(" ".join(cmd))
        return obj

    with ThreadPoolExecutor(max_workers=min(len(SOURCES), os.cpu_count() or 4)) as ex:
        objs = list(ex.map(compile_one, SOURCES))
    tmp = lib + ".tmp"
    rocm_lib = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "lib")
    # rocBLAS (dense path of lscd_linear): when torch is loaded first, its copy (same soname)
    # is the one bound.
    cmd = [hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-pthread", *objs, "-L", rocm_lib, "-lrocblas", "-lhipblaslt",
           "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, lib)
    return lib


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
