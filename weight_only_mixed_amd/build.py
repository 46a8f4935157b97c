"""Build libqpack.so (the HIP library behind include/qpack.h) for gfx950, in-tree.

Every .hip under csrc/ is compiled to an object with hipcc (and every host-only .cpp with g++),
then linked into one shared library next to this file.  The quantizer is compiled without floating-point contraction so
its fp32 arithmetic is exactly the stated sequence of IEEE operations.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor
from pathlib import Path

PKG = Path(__file__).resolve().parent
ROOT = PKG.parent
CSRC = PKG / "csrc"
OBJ = PKG / "_build"
LIB = PKG / "libqpack.so"
ARCH = "gfx950"

COMMON = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-Wno-unused-variable",
    "-I", str(ROOT / "include"), "-I", str(CSRC),
]
# The GEMV's matrix-core results feed vector fmas right away: with the VGPR form of MFMA
# they are written where the fmas read them, instead of accumulation registers copied over
# one by one (eight copies per k-tile in the 4-wave kernels).
PER_FILE = {"quantize.hip": ["-ffp-contract=off"], "quant_fp8.hip": ["-ffp-contract=off"], "kvattn.hip": ["-ffp-contract=off", "-mllvm", "-amdgpu-mfma-vgpr-form=1"], "qmm_small.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"]}


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    return os.path.join(rocm, "bin", "hipcc")


# Host-only sources (.cpp): plain C++ (g++, OpenMP), no device code.  Vector code is selected
# per function with target attributes, so the objects run on any x86-64 host.
HOST = ["g++", "-O3", "-std=c++17", "-fPIC", "-Wall", "-fopenmp", "-I", str(ROOT / "include"), "-I", str(CSRC)]


def _compile(src: Path) -> Path:
    obj = OBJ / (src.stem + ".o")
    if src.suffix == ".cpp":
        cmd = [*HOST, "-c", str(src), "-o", str(obj)]
    else:
        cmd = [hipcc(), *COMMON, *PER_FILE.get(src.name, []), "-c", str(src), "-o", str(obj)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src.name}:\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = False) -> Path:
    OBJ.mkdir(exist_ok=True)
    srcs = sorted(CSRC.glob("*.hip")) + sorted(CSRC.glob("*.cpp"))
    jobs = min(len(srcs), max(1, min(16, os.cpu_count() or 1)))
    with ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(_compile, srcs))
    tmp = LIB.with_suffix(".so.tmp")
    cmd = [hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", *map(str, objs), "-lgomp", "-o", str(tmp)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
