"""Build ``libosx.so`` (HIP kernels + C ABI) in-tree for gfx950 with hipcc.

    python -m online_softmax_02_amd.build [--asm]

Objects go to ``online_softmax_02_amd/_build/``; the shared library is written
next to this file.  ``--asm`` also keeps the gfx950 assembly of every kernel
file in ``_build/`` for inspection.

Each build also writes ``libosx_debug_sync.so``: the same sources with
``OSX_DEBUG_SYNC=1``, which adds a full wait and a workgroup barrier at every
LDS stage boundary (``csrc/common.hpp``).  Its results must equal the default
library's bit for bit (``tests/test_gpu_debug_sync.py``).
"""
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libosx.so")
DEBUG_SYNC_LIB = os.path.join(HERE, "libosx_debug_sync.so")

SOURCES = [
    "abi.cpp",
    "softmax_rows.hip",
    "softmax_3pass.hip",
    "attn_prefill_bf16.hip",
    "attn_prefill_f32.hip",
    "attn_decode_bf16.hip",
    "attn_unfused.hip",
    "read_probe.hip",
    "noalloc.hip",
]

ARCH = "gfx950"
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
    # Packed fp32 VALU ops stay off: the kernels use scalar fp32 VALU and MFMA only.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build the HIP library)")


def _compile(src: str, asm: bool, build_dir: str, extra: list) -> str:
    obj = os.path.join(build_dir, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), *FLAGS, *extra, "-c", os.path.join(CSRC, src), "-o", obj]
    if src.endswith(".hip"):
        cmd[1:1] = ["-x", "hip"]
        # Device code only: no value in the kernels is NaN (inputs with NaN are
        # outside the contract, and every -inf - -inf is guarded), which lets
        # fmaxf skip its operand canonicalisation.  Host code keeps IEEE NaN
        # semantics for its argument checks.
        cmd += ["-Xarch_device", "-fno-honor-nans"]
    if asm and src.endswith(".hip"):
        cmd += ["--save-temps"]
    r = subprocess.run(cmd, cwd=build_dir, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile of {src} failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def _build_one(lib: str, build_dir: str, extra: list, asm: bool, verbose: bool) -> str:
    os.makedirs(build_dir, exist_ok=True)
    with ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(lambda s: _compile(s, asm, build_dir, extra), SOURCES))
    tmp = lib + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-Wl,--no-undefined", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, lib)
    if verbose:
        print(f"built {lib}")
    return lib


def build(asm: bool = False, verbose: bool = False) -> str:
    """Build libosx.so, then libosx_debug_sync.so; returns the first's path."""
    _build_one(LIB, BUILD, [], asm, verbose)
    _build_one(DEBUG_SYNC_LIB, os.path.join(BUILD, "debug_sync"), ["-DOSX_DEBUG_SYNC=1"], False, verbose)
    return LIB


if __name__ == "__main__":
    build(asm="--asm" in sys.argv, verbose=True)
