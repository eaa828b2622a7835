"""Build libsa.so in-tree with hipcc for gfx950 (MI355X).

Usage: ``python -m prototype_attention_compression_amd.build`` or
``build_library()`` from Python.  Each ``csrc/*.hip`` file compiles to an
object under ``_build/`` (ignored by git), then all link into
``prototype_attention_compression_amd/libsa.so``.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libsa.so")
ARCH = "gfx950"

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    "-Wno-unused-function",
    # keep packed fp32 VALU ops out of the device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
    "-I", CSRC,
]


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libsa)")


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


# per-file code generation options: keep MFMA accumulators in ordinary VGPRs
# (the VALU reads them directly, no accumulator-register copies)
FILE_FLAGS = {
    "sa_pass1.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
    "sa_pass2.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
    "sa_pass1q.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
}


def _compile(src: str, hipcc: str, verbose: bool) -> str:
    obj = os.path.join(BUILD, os.path.basename(src)[:-4] + ".o")
    cmd = [hipcc, *HIPCC_FLAGS, *FILE_FLAGS.get(os.path.basename(src), []), "-c", src, "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    out = (res.stdout + res.stderr).strip()
    # the host pass does not know the device-only feature flag: harmless
    lines = [ln for ln in out.splitlines() if "packed-fp32-ops" not in ln]
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n" + "\n".join(lines))
    if verbose and lines:
        print("\n".join(lines))
    return obj


def _check_kernel_stubs(lib: str) -> None:
    """Fail if a kernel's host launch stub was left undefined.

    clang can drop a kernel template's host-side instantiation without any
    diagnostic; the shared library then links but cannot be loaded.
    """
    nm = shutil.which("nm")
    if nm is None:
        return
    res = subprocess.run([nm, "-D", "--undefined-only", lib], capture_output=True, text=True)
    missing = [ln.split()[-1] for ln in res.stdout.splitlines() if "__device_stub__" in ln]
    if missing:
        raise RuntimeError("kernel launch stubs undefined in the linked library: " + ", ".join(missing))


def build_library(verbose: bool = False) -> str:
    """Compile every HIP source and link libsa.so.  Returns the library path."""
    hipcc = _hipcc()
    os.makedirs(BUILD, exist_ok=True)
    srcs = sources()
    with ThreadPoolExecutor(min(8, len(srcs))) as ex:
        objs = list(ex.map(lambda s: _compile(s, hipcc, verbose), srcs))
    tmp = LIB + ".tmp"
    cmd = [hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("link failed:\n" + res.stdout + res.stderr)
    _check_kernel_stubs(tmp)
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build_library(verbose="-q" not in sys.argv)
