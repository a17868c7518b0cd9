"""Build the HIP library liblime.so for gfx950, in-tree.

    python decoupled_linear_link_amd/build.py     (or __graft_entry__.build())

Run it by path: importing the package first would load the library being
rebuilt.

hipcc cross-compiles without a GPU.  The library links the HIP runtime that
PyTorch ships (with an rpath to it), so a process that also uses torch holds
a single HIP runtime.
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIBDIR = os.path.join(PKG, "_lib")
LIB = os.path.join(LIBDIR, "liblime.so")
SOURCES = ["lime_api.hip"]
ARCH = "gfx950"


def _torch_libdir() -> str:
    import importlib.util
    spec = importlib.util.find_spec("torch")
    if spec is None or not spec.origin:
        raise RuntimeError("torch is needed to locate its HIP runtime")
    return os.path.join(os.path.dirname(spec.origin), "lib")


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    return os.path.join(rocm, "bin", "hipcc")


def compile_flags() -> list[str]:
    return [
        f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
        "-mcode-object-version=5",
        # keep the compiler from forming packed fp32 instructions
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        # matrix-core accumulators in ordinary VGPRs: no accvgpr moves
        # around every product, and the attention kernels fit two waves per
        # SIMD
        "-mllvm", "-amdgpu-mfma-vgpr-form=1",
        "-I", os.path.join(ROOT, "include"), "-I", CSRC,
        "-Wall", "-Wno-unused-function",
    ]


def build(verbose: bool = False) -> str:
    os.makedirs(LIBDIR, exist_ok=True)
    tl = _torch_libdir()
    tmp = LIB + ".tmp"
    cmd = [hipcc(), *compile_flags(), "-shared", "-o", tmp,
           *[os.path.join(CSRC, s) for s in SOURCES],
           f"-L{tl}", f"-Wl,-rpath,{tl}", "-lamdhip64"]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    errs = "\n".join(l for l in (r.stderr or "").splitlines()
                     if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed ({r.returncode}):\n{errs}")
    if errs.strip() and verbose:
        print(errs, file=sys.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
