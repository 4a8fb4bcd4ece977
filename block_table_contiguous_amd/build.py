"""Build libkvx.so (the HIP library behind the C ABI in include/kvx.h) for gfx950, in-tree.

    python -m block_table_contiguous_amd.build          # compile
    python -m block_table_contiguous_amd.build --asm    # also keep the device assembly

Runs hipcc cross-compilation; no GPU is needed.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libkvx.so")
SOURCES = ["kvx_api.hip", "kvx_kernels.hip", "kvx_signal.hip"]
ARCH = "gfx950"

# Packed-FP32 instructions are disabled for all device code (the kernels do no float
# arithmetic, but the flag keeps the compiler from ever forming them).
HIP_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


def hipcc() -> str:
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found; ROCm is required to build libkvx")
    return path


def build(asm_dir: str | None = None, verbose: bool = False) -> str:
    """Compile every source and link libkvx.so next to this file. Always recompiles."""
    cc = hipcc()
    objs = []
    tmp = os.path.join(PKG, "_build")
    os.makedirs(tmp, exist_ok=True)
    for src in SOURCES:
        obj = os.path.join(tmp, src.replace(".hip", ".o"))
        cmd = [cc, *HIP_FLAGS, f"-I{INCLUDE}", f"-I{CSRC}", "-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.run(cmd, check=True)
        objs.append(obj)
        if asm_dir:
            os.makedirs(asm_dir, exist_ok=True)
            out = os.path.join(asm_dir, src.replace(".hip", f"-{ARCH}.s"))
            subprocess.run([cc, *HIP_FLAGS, f"-I{INCLUDE}", f"-I{CSRC}", "--cuda-device-only", "-S",
                            os.path.join(CSRC, src), "-o", out], check=True)
    tmp_lib = LIB + ".tmp"
    cmd = [cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp_lib]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp_lib, LIB)
    return LIB


if __name__ == "__main__":
    # --asm [DIR]: also write each source's gfx950 assembly (default: _build/asm beside this file)
    asm = None
    if "--asm" in sys.argv:
        i = sys.argv.index("--asm")
        given = sys.argv[i + 1] if i + 1 < len(sys.argv) and not sys.argv[i + 1].startswith("-") else None
        asm = given or os.path.join(os.path.dirname(os.path.abspath(__file__)), "_build", "asm")
    print(build(asm_dir=asm, verbose=True))
