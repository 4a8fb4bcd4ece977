"""Sanitizer build for the CPU test of argument validation (tests/test_host_sanitizers.py):
libkvx with AddressSanitizer and UndefinedBehaviorSanitizer on its host code only (the device
code is compiled as usual and never run), and the plain C driver tests/c_abi/validate.c linked
against it. Host code only runs; no GPU is needed. Rebuilds when a source is newer."""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
sys.path.insert(0, ROOT)
from block_table_contiguous_amd import build as B  # noqa: E402

LIB = os.path.join(HERE, "libkvx_hostsan.so")
EXE = os.path.join(HERE, "validate")
DRIVER = os.path.join(HERE, "validate.c")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
# sanitizers for the host pass only: each flag follows its own -Xarch_host
HOST_SANITIZERS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined"]


def _stale(target, inputs):
    if not os.path.exists(target):
        return True
    t = os.path.getmtime(target)
    return any(os.path.getmtime(p) > t for p in inputs)


def build() -> str:
    sources = [os.path.join(B.CSRC, s) for s in B.SOURCES]
    headers = [os.path.join(B.INCLUDE, "kvx.h"), os.path.join(B.CSRC, "kvx_launch.h")]
    if _stale(LIB, sources + headers):
        flags = [f for f in B.HIP_FLAGS if f != "-O3"]
        cmd = [B.hipcc(), *flags, "-O1", "-g", "-fno-omit-frame-pointer", *HOST_SANITIZERS,
               f"-I{B.INCLUDE}", f"-I{B.CSRC}", *sources, "-shared", "-o", LIB + ".tmp"]
        subprocess.run(cmd, check=True)
        os.replace(LIB + ".tmp", LIB)
    if _stale(EXE, [LIB, DRIVER, headers[0]]):
        clang = os.path.join(ROCM, "llvm", "bin", "clang")
        cmd = [clang, "-std=c11", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
               "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__", f"-I{B.INCLUDE}",
               f"-I{os.path.join(ROCM, 'include')}", DRIVER, "-o", EXE + ".tmp", f"-L{HERE}", "-lkvx_hostsan",
               f"-L{os.path.join(ROCM, 'lib')}", "-lamdhip64", f"-Wl,-rpath,{HERE}",
               f"-Wl,-rpath,{os.path.join(ROCM, 'lib')}"]
        subprocess.run(cmd, check=True)
        os.replace(EXE + ".tmp", EXE)
    return EXE


if __name__ == "__main__":
    print(build())
