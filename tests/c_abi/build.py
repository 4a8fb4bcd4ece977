"""Compile the plain C consumers of libkvx (tests/c_abi/roundtrip.c and rest.c) with gcc
against include/kvx.h and the in-tree libkvx.so. Host code only; no GPU is needed to build
them."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
PROGRAMS = ("roundtrip", "rest")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def build() -> list:
    lib_dir = os.path.join(ROOT, "block_table_contiguous_amd")
    out = []
    for name in PROGRAMS:
        exe = os.path.join(HERE, name)
        cmd = ["gcc", "-std=c11", "-O2", "-Wall", "-Wextra", "-D__HIP_PLATFORM_AMD__",
               f"-I{os.path.join(ROOT, 'include')}", f"-I{os.path.join(ROCM, 'include')}",
               os.path.join(HERE, name + ".c"), "-o", exe + ".tmp",
               f"-L{lib_dir}", "-lkvx", f"-L{os.path.join(ROCM, 'lib')}", "-lamdhip64",
               "-Wl,-rpath,$ORIGIN/../../block_table_contiguous_amd", f"-Wl,-rpath,{os.path.join(ROCM, 'lib')}"]
        subprocess.run(cmd, check=True)
        os.replace(exe + ".tmp", exe)
        out.append(exe)
    return out


if __name__ == "__main__":
    print("\n".join(build()))
