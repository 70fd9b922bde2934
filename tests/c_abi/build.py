"""Build tests/c_abi/pc_abi_check: a plain-C program that links
libpcdp.so and drives it through include/pc.h (no Python, no torch)."""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
SRC = os.path.join(HERE, "pc_abi_check.c")
OUT = os.path.join(HERE, "pc_abi_check")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def build(verbose: bool = False) -> str:
    libdir = os.path.join(ROOT, "collective_datapath_amd")
    tmp = OUT + ".tmp"
    cmd = ["gcc", "-std=c11", "-O2", "-Wall", "-Wextra", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(ROOT, "include"), "-I", os.path.join(ROCM, "include"), SRC,
           "-L", libdir, "-l:libpcdp.so", "-L", os.path.join(ROCM, "lib"), "-lamdhip64",
           "-Wl,-rpath,$ORIGIN/../../collective_datapath_amd", "-Wl,-rpath," + os.path.join(ROCM, "lib"),
           "-o", tmp]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(tmp, OUT)
    return OUT


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
