"""Build the HIP datapath library (libpcdp.so) for gfx950, in-tree.

Every source under csrc/ is compiled by its own hipcc process (in parallel)
into collective_datapath_amd/_build/, and the objects are linked into
collective_datapath_amd/libpcdp.so.  A second library, libpcdp_delay.so,
differs only in the flag-linked twoshot, built with injected pseudo-random
delays; only the tests load it.  The sources share no device symbols, so
no relocatable device code is needed.  Flags that matter for bit-exactness:
no fast-math, no fp contraction, and fp32 subnormals kept on the device.
Packed-fp32 instruction selection is switched off (plain v_add_f32 per
element).
"""
from __future__ import annotations

import glob
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
OBJ_DIR = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libpcdp.so")
DELAY_LIB = os.path.join(HERE, "libpcdp_delay.so")  # test-only variant, see build()
ARCH = "gfx950"

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-fvisibility=hidden", "-ffp-contract=off", "-fno-fast-math",
    "-fno-gpu-flush-denormals-to-zero",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-command-line-argument",
]


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)


def build(verbose: bool = False, out: str = LIB, extra_flags=()) -> str:
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    os.makedirs(OBJ_DIR, exist_ok=True)
    inc = f"-I{os.path.join(ROOT, 'include')}"
    jobs = []
    objs = []
    for src in sources():
        obj = os.path.join(OBJ_DIR, os.path.splitext(os.path.basename(src))[0] + ".o")
        objs.append(obj)
        jobs.append([hipcc, *HIPCC_FLAGS, *extra_flags, inc, "-c", src, "-o", obj])
    # The test-only delay-stress build of the flag-linked twoshot: the same
    # library with pc_linked.hip compiled with PC_LINKED_DELAY_STRESS.
    linked_src = os.path.join(CSRC, "pc_linked.hip")
    delay_obj = os.path.join(OBJ_DIR, "pc_linked_delay.o")
    jobs.append([hipcc, *HIPCC_FLAGS, *extra_flags, "-DPC_LINKED_DELAY_STRESS", inc, "-c", linked_src,
                 "-o", delay_obj])
    workers = max(1, min(len(jobs), int(os.environ.get("MAX_JOBS", os.cpu_count() or 1))))
    with ThreadPoolExecutor(max_workers=workers) as pool:
        for f in [pool.submit(_run, cmd, verbose) for cmd in jobs]:
            f.result()
    link = [hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC"]
    tmp = out + ".tmp"
    _run([*link, *objs, "-o", tmp], verbose)
    os.replace(tmp, out)
    delay_objs = [delay_obj if o.endswith(os.sep + "pc_linked.o") else o for o in objs]
    tmp = DELAY_LIB + ".tmp"
    _run([*link, *delay_objs, "-o", tmp], verbose)
    os.replace(tmp, DELAY_LIB)
    return out


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
