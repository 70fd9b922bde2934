"""The library driven from plain C through include/pc.h (tests/c_abi).

The program links libpcdp.so and the HIP runtime only: no Python, no torch.
Its expected values are closed forms (exact sums, the cancellation triple,
the LL identity, the all-gather concatenation) and status codes."""
import os
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
EXE = os.path.join(HERE, "c_abi", "pc_abi_check")


def exe():
    if not os.path.exists(EXE):
        pytest.skip("tests/c_abi/pc_abi_check is not built (run tests/c_abi/build.py)")
    return EXE


def test_c_program_links_the_library():
    out = subprocess.run(["ldd", exe()], check=True, capture_output=True, text=True).stdout
    assert "libpcdp.so" in out and "not found" not in out


def test_c_program_without_gpu_reports_it():
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present: the GPU test runs the program")
    r = subprocess.run([exe()], capture_output=True, text=True, timeout=60)
    assert r.returncode == 77, r.stdout + r.stderr


@pytest.mark.gpu
def test_c_program_checks_pass_on_gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    r = subprocess.run([exe()], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "pc_abi_check: OK" in r.stdout
