"""pc_twoshot_linked_static (the flag-linked twoshot with the library's static
workspace, for callers that cannot allocate) against pc_twoshot_linked with
a caller-owned workspace: bit-identical outputs on consecutive calls, the
second smaller than the first, and no abandoned wait."""
import os

import numpy as np
import pytest
import torch

from collective_datapath_amd import synth

pytestmark = pytest.mark.gpu

THREADS = max(1, min(16, os.cpu_count() or 1))


def say(*a):
    print("[case]", *a, flush=True)


@pytest.fixture(scope="module")
def B():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from collective_datapath_amd import binding
    return binding


@pytest.fixture(scope="module")
def D():
    import devbuf
    return devbuf


def test_static_workspace_matches_caller_workspace(B, D, orc):
    # 8 ranks x 5 MiB (320 tiles, several per workgroup), then 8 ranks x
    # 8 KiB (8 tiles), then a ragged 3-rank call.
    shapes = [(8, 8 * 8 * 1024 * 40), (8, 8 * 512), (3, 3 * 8 * 1001)]
    gave_up = torch.zeros(1, dtype=torch.int64, device=D.DEV)
    for i, (n, k) in enumerate(shapes):
        say("linked static", i, n, k)
        xs = [synth.normal_bf16(2300 + i, 0, r, k) for r in range(n)]
        ins = [D.up(x) for x in xs]
        ref = [D.filled(k, 0xFFFF) for _ in range(n)]
        ws = torch.zeros(B.pc_twoshot_linked_workspace_bytes(n, k) // 8, dtype=torch.int64, device=D.DEV)
        B.pc_twoshot_linked(ins, ref, k, ws)
        got = [D.filled(k, 0xFFFF) for _ in range(n)]
        B.pc_twoshot_linked_static(ins, got, k, gave_up if i != 2 else None)
        want = orc.reduce(xs, threads=THREADS)
        for r in range(n):
            g, w = D.down(got[r], np.uint16), D.down(ref[r], np.uint16)
            assert np.array_equal(g, w), (i, r, int(np.count_nonzero(g != w)))
            assert np.array_equal(g, want), (i, r)
        assert int(D.down(gave_up, np.uint64)[0]) == 0, i
        assert int(D.down(ws, np.uint64)[B.PC_LINKED_STATUS_WORD]) == 0, i


def test_static_workspace_first_call_inside_a_capture(B):
    """A fresh process whose first pc_twoshot_linked_static call is captured
    in a graph: the static workspace's address is looked up during capture,
    and every replay is exact."""
    import subprocess
    import sys
    here = os.path.dirname(os.path.abspath(__file__))
    r = subprocess.run([sys.executable, os.path.join(here, "linked_static_capture_first.py")],
                       capture_output=True, text=True, timeout=240)
    assert r.returncode == 0 and "OK" in r.stdout, (r.stdout[-2000:], r.stderr[-2000:])
