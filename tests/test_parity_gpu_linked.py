"""The flag-linked twoshot's failure contract and a delay-injection stress.

Give-up: include/pc.h promises that a wait that gives up adds its tiles to
workspace[PC_LINKED_STATUS_WORD], skips their copies into the non-owner
outputs and still ends.  The test forces it from the host, with no kernel
fault or hang: in a fresh zeroed workspace, workgroup 0's call counter is
offset, so workgroup 0 stamps its flags with an epoch its consumer never
waits for and waits for an epoch its producer never stamps; the poll limit
word bounds each wait to a few thousand polls.  (flash-comm, Section 4.4:
bounded polling, then explicit verification.)

Stress: libpcdp_delay.so is the same library with the flag-linked twoshot
built to sleep a pseudo-random time, different per workgroup, wave and
call, before its phase-1 stores, before its flags are published and before
its phase-2 reads, so the release/acquire hand-off between workgroups is
exercised at timings the natural schedule does not produce (flash-comm,
Section 2.2: data published before it is consumed, phases ordered).  Every
call is compared bit for bit with the oracle, and the run stops at the
first difference or abandoned wait.
"""
import ctypes
import os
import time

import numpy as np
import pytest
import torch

from collective_datapath_amd import synth

pytestmark = pytest.mark.gpu

THREADS = max(1, min(16, os.cpu_count() or 1))
HERE = os.path.dirname(os.path.abspath(__file__))
DELAY_LIB = os.path.join(os.path.dirname(HERE), "collective_datapath_amd", "libpcdp_delay.so")


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


def slice_tile_chunks(s, j, nslice, tile):
    """Chunk range [lo, hi) of tile j of slice s: tiles on the 8-chunk
    (128-byte) grid of the buffer, clipped to the slice (as pc.h states for
    every twoshot form)."""
    start, end = s * nslice, (s + 1) * nslice
    lo = (start & ~7) + j * tile
    hi = lo + tile
    return max(lo, start), min(hi, end)


def test_twoshot_linked_gives_up_and_counts(B, D, orc):
    # 8 ranks x 5 MiB: slices of 40,960 chunks in tiles of 1,024 chunks, 40
    # tiles per slice, 320 tiles.  Workgroup w folds tiles w and w + 256 and
    # copies out tiles w + 128 (w < 128) or w - 128 (w >= 128, and w + 128).
    n, nslice, tile = 8, 40960, 1024
    k = n * nslice * 8
    tiles_per_slice = nslice // tile
    xs = [synth.uniform_bf16(2100, 0, r, k) for r in range(n)]
    ins = [D.up(x) for x in xs]
    outs = [D.filled(k, 0xFFFF) for _ in range(n)]
    ws = torch.zeros(B.pc_twoshot_linked_workspace_bytes(n, k) // 8, dtype=torch.int64, device=D.DEV)
    ws[0] = 5                                   # workgroup 0 runs five calls ahead
    # A wait gives up after 4,096 polls: milliseconds, so the planted waits
    # end soon, while every producer that really runs publishes long before
    # (64 polls, a few microseconds, also cut short waits for producers that
    # merely started late).
    ws[B.PC_LINKED_POLL_LIMIT_WORD] = 4096
    say("linked give-up", n, k)
    t0 = time.perf_counter()
    B.pc_twoshot_linked(ins, outs, k, ws)
    torch.cuda.synchronize()                     # every workgroup has ended
    took = time.perf_counter() - t0
    # Workgroup 0 stamps tiles 0 and 256 with epoch 6; their consumer,
    # workgroup 128, waits for epoch 1 and abandons both.  Workgroup 0 itself
    # copies tile 128, stamped 1 by workgroup 128, and waits for 6: abandoned.
    skipped = [0, 128, 256]
    w = D.down(ws, np.uint64)
    assert w[B.PC_LINKED_STATUS_WORD] == len(skipped)
    assert w[0] == 6 and np.all(w[1:B.PC_LINKED_GROUPS] == 1)
    want = orc.reduce(xs, threads=THREADS)
    for r, o in enumerate(outs):
        got = D.down(o, np.uint16)
        expect = want.copy()
        for t in skipped:
            s, j = divmod(t, tiles_per_slice)
            lo, hi = slice_tile_chunks(s, j, nslice, tile)
            if r != s:                           # the non-owner copy was skipped
                expect[lo * 8:hi * 8] = 0xFFFF
        assert np.array_equal(got, expect), (r, int(np.count_nonzero(got != expect)))
    # The status word is a running sum: a second call on the same workspace
    # (workgroup 0 still ahead) abandons the same three tiles again.
    B.pc_twoshot_linked(ins, outs, k, ws)
    torch.cuda.synchronize()
    assert int(D.down(ws, np.uint64)[B.PC_LINKED_STATUS_WORD]) == 2 * len(skipped)
    assert took < 60, took


def _delay_lib(B):
    if not os.path.exists(DELAY_LIB):
        pytest.fail(f"{DELAY_LIB} is not built (collective_datapath_amd/build.py builds it)")
    lib = ctypes.CDLL(DELAY_LIB)
    lib.pc_twoshot_linked.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p, ctypes.c_size_t,
                                      ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
    lib.pc_twoshot_linked.restype = ctypes.c_int
    lib.pc_abi_version.restype = ctypes.c_int
    assert lib.pc_abi_version() == B.PC_ABI_VERSION
    return lib


def _delay_call(lib, ins, outs, k, ws):
    n = len(ins)
    pin = (ctypes.c_void_p * n)(*[t.data_ptr() for t in ins])
    pout = (ctypes.c_void_p * n)(*[t.data_ptr() for t in outs])
    stream = torch.cuda.current_stream().cuda_stream
    st = lib.pc_twoshot_linked(pin, n, pout, k, ws.data_ptr(), ws.numel() * 8, stream)
    assert st == 0, st


def test_twoshot_linked_under_delay_stress(B, D, orc):
    lib = _delay_lib(B)
    # Decode sizes (one and two chunks per lane), a ragged 3-rank shape, a
    # size past 256 tiles (a workgroup folds and copies several tiles) and
    # the non-temporal large-size kernel.  Each shape runs several calls on
    # one workspace, so epochs advance under the delays.
    shapes = [(8, 8 * 512), (8, 8 * 65536), (3, 3 * 8 * 1001), (8, 8 * 8 * 1024 * 40), (5, 5 * 8 * 256 * 3),
              (8, 8 * 8 * 1024 * 400)]
    for i, (n, k) in enumerate(shapes):
        xs = [synth.normal_bf16(2200 + i, 0, r, k) for r in range(n)]
        ins = [D.up(x) for x in xs]
        want = orc.reduce(xs, threads=THREADS)
        ws = torch.zeros(B.pc_twoshot_linked_workspace_bytes(n, k) // 8, dtype=torch.int64, device=D.DEV)
        calls = 3 if k * 2 > (32 << 20) else 6
        for c in range(calls):
            say("linked delay stress", n, k, "call", c)
            outs = [D.filled(k, 0xFFFF) for _ in range(n)]
            _delay_call(lib, ins, outs, k, ws)
            w = D.down(ws, np.uint64)
            assert w[B.PC_LINKED_STATUS_WORD] == 0, (n, k, c)
            assert np.all(w[:B.PC_LINKED_GROUPS] == c + 1), (n, k, c)
            for r, o in enumerate(outs):
                got = D.down(o, np.uint16)
                assert np.array_equal(got, want), (n, k, c, r, int(np.count_nonzero(got != want)))
        del ins, outs, ws
        torch.cuda.empty_cache()


def test_delay_stress_build_really_delays(B, D):
    """The stress library's calls take markedly longer than the product's
    on the same workload, so its delays are compiled in."""
    lib = _delay_lib(B)
    n, k = 8, 8 * 512
    ins = [D.filled(k, 0x3F80) for _ in range(n)]
    outs = [D.filled(k, 0) for _ in range(n)]
    ws_a = torch.zeros(B.pc_twoshot_linked_workspace_bytes(n, k) // 8, dtype=torch.int64, device=D.DEV)
    ws_b = torch.zeros_like(ws_a)

    def timed(fn, reps=20):
        fn()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(reps):
            fn()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) * 1000.0 / reps
    plain = timed(lambda: B.pc_twoshot_linked(ins, outs, k, ws_a))
    stressed = timed(lambda: _delay_call(lib, ins, outs, k, ws_b))
    say("linked plain", round(plain, 2), "us, stressed", round(stressed, 2), "us")
    assert stressed > 5 * plain, (plain, stressed)
