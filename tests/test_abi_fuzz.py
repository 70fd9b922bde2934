"""Property-based check of the C ABI's argument admission (host logic only).

Every generated call is valid except for at most one defect, drawn from the
errors include/pc.h documents for that call, and its status must be exactly
the documented one.  A size of zero is a no-op whose pointers are not
examined, so a pointer defect in an empty call must still return PC_OK.

The addresses are fake and never dereferenced: a call with no defect and a
nonzero size would launch, so this module runs only where no GPU is visible,
and there such a call must return PC_EHIP (the launch is refused).
"""
import pytest

pytest.importorskip("hypothesis")
torch = pytest.importorskip("torch")
from hypothesis import HealthCheck, given, settings  # noqa: E402
from hypothesis import strategies as st  # noqa: E402

from collective_datapath_amd import binding as B  # noqa: E402



def hip_device_count():
    """Devices the HIP runtime the library uses can see (torch's view can
    differ, e.g. a CPU-only torch on a GPU machine)."""
    import ctypes
    runtimes = sorted(B._hip_runtimes())
    if not runtimes:
        return 0
    count = ctypes.c_int(0)
    status = ctypes.CDLL(runtimes[0]).hipGetDeviceCount(ctypes.byref(count))
    return count.value if status == 0 else 0


pytestmark = pytest.mark.skipif(torch.cuda.is_available() or hip_device_count() > 0,
                                reason="valid calls would launch on fake addresses: CPU-only module")

BASE = 0x7F0000000000
SPAN = 1 << 38            # far apart: no two slots overlap at any legal size
MAX = 1 << 34             # PC_MAX_ELEMS
# Derandomized, so every run checks the same examples and a failure reproduces.
SETTINGS = settings(max_examples=500, deadline=None, derandomize=True,
                    suppress_health_check=[HealthCheck.too_slow])


def slot(i):
    return BASE + i * SPAN


def ran(k):
    """Status of a defect-free call: a launch (refused here) or a no-op."""
    return B.PC_EHIP if k else B.PC_OK


def ptr_defect(k, status):
    """A pointer defect is only seen when the call has work to do."""
    return status if k else B.PC_OK


# ---- pc_reduce ------------------------------------------------------------------

@SETTINGS
@given(n=st.integers(1, 8), kq=st.integers(0, 1 << 22), j=st.integers(0, 7), off=st.integers(1, 15),
       defect=st.sampled_from(["none", "n0", "n9", "bad_order", "k_big", "k_odd", "null_in", "mis_in",
                               "null_out", "mis_out", "overlap_out", "in_place", "order_ok"]))
def test_reduce_admission(n, kq, j, off, defect):
    k = 8 * kq
    ins = [slot(r) for r in range(n)]
    out, order, want = slot(9), None, ran(k)
    r = j % n
    if defect == "n0":
        ins, want = [], B.PC_EINVAL
    elif defect == "n9":
        ins, want = [slot(i) for i in range(9)], B.PC_EINVAL
    elif defect == "bad_order":
        order = list(range(n))
        order[r] = (r + 1) % n if n > 1 else 1     # a duplicate, or out of range at n = 1
        want = B.PC_EINVAL
    elif defect == "order_ok":
        order = list(reversed(range(n)))
    elif defect == "k_big":
        k, want = MAX + 8, B.PC_EINVAL
    elif defect == "k_odd":
        k, want = min(k + 1 + j % 7, MAX - 1), B.PC_EALIGN     # 1..7 past a multiple of 8
    elif defect == "null_in":
        ins[r], want = 0, ptr_defect(k, B.PC_EINVAL)
    elif defect == "mis_in":
        ins[r] += off
        want = ptr_defect(k, B.PC_EALIGN)
    elif defect == "null_out":
        out, want = 0, ptr_defect(k, B.PC_EINVAL)
    elif defect == "mis_out":
        out, want = out + off, ptr_defect(k, B.PC_EALIGN)
    elif defect == "overlap_out" and k > 8:
        out, want = ins[r] + 16, B.PC_EINVAL
    elif defect == "in_place":
        out = ins[r]
    assert B.pc_reduce(ins, out, k, order=order, stream=0, check=False) == want


# ---- pc_copy ----------------------------------------------------------------------

@SETTINGS
@given(q=st.integers(0, 1 << 30), off=st.integers(1, 15), j=st.integers(1, 15),
       defect=st.sampled_from(["none", "null_dst", "null_src", "mis_dst", "mis_src", "odd", "big",
                               "overlap", "alias"]))
def test_copy_admission(q, off, j, defect):
    nbytes, dst, src = 16 * q, slot(1), slot(0)
    want = ran(nbytes)
    if defect == "null_dst":
        dst, want = 0, ptr_defect(nbytes, B.PC_EINVAL)
    elif defect == "null_src":
        src, want = 0, ptr_defect(nbytes, B.PC_EINVAL)
    elif defect == "mis_dst":
        dst, want = dst + off, ptr_defect(nbytes, B.PC_EALIGN)
    elif defect == "mis_src":
        src, want = src + off, ptr_defect(nbytes, B.PC_EALIGN)
    elif defect == "odd":
        nbytes, want = nbytes + j, B.PC_EALIGN
    elif defect == "big":
        nbytes, want = 2 * MAX + 16, B.PC_EINVAL
    elif defect == "overlap" and nbytes > 16:
        dst, want = src + 16, B.PC_EINVAL
    elif defect == "alias":
        dst, want = src, B.PC_OK                     # onto itself: nothing to do
    assert B.pc_copy(dst, src, nbytes, stream=0, check=False) == want


# ---- twoshot, all three forms -------------------------------------------------------

@SETTINGS
@given(n=st.integers(1, 8), q=st.integers(0, 1 << 18), j=st.integers(0, 7), off=st.integers(1, 15),
       form=st.sampled_from(["two", "fused", "linked"]),
       defect=st.sampled_from(["none", "n9", "k_odd", "k_big", "null_in", "mis_in", "null_out",
                               "mis_out", "outs_overlap", "out_overlaps_in", "in_place",
                               "ws_null", "ws_mis", "ws_small", "ws_overlap"]))
def test_twoshot_admission(n, q, j, off, form, defect):
    k = 8 * n * q
    ins = [slot(r) for r in range(n)]
    outs = [slot(10 + r) for r in range(n)]
    ws, ws_bytes = slot(30), 1 << 30
    want = ran(k)
    r = j % n
    if defect == "n9":
        ins, outs, want = [slot(i) for i in range(9)], [slot(10 + i) for i in range(9)], B.PC_EINVAL
    elif defect == "k_odd" and n > 1:
        k, want = k + 8, B.PC_EALIGN                 # a multiple of 8 but not of 8n
    elif defect == "k_big":
        k, want = 8 * n * (MAX // (8 * n) + 1), B.PC_EINVAL
    elif defect == "null_in":
        ins[r], want = 0, ptr_defect(k, B.PC_EINVAL)
    elif defect == "mis_in":
        ins[r] += off
        want = ptr_defect(k, B.PC_EALIGN)
    elif defect == "null_out":
        outs[r], want = 0, ptr_defect(k, B.PC_EINVAL)
    elif defect == "mis_out":
        outs[r] += off
        want = ptr_defect(k, B.PC_EALIGN)
    elif defect == "outs_overlap" and n > 1 and k > 8:
        outs[(r + 1) % n], want = outs[r] + 16, B.PC_EINVAL
    elif defect == "out_overlaps_in" and k > 8:
        outs[r], want = ins[(r + 1) % n] + 16, B.PC_EINVAL
    elif defect == "in_place":
        outs = list(ins)
    elif form == "linked" and defect == "ws_null":
        ws, want = 0, ptr_defect(k, B.PC_EINVAL)
    elif form == "linked" and defect == "ws_mis":
        ws, want = ws + off, ptr_defect(k, B.PC_EALIGN)
    elif form == "linked" and defect == "ws_small" and k:
        ws_bytes, want = B.pc_twoshot_linked_workspace_bytes(n, k) - 4, B.PC_EINVAL
    elif form == "linked" and defect == "ws_overlap" and k:
        ws, want = outs[r] - 16, B.PC_EINVAL          # the workspace runs into outs[r]
    if form == "two":
        got = B.pc_twoshot(ins, outs, k, stream=0, check=False)
    elif form == "fused":
        got = B.pc_twoshot_fused(ins, outs, k, stream=0, check=False)
    else:
        got = B.pc_twoshot_linked(ins, outs, k, ws, workspace_bytes=ws_bytes, stream=0, check=False)
    assert got == want


# ---- LL pack and consume -------------------------------------------------------------

@SETTINGS
@given(q=st.integers(0, 1 << 22), j=st.integers(1, 7), off=st.integers(1, 15),
       seq=st.integers(1, (1 << 32) - 1),
       defect=st.sampled_from(["none", "seq0", "k_odd", "k_big", "null_src", "null_dst", "mis_src",
                               "mis_dst", "overlap"]))
def test_pack_ll_admission(q, j, off, seq, defect):
    k, src, dst = 8 * q, slot(0), slot(1)
    want = ran(k)
    if defect == "seq0":
        seq, want = 0, B.PC_EINVAL
    elif defect == "k_odd":
        k, want = k + j, B.PC_EALIGN
    elif defect == "k_big":
        k, want = MAX + 8, B.PC_EINVAL
    elif defect == "null_src":
        src, want = 0, ptr_defect(k, B.PC_EINVAL)
    elif defect == "null_dst":
        dst, want = 0, ptr_defect(k, B.PC_EINVAL)
    elif defect == "mis_src":
        src, want = src + off, ptr_defect(k, B.PC_EALIGN)
    elif defect == "mis_dst":
        dst, want = dst + off, ptr_defect(k, B.PC_EALIGN)
    elif defect == "overlap" and k:
        dst, want = src - 16, B.PC_EINVAL             # the lines run over the source
    assert B.pc_pack_ll(src, dst, k, seq, stream=0, check=False) == want


@SETTINGS
@given(n=st.integers(1, 8), q=st.integers(0, 1 << 18), j=st.integers(0, 7), off=st.integers(1, 15),
       defect=st.sampled_from(["none", "n9", "seq0", "k64", "k_big", "null_line", "mis_line",
                               "null_out", "mis_out", "null_bm", "mis_bm", "bm_on_out", "out_on_line"]))
def test_consume_ll_admission(n, q, j, off, defect):
    k, seq = 128 * q, 7
    lines = [slot(r) for r in range(n)]
    out, bm = slot(9), slot(10)
    want = ran(k)
    r = j % n
    if defect == "n9":
        lines, want = [slot(i) for i in range(9)], B.PC_EINVAL
    elif defect == "seq0":
        seq, want = 0, B.PC_EINVAL
    elif defect == "k64":
        k, want = k + 64, B.PC_EALIGN
    elif defect == "k_big":
        k, want = MAX + 128, B.PC_EINVAL
    elif defect == "null_line":
        lines[r], want = 0, ptr_defect(k, B.PC_EINVAL)
    elif defect == "mis_line":
        lines[r] += off
        want = ptr_defect(k, B.PC_EALIGN)
    elif defect == "null_out":
        out, want = 0, ptr_defect(k, B.PC_EINVAL)
    elif defect == "mis_out":
        out, want = out + off, ptr_defect(k, B.PC_EALIGN)
    elif defect == "null_bm":
        bm, want = 0, ptr_defect(k, B.PC_EINVAL)
    elif defect == "mis_bm":
        bm, want = bm + off, ptr_defect(k, B.PC_EALIGN)
    elif defect == "bm_on_out" and k:
        bm, want = out + 16 * (q % 8), B.PC_EINVAL
    elif defect == "out_on_line" and k:
        out, want = lines[r] + 16, B.PC_EINVAL
    assert B.pc_consume_ll(lines, out, k, seq, bm, stream=0, check=False) == want


# ---- all-gather --------------------------------------------------------------------

@SETTINGS
@given(n=st.integers(1, 8), q=st.integers(0, 1 << 16), j=st.integers(0, 7), off=st.integers(1, 15),
       seq=st.integers(1, (1 << 64) - 1),
       defect=st.sampled_from(["none", "n9", "seq0", "bytes_odd", "bytes_big", "null_shard",
                               "mis_shard", "null_out", "mis_out", "null_bm", "mis_bm", "bm_on_out"]))
def test_allgather_admission(n, q, j, off, seq, defect):
    sb = 8192 * q
    shards = [slot(r) for r in range(n)]
    out, bm = slot(9), slot(10)
    want = ran(sb)
    r = j % n
    if defect == "n9":
        shards, want = [slot(i) for i in range(9)], B.PC_EINVAL
    elif defect == "seq0":
        seq, want = 0, B.PC_EINVAL
    elif defect == "bytes_odd":
        sb, want = sb + 4096, B.PC_EALIGN
    elif defect == "bytes_big":
        sb, want = 2 * MAX + 8192, B.PC_EINVAL
    elif defect == "null_shard":
        shards[r], want = 0, ptr_defect(sb, B.PC_EINVAL)
    elif defect == "mis_shard":
        shards[r] += off
        want = ptr_defect(sb, B.PC_EALIGN)
    elif defect == "null_out":
        out, want = 0, ptr_defect(sb, B.PC_EINVAL)
    elif defect == "mis_out":
        out, want = out + off, ptr_defect(sb, B.PC_EALIGN)
    elif defect == "null_bm":
        bm, want = 0, ptr_defect(sb, B.PC_EINVAL)
    elif defect == "mis_bm":
        bm, want = bm + off, ptr_defect(sb, B.PC_EALIGN)
    elif defect == "bm_on_out" and sb:
        bm, want = out + 16, B.PC_EINVAL
    assert B.pc_allgather_copy(shards, out, sb, seq, bm, stream=0, check=False) == want


# ---- sentinel readiness ----------------------------------------------------------------

@SETTINGS
@given(q=st.integers(0, 1 << 22), j=st.integers(1, 7), off=st.integers(1, 15),
       defect=st.sampled_from(["none", "k_odd", "k_big", "null_src", "null_slot", "mis_src",
                               "mis_slot", "overlap", "in_place"]))
def test_publish_sentinel_admission(q, j, off, defect):
    k, src, dst = 8 * q, slot(0), slot(1)
    want = ran(k)
    if defect == "k_odd":
        k, want = k + j, B.PC_EALIGN
    elif defect == "k_big":
        k, want = MAX + 8, B.PC_EINVAL
    elif defect == "null_src":
        src, want = 0, ptr_defect(k, B.PC_EINVAL)
    elif defect == "null_slot":
        dst, want = 0, ptr_defect(k, B.PC_EINVAL)
    elif defect == "mis_src":
        src, want = src + off, ptr_defect(k, B.PC_EALIGN)
    elif defect == "mis_slot":
        dst, want = dst + off, ptr_defect(k, B.PC_EALIGN)
    elif defect == "overlap" and k > 8:
        dst, want = src + 16, B.PC_EINVAL
    elif defect == "in_place":
        dst = src
    assert B.pc_publish_sentinel(src, dst, k, stream=0, check=False) == want


@SETTINGS
@given(n=st.integers(1, 8), q=st.integers(0, 1 << 18), j=st.integers(0, 7), off=st.integers(1, 15),
       defect=st.sampled_from(["none", "n9", "k256", "k_big", "null_slot", "mis_slot", "null_out",
                               "mis_out", "null_bm", "mis_bm", "out_on_slot"]))
def test_consume_sentinel_admission(n, q, j, off, defect):
    k = 512 * q
    slots = [slot(r) for r in range(n)]
    out, bm = slot(9), slot(10)
    want = ran(k)
    r = j % n
    if defect == "n9":
        slots, want = [slot(i) for i in range(9)], B.PC_EINVAL
    elif defect == "k256":
        k, want = k + 256, B.PC_EALIGN
    elif defect == "k_big":
        k, want = MAX + 512, B.PC_EINVAL
    elif defect == "null_slot":
        slots[r], want = 0, ptr_defect(k, B.PC_EINVAL)
    elif defect == "mis_slot":
        slots[r] += off
        want = ptr_defect(k, B.PC_EALIGN)
    elif defect == "null_out":
        out, want = 0, ptr_defect(k, B.PC_EINVAL)
    elif defect == "mis_out":
        out, want = out + off, ptr_defect(k, B.PC_EALIGN)
    elif defect == "null_bm":
        bm, want = 0, ptr_defect(k, B.PC_EINVAL)
    elif defect == "mis_bm":
        bm, want = bm + off, ptr_defect(k, B.PC_EALIGN)
    elif defect == "out_on_slot" and k:
        out, want = slots[r] + 16, B.PC_EINVAL
    assert B.pc_consume_sentinel(slots, out, k, bm, stream=0, check=False) == want


# ---- speculative reduce -------------------------------------------------------------------

@SETTINGS
@given(n=st.integers(1, 8), u=st.integers(1, 4), q=st.integers(0, 1 << 12), j=st.integers(0, 7),
       off=st.integers(1, 15), flag=st.integers(0, (1 << 32) - 1),
       defect=st.sampled_from(["none", "n9", "epf_bad", "k_odd", "k_big", "attempts0", "attempts_big",
                               "null_in", "mis_in", "null_flag", "mis_flag", "null_out", "mis_out",
                               "null_att", "mis_att", "in_place", "out_overlap"]))
def test_reduce_validated_admission(n, u, q, j, off, flag, defect):
    epf = 2048 * u
    k = epf * q
    ins = [slot(r) for r in range(n)]
    flags = [slot(10 + r) for r in range(n)]
    out, att, max_attempts = slot(20), slot(21), 3
    want = ran(k)
    r = j % n
    if defect == "n9":
        ins, flags, want = [slot(i) for i in range(9)], [slot(10 + i) for i in range(9)], B.PC_EINVAL
    elif defect == "epf_bad":
        epf, want = (1024, 2048 * 5, 0, 2049)[j % 4], B.PC_EINVAL
    elif defect == "k_odd":
        k, want = k + 8, B.PC_EALIGN
    elif defect == "k_big":
        k, want = MAX + epf, B.PC_EINVAL
    elif defect == "attempts0":
        max_attempts, want = 0, B.PC_EINVAL
    elif defect == "attempts_big":
        max_attempts, want = B.PC_MAX_ATTEMPTS + 1, B.PC_EINVAL
    elif defect == "null_in":
        ins[r], want = 0, ptr_defect(k, B.PC_EINVAL)
    elif defect == "mis_in":
        ins[r] += off
        want = ptr_defect(k, B.PC_EALIGN)
    elif defect == "null_flag":
        flags[r], want = 0, ptr_defect(k, B.PC_EINVAL)
    elif defect == "mis_flag":
        flags[r] += 1 + off % 3                      # flags need 4-byte alignment only
        want = ptr_defect(k, B.PC_EALIGN)
    elif defect == "null_out":
        out, want = 0, ptr_defect(k, B.PC_EINVAL)
    elif defect == "mis_out":
        out, want = out + off, ptr_defect(k, B.PC_EALIGN)
    elif defect == "null_att":
        att, want = 0, ptr_defect(k, B.PC_EINVAL)
    elif defect == "mis_att":
        att, want = att + 1 + off % 3, ptr_defect(k, B.PC_EALIGN)
    elif defect == "in_place":
        out = ins[r]
    elif defect == "out_overlap" and k:
        out, want = ins[r] + 16, B.PC_EINVAL
    assert B.pc_reduce_validated(ins, flags, out, k, epf, flag, max_attempts, att, stream=0,
                                 check=False) == want
