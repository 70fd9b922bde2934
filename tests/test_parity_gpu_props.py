"""Property-based parity on the GPU: drawn rank counts, fold orders and sizes,
with sizes concentrated just below, at and just above every size at which a
call switches launch shape (the 64 MiB working set of the persistent kernels,
the mid shape of the reduce, the 4 MiB per rank of the LL, sentinel and
copy kernels, the linked twoshot's tile sizes).  Every result is compared
bit for bit with the oracle.  Examples are derandomized, so every run checks
the same cases and a failure reproduces.
"""
import os

import numpy as np
import pytest

pytest.importorskip("hypothesis")
torch = pytest.importorskip("torch")
from hypothesis import HealthCheck, given, settings  # noqa: E402
from hypothesis import strategies as st  # noqa: E402

from collective_datapath_amd import synth  # noqa: E402

pytestmark = pytest.mark.gpu

THREADS = max(1, min(16, os.cpu_count() or 1))
SETTINGS = settings(max_examples=24, deadline=None, derandomize=True,
                    suppress_health_check=[HealthCheck.too_slow, HealthCheck.function_scoped_fixture])
MIB = 1 << 20


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


def near(points, unit):
    """Each point and its neighbours one unit away."""
    return sorted({max(unit, p + d * unit) for p in points for d in (-1, 0, 1)})


# Chunk counts (16-byte units per rank) at which the reduce changes shape at
# rank count n: the mid shape from 262144 chunks, the persistent kernel from
# a 64 MiB working set, (n + 1) * 16 bytes per chunk.
def reduce_chunks(n):
    return near([262144, -(-(64 * MIB) // (16 * (n + 1))), 256, 512], 1)


@SETTINGS
@given(data=st.data(), n=st.integers(1, 8))
def test_reduce_properties(B, D, orc, data, n):
    chunks = data.draw(st.one_of(st.sampled_from(reduce_chunks(n)), st.integers(1, 1 << 19)))
    k = 8 * chunks
    order = data.draw(st.permutations(list(range(n))))
    xs = [synth.uniform_bf16(2000 + n, 0, r, k) for r in range(n)]
    ins = [D.up(x) for x in xs]
    out = D.filled(k, 0xFFFF)
    B.pc_reduce(ins, out, k, order=list(order))
    assert np.array_equal(D.down(out, np.uint16), orc.reduce(xs, order=list(order), threads=THREADS))


@SETTINGS
@given(data=st.data(), n=st.integers(1, 8), form=st.sampled_from(["two", "fused", "linked"]))
def test_twoshot_properties(B, D, orc, data, n, form):
    # Slice chunk counts around the persistent switch of each form and the
    # linked tile-size switches (512 KiB and 4 MiB per rank).
    per_rank_points = [-(-(64 * MIB) // (16 * (n + 1))), -(-(64 * MIB) // (16 * 2 * n)),
                       (512 << 10) // 16, (4 * MIB) // 16, 262144]
    slice_points = near([max(1, p // n) for p in per_rank_points], 1)
    sc = data.draw(st.one_of(st.sampled_from(slice_points), st.integers(1, 40000)))
    k = 8 * n * sc
    xs = [synth.normal_bf16(2100 + n, 0, r, k) for r in range(n)]
    ins = [D.up(x) for x in xs]
    outs = [D.filled(k, 0xFFFF) for _ in range(n)]
    if form == "two":
        B.pc_twoshot(ins, outs, k)
    elif form == "fused":
        B.pc_twoshot_fused(ins, outs, k)
    else:
        ws = torch.zeros(B.pc_twoshot_linked_workspace_bytes(n, k) // 8, dtype=torch.int64, device="cuda:0")
        B.pc_twoshot_linked(ins, outs, k, ws)
        assert int(ws[B.PC_LINKED_STATUS_WORD]) == 0
    want = orc.reduce(xs, threads=THREADS)
    for o in outs:
        assert np.array_equal(D.down(o, np.uint16), want)


@SETTINGS
@given(data=st.data(), n=st.integers(1, 8))
def test_ll_properties(B, D, orc, data, n):
    # k in units of 128 elements (whole bitmap words); the shapes switch at 4 MiB per rank.
    units = data.draw(st.one_of(st.sampled_from(near([(4 * MIB) // 256], 1)), st.integers(1, 4096)))
    k = 128 * units
    case = synth.LLCase("prop", 2200 + n, n, k, stale_frac=0.04)
    staged = [np.where(m, orc.pack_ll(s, case.stale_seq), orc.pack_ll(x, case.seq))
              for x, s, m in zip(case.payloads(), case.stale_payloads(), case.stale_masks())]
    # Pack on the GPU too, for one rank, and compare the lines.
    src = D.up(case.payloads()[0])
    lines0 = torch.empty(k // 2, dtype=torch.int64, device="cuda:0")
    B.pc_pack_ll(src, lines0, k, case.seq)
    assert np.array_equal(D.down(lines0, np.uint64), orc.pack_ll(case.payloads()[0], case.seq))
    out = D.filled(k, 0xFFFF)
    bm = torch.full((k // 128,), -1, dtype=torch.int64, device="cuda:0")
    B.pc_consume_ll([D.up(s) for s in staged], out, k, case.seq, bm)
    wo, wb = orc.consume_ll(staged, k, case.seq)
    assert np.array_equal(D.down(bm, np.uint64), wb)
    assert np.array_equal(D.down(out, np.uint16), wo)


@SETTINGS
@given(data=st.data(), n=st.integers(1, 8))
def test_sentinel_properties(B, D, orc, data, n):
    units = data.draw(st.one_of(st.sampled_from(near([(4 * MIB) // 1024], 1)), st.integers(1, 1024)))
    k = 512 * units
    case = synth.SentinelCase("prop", 2300 + n, n, k, 0.03, 0.01, 0.01)
    xs = case.payloads()
    pub = D.filled(k, 0)
    B.pc_publish_sentinel(D.up(xs[0]), pub, k)
    assert np.array_equal(D.down(pub, np.uint16), orc.publish_sentinel(xs[0]))
    slots = [synth.unarrive(orc.publish_sentinel(x), m, t) for x, (m, t) in zip(xs, case.masks())]
    dev = [D.up(s) for s in slots]
    out = D.filled(k, 0xFFFF)
    bm = torch.full((k // 512,), -1, dtype=torch.int64, device="cuda:0")
    B.pc_consume_sentinel(dev, out, k, bm)
    wo, wb, wsl = orc.consume_sentinel(slots, k)
    assert np.array_equal(D.down(bm, np.uint64), wb)
    assert np.array_equal(D.down(out, np.uint16), wo)
    assert all(np.array_equal(D.down(a, np.uint16), b) for a, b in zip(dev, wsl))


@SETTINGS
@given(data=st.data(), n=st.integers(1, 8))
def test_allgather_properties(B, D, orc, data, n):
    groups = data.draw(st.integers(1, 96))
    sb = 8192 * groups
    case = synth.GatherCase("prop", 2400 + n, n, sb, stale_frac=data.draw(st.sampled_from([0.0, 0.1, 0.5, 1.0])))
    recs, _ = case.records()
    out = D.filled(n * sb // 2, 0xFFFF)
    bm = torch.full((n * case.blocks // 64,), -1, dtype=torch.int64, device="cuda:0")
    B.pc_allgather_copy([D.up(r) for r in recs], out, sb, case.seq, bm)
    wo, wb = orc.allgather_copy(recs, sb, case.seq)
    assert np.array_equal(D.down(bm, np.uint64), wb)
    assert np.array_equal(D.down(out, np.uint16), wo)


@SETTINGS
@given(data=st.data(), n=st.integers(1, 8), u=st.integers(1, 4))
def test_reduce_validated_properties(B, D, orc, data, n, u):
    epf = 2048 * u
    tiles = data.draw(st.integers(1, 64))
    k = epf * tiles
    case = synth.ValidatedCase("prop", 2500 + n, n, k, epf, flag=data.draw(st.integers(1, (1 << 32) - 1)))
    xs, fl = case.payloads(), case.flags()
    out = D.filled(k, 0xFFFF)
    at = torch.empty(tiles, dtype=torch.int32, device="cuda:0")
    B.pc_reduce_validated([D.up(x) for x in xs], [D.up(f) for f in fl], out, k, epf, case.flag, 1, at)
    wo, wok = orc.reduce_validated(xs, fl, epf, case.flag)
    assert np.array_equal(D.down(at, np.uint32), wok)
    assert np.array_equal(D.down(out, np.uint16), wo)


@SETTINGS
@given(data=st.data())
def test_copy_properties(B, D, data):
    chunks = data.draw(st.one_of(st.sampled_from(near([(4 * MIB) // 16, (32 * MIB) // 16], 1)),
                                 st.integers(1, 1 << 16)))
    nbytes = 16 * chunks
    src = np.random.default_rng(chunks).integers(0, 256, nbytes, dtype=np.uint8)
    dst = torch.zeros(nbytes, dtype=torch.uint8, device="cuda:0")
    B.pc_copy(dst, D.up(src), nbytes)
    assert np.array_equal(D.down(dst, np.uint8), src)
