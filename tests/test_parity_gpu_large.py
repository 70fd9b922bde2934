"""Byte offsets above 4 GiB, and the largest accepted size, for every entry
point whose other tests stay below them (the reduce and the copy have their
own); and one call large enough that a kernel's grid cap makes workgroups
take several work items.

Each call runs twice: on buffers that reach just past 2^32 bytes, with sizes
ragged against every tile shape, and at the largest size it accepts
(PC_MAX_ELEMS elements per rank, or twice that many bytes), so every
kernel's address arithmetic is exercised where 32 bits no longer suffice.  Outputs are compared bit for bit with the
oracle over sampled windows: the head, a window around each multiple of
2^32 bytes of every buffer the call touches, and the tail.  Windows of the
calls that write a bitmap start and end on whole bitmap words.

Inputs come from torch's device RNG, and stale units are planted by index
from the host: nothing comes from the HIP path.  Every expected value is the
oracle's, computed from the same input bytes copied back from the device.
"""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
GiB = 1 << 30
FAR = 1 << 32  # the byte offset every buffer under test reaches past
MAX_ELEMS = 1 << 34  # PC_MAX_ELEMS of include/pc.h
SIZES = ["past_4gib", "maximum"]


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


@pytest.fixture(autouse=True)
def release_memory():
    yield
    torch.cuda.empty_cache()


def need_memory(nbytes):
    free, _ = torch.cuda.mem_get_info()
    if free < nbytes:
        pytest.skip(f"needs {nbytes >> 30} GiB of free device memory, {free >> 30} GiB free")


def gen(seed):
    g = torch.Generator(device=DEV)
    g.manual_seed(seed)
    return g


def finite_bf16(k, g):
    """k random bf16 patterns with the top exponent bit clear: finite, of
    magnitude below 2, and never the sentinel 0xFFFF."""
    t = torch.empty(k, dtype=torch.int16, device=DEV).random_(-32768, 32767, generator=g)
    return t.bitwise_and_(~0x4000)


def windows(count, boundaries, width, align=1):
    """Ranges [a, b) of `count` units: the head, one around each boundary
    unit below `count`, and the tail.  Starts are multiples of `align`; every
    end is a start plus `width` (a multiple of `align`) or `count`."""
    spans = [(0, min(width, count))]
    for c in sorted(set(boundaries)):
        if 0 < c < count:
            a = max(0, c - width // 2) // align * align
            spans.append((a, min(a + width, count)))
    spans.append((max(0, count - width) // align * align, count))
    return spans


def byte_marks(count, unit_bytes, offset_units=0):
    """Units of a buffer (of `unit_bytes` per unit, starting `offset_units`
    into it) at which its byte offset crosses a multiple of 2^32."""
    marks, j = [], 1
    while j * FAR // unit_bytes < offset_units + count:
        marks.append(j * FAR // unit_bytes - offset_units)
        j += 1
    return marks


def plant(rng, span, frac):
    a, b = span
    return rng.choice(np.arange(a, b), max(1, int((b - a) * frac)), replace=False)


# ---- LL pack and consume ------------------------------------------------------------

@pytest.mark.parametrize("size", SIZES)
def test_pack_ll_far(B, D, orc, size):
    # past 4 GiB: src 4 GiB + 80 B, lines 8 GiB + 160 B
    k = FAR // 2 + 8 * 5 if size == "past_4gib" else MAX_ELEMS
    need_memory(6 * k + GiB)
    say("pack_ll", size, k)
    seq = 0x5EED0001
    src = finite_bf16(k, gen(41))
    lines = torch.empty(k // 2, dtype=torch.int64, device=DEV)
    B.pc_pack_ll(src, lines, k, seq)
    nl = k // 2
    for a, b in windows(nl, byte_marks(nl, 8) + byte_marks(nl, 4), 4096):
        want = orc.pack_ll(D.down(src[2 * a:2 * b], np.uint16), seq)
        assert np.array_equal(D.down(lines[a:b], np.uint64), want), (a, b)


@pytest.mark.parametrize("size", SIZES)
def test_consume_ll_far(B, D, orc, size):
    # Past 4 GiB: 8 GiB + 1.5 KiB of lines per rank, 4 GiB + 768 B of
    # output (the persistent consumer).  A tenth of each window's lines is stale on some
    # rank, and one 64-line group is stale on rank 0 (a zero bitmap word).
    n, k = 2, FAR // 2 + 128 * 3 if size == "past_4gib" else MAX_ELEMS
    nl = k // 2
    need_memory(n * 8 * nl + 2 * k + 6 * GiB)
    say("consume_ll", size, n, k)
    seq = 0x0C0FFEE1
    g = gen(42)
    lines = []
    for _ in range(n):
        t = torch.empty(nl, dtype=torch.int64, device=DEV).random_(generator=g)
        lines.append(t.bitwise_and_(0xBFFFBFFF).bitwise_or_(seq << 32))
    spans = windows(nl, byte_marks(nl, 8) + byte_marks(nl, 4), 4096, align=64)
    rng = np.random.default_rng(42)
    for a, b in spans:
        for r, t in enumerate(lines):
            idx = torch.from_numpy(plant(rng, (a, b), 0.05)).to(DEV)
            t[idx] = t[idx].bitwise_and(0xFFFFFFFF).bitwise_or((seq - 1) << 32)
        grp = torch.arange(a + 64, a + 128, device=DEV)
        lines[0][grp] = lines[0][grp].bitwise_and(0xFFFFFFFF)
    out = D.filled(k, 0xFFFF)
    bm = torch.full((k // 128,), -1, dtype=torch.int64, device=DEV)
    B.pc_consume_ll(lines, out, k, seq, bm)
    for a, b in spans:
        want_out, want_bm = orc.consume_ll([D.down(t[a:b], np.uint64) for t in lines], 2 * (b - a), seq)
        assert 0 < int(np.unpackbits(want_bm.view(np.uint8)).sum()) < b - a
        assert np.array_equal(D.down(bm[a // 64:b // 64], np.uint64), want_bm), (a, b)
        assert np.array_equal(D.down(out[2 * a:2 * b], np.uint16), want_out), (a, b)


# ---- twoshot, all three forms ------------------------------------------------------------

@pytest.mark.parametrize("size", SIZES)
def test_twoshot_forms_far(B, D, orc, size):
    # Past 4 GiB: 4 GiB + 224 B per rank, so every byte offset past 4 GiB
    # lies in slice 1.
    n, k = 2, FAR // 2 + 16 * 7 if size == "past_4gib" else MAX_ELEMS
    need_memory(4 * 2 * k + 2 * GiB)
    g = gen(43)
    ins = [finite_bf16(k, g) for _ in range(n)]
    outs = [torch.empty(k, dtype=torch.int16, device=DEV) for _ in range(n)]
    ws = torch.zeros(B.pc_twoshot_linked_workspace_bytes(n, k) // 8, dtype=torch.int64, device=DEV)
    spans = windows(k, byte_marks(k, 2) + [k // n], 8192, align=8)
    wants = [orc.reduce([D.down(x[a:b], np.uint16) for x in ins]) for a, b in spans]
    for form in ("pc_twoshot", "pc_twoshot_fused", "pc_twoshot_linked"):
        say(form, size, n, k)
        for o in outs:
            o.fill_(-1)
        if form == "pc_twoshot_linked":
            B.pc_twoshot_linked(ins, outs, k, ws)
        else:
            getattr(B, form)(ins, outs, k)
        for (a, b), want in zip(spans, wants):
            for r, o in enumerate(outs):
                assert np.array_equal(D.down(o[a:b], np.uint16), want), (form, r, a, b)
    torch.cuda.synchronize()
    assert int(ws[B.PC_LINKED_STATUS_WORD]) == 0


def test_twoshot_fused_split_past_4gib(B, D, orc):
    # Five ranks of 4 GiB + 280 B: the single-launch twoshot that folds its
    # tiles into the owners' outputs first and hands them out afterwards.
    n = 5
    k = (FAR // 2 // (8 * n) + 7) * 8 * n
    need_memory(2 * n * 2 * k + 2 * GiB)
    say("pc_twoshot_fused split past 4 GiB", n, k)
    g = gen(48)
    ins = [finite_bf16(k, g) for _ in range(n)]
    outs = [torch.full((k,), -1, dtype=torch.int16, device=DEV) for _ in range(n)]
    spans = windows(k, byte_marks(k, 2) + [s * k // n for s in range(1, n)], 8192, align=8)
    B.pc_twoshot_fused(ins, outs, k)
    for a, b in spans:
        want = orc.reduce([D.down(x[a:b], np.uint16) for x in ins])
        for r, o in enumerate(outs):
            assert np.array_equal(D.down(o[a:b], np.uint16), want), (r, a, b)


@pytest.mark.parametrize("shape", ["ragged", "whole_tiles"])
def test_staged_paths_past_4gib(B, D, orc, shape):
    # Four ranks of 4 GiB + 64 KiB (slices of whole 1,024-chunk tiles) or of
    # 4 GiB + 32,896 B (ragged): the LDS-staged oneshot, twoshot phase 1 and
    # the flag-linked twoshot's staged phase 1, each past byte offset 2^32.
    n = 4
    k = FAR // 2 + (32768 if shape == "whole_tiles" else 8 * n * 514)
    need_memory(3 * n * 2 * k + 2 * GiB)
    say("staged paths past 4 GiB", shape, n, k)
    g = gen(52)
    ins = [finite_bf16(k, g) for _ in range(n)]
    outs = [torch.full((k,), -1, dtype=torch.int16, device=DEV) for _ in range(n)]
    spans = windows(k, byte_marks(k, 2) + [s * k // n for s in range(1, n)], 8192, align=8)
    wants = [orc.reduce([D.down(x[a:b], np.uint16) for x in ins]) for a, b in spans]
    B.pc_reduce(ins, outs[0], k)
    for (a, b), want in zip(spans, wants):
        assert np.array_equal(D.down(outs[0][a:b], np.uint16), want), ("reduce", a, b)
    ws = torch.zeros(B.pc_twoshot_linked_workspace_bytes(n, k) // 8, dtype=torch.int64, device=DEV)
    for form in ("pc_twoshot", "pc_twoshot_linked"):
        for o in outs:
            o.fill_(-1)
        if form == "pc_twoshot_linked":
            B.pc_twoshot_linked(ins, outs, k, ws)
        else:
            B.pc_twoshot(ins, outs, k)
        for (a, b), want in zip(spans, wants):
            for r, o in enumerate(outs):
                assert np.array_equal(D.down(o[a:b], np.uint16), want), (form, r, a, b)
    torch.cuda.synchronize()
    assert int(ws[B.PC_LINKED_STATUS_WORD]) == 0


def test_twoshot_copyout_one_destination_past_4gib(B, D, orc):
    # Seven ranks of 4 GiB + 3,552 B: the two-launch twoshot's copy-out with
    # one destination per workgroup, past byte offset 2^32 and past its grid
    # cap (about 1.05M tiles x 6 destinations = 6.3M work items, against a
    # grid of about 4.19M workgroups).
    n = 7
    k = (FAR // 2 // (8 * n) + 32) * 8 * n
    need_memory(2 * n * 2 * k + 2 * GiB)
    say("twoshot one-destination copy-out past 4 GiB", n, k)
    g = gen(53)
    ins = [finite_bf16(k, g) for _ in range(n)]
    outs = [torch.full((k,), -1, dtype=torch.int16, device=DEV) for _ in range(n)]
    spans = windows(k, byte_marks(k, 2) + [s * k // n for s in range(1, n)], 8192, align=8)
    B.pc_twoshot(ins, outs, k)
    for a, b in spans:
        want = orc.reduce([D.down(x[a:b], np.uint16) for x in ins])
        for r, o in enumerate(outs):
            assert np.array_equal(D.down(o[a:b], np.uint16), want), (r, a, b)


def test_twoshot_copyout_past_its_grid_cap(B, D, orc):
    # Eight ranks of 2.5 GiB + 896 B: the two-launch twoshot's copy-out, one
    # destination per workgroup, has 8 x 81,921 tiles x 7 destinations =
    # 4.59M work items, more than its grid of about 4.19M workgroups, so the
    # first workgroups take a second item.
    n = 8
    k = ((5 * GiB // 4) // (8 * n) + 7) * 8 * n
    need_memory(2 * n * 2 * k + 2 * GiB)
    say("pc_twoshot copy-out past its grid cap", n, k)
    g = gen(49)
    ins = [finite_bf16(k, g) for _ in range(n)]
    outs = [torch.full((k,), -1, dtype=torch.int16, device=DEV) for _ in range(n)]
    spans = windows(k, byte_marks(k, 2) + [s * k // n for s in range(1, n)], 8192, align=8)
    B.pc_twoshot(ins, outs, k)
    for a, b in spans:
        want = orc.reduce([D.down(x[a:b], np.uint16) for x in ins])
        for r, o in enumerate(outs):
            assert np.array_equal(D.down(o[a:b], np.uint16), want), (r, a, b)


# ---- all-gather of 136-byte records --------------------------------------------------------

@pytest.mark.parametrize("size", SIZES)
def test_allgather_far(B, D, orc, size):
    # Past 4 GiB: 4 GiB + 24 KiB of payload per shard, so records reach
    # 4.25 GiB and the output 8 GiB.  Headers are compared as u64: stale ones differ from seq
    # only in the upper word.
    n = 2
    shard_bytes = FAR + 8192 * 3 if size == "past_4gib" else 2 * MAX_ELEMS
    bs = shard_bytes // 128
    need_memory(n * 136 * bs + n * shard_bytes + 2 * GiB)
    say("allgather", size, n, shard_bytes)
    seq = (7 << 32) | 0x2468ACE1
    stale = seq ^ (1 << 40)
    g = gen(44)
    recs = []
    for _ in range(n):
        t = torch.empty(bs * 17, dtype=torch.int64, device=DEV).random_(generator=g)
        t.view(bs, 17)[:, 0] = seq
        recs.append(t)
    spans = [windows(bs, byte_marks(bs, 136) + byte_marks(bs, 128, r * bs), 2048, align=64)
             for r in range(n)]
    rng = np.random.default_rng(44)
    for r in range(n):
        heads = recs[r].view(bs, 17)
        for a, b in spans[r]:
            heads[torch.from_numpy(plant(rng, (a, b), 0.1)).to(DEV), 0] = stale
            heads[a + 64:a + 128, 0] = stale
    out = D.filled(n * shard_bytes // 2, 0xFFFF)
    bm = torch.full((n * bs // 64,), -1, dtype=torch.int64, device=DEV)
    B.pc_allgather_copy(recs, out, shard_bytes, seq, bm)
    for r in range(n):
        for a, b in spans[r]:
            rec = D.down(recs[r][a * 17:b * 17], np.uint64).view(np.uint8)
            want_out, want_bm = orc.allgather_copy([rec], (b - a) * 128, seq)
            o0 = r * bs + a
            assert np.array_equal(D.down(bm[o0 // 64:(r * bs + b) // 64], np.uint64), want_bm), (r, a, b)
            assert np.array_equal(D.down(out[o0 * 64:(r * bs + b) * 64], np.uint16), want_out), (r, a, b)


# ---- sentinel publish and consume -------------------------------------------------------

@pytest.mark.parametrize("size", SIZES)
def test_publish_sentinel_far(B, D, orc, size):
    k = FAR // 2 + 8 * 9 if size == "past_4gib" else MAX_ELEMS  # past 4 GiB: 4 GiB + 144 B
    need_memory(4 * k + GiB)
    say("publish_sentinel", size, k)
    src = finite_bf16(k, gen(45))
    spans = windows(k, byte_marks(k, 2), 8192, align=8)
    rng = np.random.default_rng(45)
    for span in spans:  # sentinel patterns to be made canonical
        src[torch.from_numpy(plant(rng, span, 0.01)).to(DEV)] = -1
    slot = torch.empty(k, dtype=torch.int16, device=DEV)
    B.pc_publish_sentinel(src, slot, k)
    for a, b in spans:
        want = orc.publish_sentinel(D.down(src[a:b], np.uint16))
        assert np.array_equal(D.down(slot[a:b], np.uint16), want), (a, b)


@pytest.mark.parametrize("size", SIZES)
def test_consume_sentinel_far(B, D, orc, size):
    # Past 4 GiB: 4 GiB + 3 KiB per slot (the two-pass consumer).  A few elements of each
    # window hold the sentinel on every rank, and one 64-pack group is still
    # armed on rank 1.
    n, k = 2, FAR // 2 + 512 * 3 if size == "past_4gib" else MAX_ELEMS
    need_memory(3 * 2 * k + 2 * GiB)
    say("consume_sentinel", size, n, k)
    g = gen(46)
    slots = [finite_bf16(k, g) for _ in range(n)]
    spans = windows(k, byte_marks(k, 2), 16384, align=512)
    rng = np.random.default_rng(46)
    for a, b in spans:
        for s in slots:
            s[torch.from_numpy(plant(rng, (a, b), 0.01)).to(DEV)] = -1
        slots[1][a + 512:a + 1024] = -1
    before = [[D.down(s[a:b], np.uint16) for s in slots] for a, b in spans]
    out = D.filled(k, 0xFFFF)
    bm = torch.full((k // 512,), -1, dtype=torch.int64, device=DEV)
    B.pc_consume_sentinel(slots, out, k, bm)
    for (a, b), ss in zip(spans, before):
        want_out, want_bm, want_slots = orc.consume_sentinel(ss, b - a)
        assert 0 < int(np.unpackbits(want_bm.view(np.uint8)).sum()) < (b - a) // 8
        assert np.array_equal(D.down(bm[a // 512:b // 512], np.uint64), want_bm), (a, b)
        assert np.array_equal(D.down(out[a:b], np.uint16), want_out), (a, b)
        for r, s in enumerate(slots):
            assert np.array_equal(D.down(s[a:b], np.uint16), want_slots[r]), (r, a, b)


# ---- speculative reduce with a folded flag ---------------------------------------------

@pytest.mark.parametrize("size", SIZES)
def test_reduce_validated_far(B, D, orc, size):
    # Past 4 GiB: 4 GiB + 48 KiB per rank, at 8192 elements per flag (the persistent
    # kernel with four chunks per lane); a quarter of each window's tiles
    # carries a stale flag on rank 1 and is left untouched.
    n, t = 2, 8192
    tiles = FAR // (2 * t) + 3 if size == "past_4gib" else MAX_ELEMS // t
    k = t * tiles
    need_memory(3 * 2 * k + GiB)
    say("reduce_validated", size, n, k, t)
    flag = 0x9E3779B9
    as_i32 = lambda v: v - (1 << 32) if v >= 1 << 31 else v  # noqa: E731
    g = gen(47)
    ins = [finite_bf16(k, g) for _ in range(n)]
    fl = [torch.full((tiles,), as_i32(flag), dtype=torch.int32, device=DEV) for _ in range(n)]
    spans = windows(tiles, byte_marks(tiles, 2 * t), 8)
    rng = np.random.default_rng(47)
    for span in spans:
        fl[1][torch.from_numpy(plant(rng, span, 0.25)).to(DEV)] = as_i32(flag - 1)
    out = D.filled(k, 0xFFFF)
    at = torch.full((tiles,), -1, dtype=torch.int32, device=DEV)
    B.pc_reduce_validated(ins, fl, out, k, t, flag, 1, at)
    for a, b in spans:
        xs = [D.down(x[a * t:b * t], np.uint16) for x in ins]
        want_out, want_ok = orc.reduce_validated(xs, [D.down(f[a:b], np.uint32) for f in fl], t, flag)
        assert 0 < int(want_ok.sum()) < b - a
        assert np.array_equal(D.down(at[a:b], np.uint32), want_ok), (a, b)
        assert np.array_equal(D.down(out[a * t:b * t], np.uint16), want_out), (a, b)
