"""Parity of the HIP path against the CPU oracle, through the C ABI.

Every comparison is bitwise over whole output and bitmap buffers (0 ULP):
the fold order is fixed, so each output element has exactly one correct bit
pattern.  Inputs come from the seeded generators (collective_datapath_amd.synth)
or from torch's own device RNG, never from the HIP path; expected values come
from the oracle only.  Outputs are prefilled with 0xFFFF on both sides so
that "left untouched" is checked too.
"""
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


def gpu_reduce(B, D, xs, order=None, out_fill=0xFFFF):
    k = xs[0].size
    ins = [D.up(x) for x in xs]
    out = D.filled(k, out_fill)
    B.pc_reduce(ins, out, k, order=order)
    return D.down(out, np.uint16)


# ---- reduce -----------------------------------------------------------------

def test_reduce_oneshot_8k(B, D, orc):
    case = synth.C1_ONESHOT_8K
    say(case.name)
    xs = case.inputs()
    assert np.array_equal(gpu_reduce(B, D, xs), orc.reduce(xs))


def test_reduce_oneshot_64m(B, D, orc):
    case = synth.C4_ONESHOT_64M
    say(case.name)
    xs = case.inputs()
    want = orc.reduce(xs, threads=THREADS)
    got = gpu_reduce(B, D, xs)
    assert np.array_equal(got, want), f"{np.count_nonzero(got != want)} mismatches"


@pytest.mark.parametrize("n", [1, 2, 3, 4, 5, 6, 7, 8])
def test_reduce_every_n_ragged_with_order(B, D, orc, n):
    # 37 full 256-chunk tiles plus a ragged tail of 5 chunks.
    k = 8 * (256 * 37 + 5)
    say("reduce ragged", n, k)
    xs = [synth.normal_bf16(200 + n, 0, r, k, 3.0) for r in range(n)]
    order = list(np.random.default_rng(n).permutation(n))
    assert np.array_equal(gpu_reduce(B, D, xs, order=order), orc.reduce(xs, order=order))
    assert np.array_equal(gpu_reduce(B, D, xs), orc.reduce(xs))


@pytest.mark.parametrize("n,chunks", [
    (3, 262144 + 1234),           # mid-size shape: 4 MiB per rank and a tail
    (2, 4718592 + 77),            # streaming shape: 72 MiB per rank and a tail
    (8, 524288 + 13),             # 8 MiB per rank: persistent kernel from a 64 MiB working set
    (8, 256 * 2 * 3 + 1),         # one chunk past whole tiles
    (4, 1),                       # a single chunk
])
def test_reduce_regimes_and_tails(B, D, orc, n, chunks):
    k = 8 * chunks
    say("reduce regime", n, k)
    xs = [synth.uniform_bf16(300 + n, 0, r, k) for r in range(n)]
    assert np.array_equal(gpu_reduce(B, D, xs), orc.reduce(xs, threads=THREADS))


def test_reduce_closed_forms(B, D, orc):
    import json
    golden = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "closed_forms.json")))
    for case in golden["fold"]["cases"]:
        xs = [np.full(64, int(v, 16), dtype=np.uint16) for v in case["inputs"]]
        got = gpu_reduce(B, D, xs, order=case["order"])
        assert np.all(got == int(case["bf16"], 16)), case


@pytest.mark.parametrize("part", range(16))
def test_reduce_two_ranks_exhaustive(B, D, orc, part):
    # All 2^32 (x0, x1) bf16 pairs, in 16 parts of 2^28 pairs.
    say("exhaustive pairs, part", part)
    allh = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    x1vals = allh[part * 4096:(part + 1) * 4096]
    x0 = np.tile(allh, x1vals.size)
    x1 = np.repeat(x1vals, allh.size)
    want = orc.reduce([x0, x1], threads=THREADS)
    got = gpu_reduce(B, D, [x0, x1])
    bad = np.flatnonzero(got != want)
    assert bad.size == 0, [(hex(x0[i]), hex(x1[i]), hex(got[i]), hex(want[i])) for i in bad[:8]]


def test_reduce_specials_three_ranks(B, D, orc):
    sp = np.array([0x0000, 0x8000, 0x0001, 0x8001, 0x0080, 0x7F7F, 0xFF7F, 0x7F80, 0xFF80,
                   0x7FC0, 0xFFC1, 0x7F81, 0x3F80, 0xBF80, 0x4C00, 0xCC00, 0x3B80, 0x007F],
                  dtype=np.uint16)
    a, b, c = np.meshgrid(sp, sp, sp, indexing="ij")
    xs = [a.reshape(-1), b.reshape(-1), c.reshape(-1)]
    pad = (-xs[0].size) % 8
    xs = [np.concatenate([x, np.zeros(pad, np.uint16)]) for x in xs]
    for order in ([0, 1, 2], [2, 0, 1]):
        assert np.array_equal(gpu_reduce(B, D, xs, order=order), orc.reduce(xs, order=order))


def test_reduce_three_ranks_random_patterns(B, D, orc):
    """2^26 triples of uniformly random bf16 bit patterns (every sign,
    exponent and payload, NaNs and infinities included), in two orders."""
    k = 1 << 26
    say("random triples", k)
    rng = np.random.default_rng(26)
    xs = [rng.integers(0, 1 << 16, k, dtype=np.uint32).astype(np.uint16) for _ in range(3)]
    for order in ([0, 1, 2], [1, 2, 0]):
        want = orc.reduce(xs, order=order, threads=THREADS)
        got = gpu_reduce(B, D, xs, order=order)
        bad = np.flatnonzero(got != want)
        assert bad.size == 0, [(hex(xs[0][i]), hex(xs[1][i]), hex(xs[2][i]), hex(got[i]), hex(want[i]))
                               for i in bad[:8]]
    torch.cuda.empty_cache()


def test_reduce_in_place(B, D, orc):
    n, k = 4, 8 * 5000
    xs = [synth.uniform_bf16(400, 0, r, k) for r in range(n)]
    ins = [D.up(x) for x in xs]
    B.pc_reduce(ins, ins[2], k)
    assert np.array_equal(D.down(ins[2], np.uint16), orc.reduce(xs))


def test_reduce_same_buffer_as_every_rank(B, D, orc):
    x = synth.uniform_bf16(401, 0, 0, 4096)
    t = D.up(x)
    out = D.filled(4096, 0xFFFF)
    B.pc_reduce([t] * 8, out, 4096)
    assert np.array_equal(D.down(out, np.uint16), orc.reduce([x] * 8))


def test_reduce_empty_is_noop(B, D):
    out = D.filled(16, 0x1234)
    e = torch.empty(0, dtype=torch.int16, device="cuda:0")
    assert B.pc_reduce([e, e], e, 0) == B.PC_OK
    assert np.all(D.down(out, np.uint16) == 0x1234)


def test_reduce_large_offsets_sampled(B, D, orc):
    # 4 GiB per rank: byte offsets above 2^32.  Inputs from torch's device RNG;
    # sampled outputs (first/last tiles, the tail and random points) are
    # compared with the oracle run on the sampled inputs.
    n, k = 2, (1 << 31) + 8 * 3
    say("large offsets", n, k)
    g = torch.Generator(device="cuda:0")
    g.manual_seed(7)
    ins = [torch.randint(-32768, 32768, (k,), dtype=torch.int32, device="cuda:0",
                         generator=g).to(torch.int16) for _ in range(n)]
    out = torch.empty(k, dtype=torch.int16, device="cuda:0")
    B.pc_reduce(ins, out, k)
    idx = np.concatenate([np.arange(0, 8192), np.arange(k - 8192, k),
                          np.random.default_rng(3).integers(0, k, 1 << 16)])
    it = torch.from_numpy(idx).to("cuda:0")
    xs = [D.down(t[it], np.uint16) for t in ins]
    got = D.down(out[it], np.uint16)
    assert np.array_equal(got, orc.reduce(xs))
    del ins, out
    torch.cuda.empty_cache()


# ---- Atom copy -------------------------------------------------------------------

# One chunk; whole tiles plus a ragged tail at several sizes on both sides
# of 32 MiB (default loads up to it, non-temporal above), and exactly
# 32 MiB, the last size that keeps the default load policy.
@pytest.mark.parametrize("nbytes", [16, 16 * (256 * 3 + 5), (4 << 20) + 16 * 3, 32 << 20,
                                    (32 << 20) + 16 * 1029, (96 << 20) + 16 * 77])
def test_copy_bytes_unchanged(B, D, nbytes):
    """Every byte arrives unchanged: the expected value is the source itself
    (NaN payloads, subnormals and all other patterns included)."""
    say("copy", nbytes)
    src = np.random.default_rng(nbytes % 1000003).integers(0, 256, nbytes, dtype=np.uint8)
    s = D.up(src)
    d = torch.full((nbytes,), 0xA5, dtype=torch.uint8, device="cuda:0")
    B.pc_copy(d, s, nbytes)
    assert np.array_equal(D.down(d, np.uint8), src)


def test_copy_into_a_window_leaves_the_rest(B, D):
    src = np.random.default_rng(5).integers(0, 256, 4096, dtype=np.uint8)
    d = torch.full((8192,), 0x3C, dtype=torch.uint8, device="cuda:0")
    B.pc_copy(d[1024:], D.up(src), 4096)
    got = D.down(d, np.uint8)
    assert np.array_equal(got[1024:5120], src)
    assert np.all(got[:1024] == 0x3C) and np.all(got[5120:] == 0x3C)


def test_maximum_size_reduce_and_copy(B, D, orc):
    """k = PC_MAX_ELEMS (32 GiB per rank) at N = 2, then a copy of the
    largest size pc_copy accepts (2 * PC_MAX_ELEMS bytes): outputs sampled at
    both ends, around every power-of-two byte offset from 4 GiB and at random
    points, against the oracle on the sampled inputs (copy: the source)."""
    k = 1 << 34
    need = 3 * 2 * k + (2 << 30)
    free, _ = torch.cuda.mem_get_info()
    if free < need:
        pytest.skip(f"needs {need >> 30} GiB of free device memory, {free >> 30} GiB free")
    say("maximum size", 2, k)
    g = torch.Generator(device="cuda:0")
    g.manual_seed(34)
    ins = [torch.empty(k, dtype=torch.int16, device="cuda:0").random_(-32768, 32767, generator=g)
           for _ in range(2)]
    out = torch.empty(k, dtype=torch.int16, device="cuda:0")
    B.pc_reduce(ins, out, k)
    edges = [(1 << b) // 2 for b in range(32, 36)]  # element index at byte offsets 4, 8, 16, 32 GiB
    idx = np.concatenate([np.arange(0, 8192), np.arange(k - 8192, k)] +
                         [np.arange(max(e - 512, 0), min(e + 512, k)) for e in edges] +
                         [np.random.default_rng(34).integers(0, k, 1 << 16)])
    it = torch.from_numpy(idx).to("cuda:0")
    xs = [D.down(t[it], np.uint16) for t in ins]
    assert np.array_equal(D.down(out[it], np.uint16), orc.reduce(xs))
    B.pc_copy(out, ins[1], 2 * k)
    assert np.array_equal(D.down(out[it], np.uint16), xs[1])
    del ins, out, it
    torch.cuda.empty_cache()


# ---- LL pack / consume ---------------------------------------------------------

def gpu_pack(B, D, x, seq):
    src = D.up(x)
    dst = torch.empty(x.size // 2, dtype=torch.int64, device="cuda:0")
    B.pc_pack_ll(src, dst, x.size, seq)
    return dst


def stage_gpu(B, D, case):
    """Stale lines keep the previous call's seq and payload (device side)."""
    staged = []
    for x, s, m in zip(case.payloads(), case.stale_payloads(), case.stale_masks()):
        cur = gpu_pack(B, D, x, case.seq)
        old = gpu_pack(B, D, s, case.stale_seq)
        staged.append(torch.where(torch.from_numpy(m).to("cuda:0"), old, cur))
    return staged


def stage_oracle(orc, case):
    return [np.where(m, orc.pack_ll(s, case.stale_seq), orc.pack_ll(x, case.seq))
            for x, s, m in zip(case.payloads(), case.stale_payloads(), case.stale_masks())]


def test_pack_ll_bits(B, D, orc):
    case = synth.C2_LL_128K
    for x in case.payloads()[:2]:
        assert np.array_equal(D.down(gpu_pack(B, D, x, 7), np.uint64), orc.pack_ll(x, 7))
    x = synth.uniform_bf16(500, 0, 0, 8 * (512 * 3 + 7))
    assert np.array_equal(D.down(gpu_pack(B, D, x, 0xDEADBEEF), np.uint64),
                          orc.pack_ll(x, 0xDEADBEEF))
    # Past 4 MiB per rank (8 input bytes per lane, default loads) and past
    # 64 MiB (non-temporal loads), each with a ragged last tile.
    for seed, chunks in ((501, (1 << 18) + 7), (502, (1 << 22) + 13)):
        x = synth.uniform_bf16(seed, 0, 0, 8 * chunks)
        assert np.array_equal(D.down(gpu_pack(B, D, x, 3), np.uint64), orc.pack_ll(x, 3))
    torch.cuda.empty_cache()


def gpu_consume(B, D, lines_dev, k, seq, out_fill=0xFFFF):
    out = D.filled(k, out_fill)
    bm = torch.full((k // 128,), -1, dtype=torch.int64, device="cuda:0")  # must be overwritten
    B.pc_consume_ll(lines_dev, out, k, seq, bm)
    return D.down(out, np.uint16), D.down(bm, np.uint64)


def test_consume_ll_128k_stale(B, D, orc):
    case = synth.C2_LL_128K
    say(case.name)
    staged_dev = stage_gpu(B, D, case)
    staged = stage_oracle(orc, case)
    for a, b in zip(staged_dev, staged):
        assert np.array_equal(D.down(a, np.uint64), b)
    want_out, want_bm = orc.consume_ll(staged, case.k, case.seq)
    got_out, got_bm = gpu_consume(B, D, staged_dev, case.k, case.seq)
    assert np.array_equal(got_bm, want_bm)
    assert np.array_equal(got_out, want_out)
    ready = int(np.unpackbits(got_bm.view(np.uint8)).sum())
    assert 0.6 * case.lines < ready < 0.72 * case.lines


# The last two shapes pass 4 MiB per rank (two 64-line groups per lane) and
# end in a partial workgroup.
@pytest.mark.parametrize("n,k", [(1, 128), (2, 128 * 3), (3, 128 * 37), (8, 128 * 1001), (5, 1 << 20),
                                 (8, (1 << 21) + 128 * 5), (3, (1 << 22) + 128 * 3)])
def test_consume_ll_shapes(B, D, orc, n, k):
    case = synth.LLCase("shape", 600 + n, n, k, stale_frac=0.03)
    staged = stage_oracle(orc, case)
    want_out, want_bm = orc.consume_ll(staged, k, case.seq)
    got_out, got_bm = gpu_consume(B, D, [D.up(s) for s in staged], k, case.seq)
    assert np.array_equal(got_bm, want_bm)
    assert np.array_equal(got_out, want_out)


@pytest.mark.parametrize("n", [1, 2, 3, 4, 5, 6, 7, 8])
def test_consume_ll_bandwidth_regime(B, D, orc, n):
    # From 512 MiB of lines read plus results written the consumer is the
    # persistent kernel.  Five 64-line groups past that size leave a ragged
    # last 2048-line tile; ranks 0, 3 and 6 carry about 2% lines of the
    # previous call (the stale payload packed with the stale sequence number).
    nl = (-(-(512 << 20) // (8 * n + 4)) // 64 + 5) * 64
    k = 2 * nl
    say("consume_ll bandwidth regime", n, k)
    pick = np.random.default_rng(800 + n)
    staged = []
    for r in range(n):
        lines = orc.pack_ll(synth.uniform_bf16(800 + n, 0, r, k), synth.SEQ_CURRENT)
        if r % 3 == 0:
            idx = np.flatnonzero(pick.random(nl) < 0.02)
            stale = orc.pack_ll(synth.uniform_bf16(800 + n, 1, r, k, 2.0, 3.0), synth.SEQ_STALE)
            lines[idx] = stale[idx]
        staged.append(lines)
    want_out, want_bm = orc.consume_ll(staged, k, synth.SEQ_CURRENT)
    got_out, got_bm = gpu_consume(B, D, [D.up(s) for s in staged], k, synth.SEQ_CURRENT)
    assert np.array_equal(got_bm, want_bm)
    assert np.array_equal(got_out, want_out)
    del staged
    torch.cuda.empty_cache()


def test_consume_ll_lines_not_torn_under_concurrent_pack(B, D, orc):
    """The LL protocol needs a line's data and sequence number to be observed
    together.  A side stream rewrites 2M lines 64 times, alternating between
    two payloads with their own sequence numbers, while the main stream
    consumes them 32 times into separate outputs.  Every line a consume marks
    ready must hold that version's payload (the oracle's fold of it, one
    rank); every other line keeps the prefill.  Consumes that saw part of a
    rewrite show the race was exercised; if none did, the test is skipped."""
    k = 1 << 22
    nl = k // 2
    seqs = (5, 6)
    pays = [synth.uniform_bf16(1900, v, 0, k) for v in range(2)]
    want = [orc.reduce([p]).reshape(-1, 2) for p in pays]
    src = [D.up(p) for p in pays]
    lines = torch.empty(nl, dtype=torch.int64, device="cuda:0")
    B.pc_pack_ll(src[0], lines, k, seqs[0])
    calls = 32
    outs = [D.filled(k, 0xFFFF) for _ in range(calls)]
    bms = [torch.full((nl // 64,), -1, dtype=torch.int64, device="cuda:0") for _ in range(calls)]
    side = torch.cuda.Stream()
    torch.cuda.synchronize()
    for i in range(2 * calls):
        v = (i + 1) % 2
        B.pc_pack_ll(src[v], lines, k, seqs[v], stream=side)
        if i % 2 == 0:
            j = i // 2
            B.pc_consume_ll([lines], outs[j], k, seqs[j % 2], bms[j])
    torch.cuda.synchronize()
    partial = 0
    for j in range(calls):
        bm = D.down(bms[j], np.uint64)
        ready = np.unpackbits(bm.view(np.uint8), bitorder="little").astype(bool)  # bit l of word w: line 64w + l
        got = D.down(outs[j], np.uint16).reshape(-1, 2)
        assert np.array_equal(got[ready], want[j % 2][ready]), j
        assert np.all(got[~ready] == 0xFFFF), j
        partial += int(0 < ready.sum() < nl)
    say("concurrent pack: consumes that saw part of a rewrite", partial, "of", calls)
    if partial == 0:
        pytest.skip("no consume overlapped a rewrite")


def test_consume_ll_one_rank_identity_all_patterns(B, D, orc):
    allh = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    lines = gpu_pack(B, D, allh, 9)
    got_out, got_bm = gpu_consume(B, D, [lines], allh.size, 9)
    want_out, want_bm = orc.consume_ll([orc.pack_ll(allh, 9)], allh.size, 9)
    assert np.array_equal(got_out, want_out)
    assert np.array_equal(got_bm, want_bm)


def test_consume_ll_wrong_seq_and_late_arrival(B, D, orc):
    case = synth.LLCase("late", 700, 8, 8192)
    staged = [D.up(s) for s in stage_oracle(orc, case)]
    out, bm = gpu_consume(B, D, staged, case.k, 8)             # nothing carries seq 8
    assert np.all(bm == 0) and np.all(out == 0xFFFF)
    # First consume sees the partial arrival, second after the late lines land.
    out_t = D.filled(case.k, 0xFFFF)
    bm_t = torch.empty(case.k // 128, dtype=torch.int64, device="cuda:0")
    B.pc_consume_ll(staged, out_t, case.k, case.seq, bm_t)
    landed = [gpu_pack(B, D, x, case.seq) for x in case.payloads()]
    B.pc_consume_ll(landed, out_t, case.k, case.seq, bm_t)
    assert np.all(D.down(bm_t, np.uint64) == np.uint64(0xFFFFFFFFFFFFFFFF))
    assert np.array_equal(D.down(out_t, np.uint16), orc.reduce(case.payloads()))


# ---- twoshot -------------------------------------------------------------------

TWOSHOT_MODES = ["two", "fused", "linked"]


def linked_workspace(B, n, k):
    """A zero-filled workspace for pc_twoshot_linked (uint64 words)."""
    nbytes = B.pc_twoshot_linked_workspace_bytes(n, k)
    assert nbytes > 0
    return torch.zeros((nbytes + 7) // 8, dtype=torch.int64, device="cuda:0")


def check_linked_workspace(B, D, ws, calls):
    """After `calls` calls every workgroup's call counter reads `calls` and
    no wait was abandoned."""
    w = D.down(ws, np.uint64)
    assert np.all(w[:B.PC_LINKED_GROUPS] == calls), np.unique(w[:B.PC_LINKED_GROUPS])
    assert w[B.PC_LINKED_STATUS_WORD] == 0


def run_twoshot(B, ins, outs, k, mode, ws=None):
    if mode == "two":
        B.pc_twoshot(ins, outs, k)
    elif mode == "fused":
        B.pc_twoshot_fused(ins, outs, k)
    else:
        B.pc_twoshot_linked(ins, outs, k, ws)


def gpu_twoshot(B, D, xs, mode="two"):
    k = xs[0].size
    ins = [D.up(x) for x in xs]
    outs = [D.filled(k, 0xFFFF) for _ in xs]
    ws = linked_workspace(B, len(xs), k) if mode == "linked" else None
    run_twoshot(B, ins, outs, k, mode, ws)
    got = [D.down(o, np.uint16) for o in outs]
    if ws is not None:
        check_linked_workspace(B, D, ws, 1)
    return got


@pytest.mark.parametrize("mode", TWOSHOT_MODES)
def test_twoshot_1m(B, D, orc, mode):
    case = synth.C3_TWOSHOT_1M
    say(case.name, mode)
    xs = case.inputs()
    want = orc.twoshot(xs)
    got = gpu_twoshot(B, D, xs, mode)
    oneshot = gpu_reduce(B, D, xs)
    for g, w in zip(got, want):
        assert np.array_equal(g, w)
        assert np.array_equal(g, oneshot)


# Slices of 1 chunk, ragged tiles, and for the linked form every tile size
# (1, 2 and 4 chunks per lane) with more tiles than its grid has workgroups.
@pytest.mark.parametrize("mode", TWOSHOT_MODES)
@pytest.mark.parametrize("n,slice_chunks", [(2, 1), (3, 257), (5, 256 * 4 + 3), (8, 300000 + 5),
                                            (1, 100), (6, 2 * 262144 + 9), (3, 100003),
                                            (8, 512 * 40 + 17), (7, 1024 * 70 + 1)])
def test_twoshot_shapes(B, D, orc, n, slice_chunks, mode):
    k = 8 * n * slice_chunks
    say("twoshot", n, k, mode)
    xs = [synth.normal_bf16(800 + n, 0, r, k) for r in range(n)]
    want = orc.reduce(xs, threads=THREADS)
    for g in gpu_twoshot(B, D, xs, mode):
        assert np.array_equal(g, want)


# From 48 MiB per rank the copies of the two-launch and the flag-linked forms
# carry the non-temporal hint, and at 7 and 8 ranks the two-launch form's
# copies go one destination per workgroup; just below and past that size,
# with ragged slices.
@pytest.mark.parametrize("n,per_rank_mib,extra", [(8, 48, 3), (8, 47, 5), (2, 50, 1), (5, 64, 7), (7, 49, 3),
                                                  (7, 47, 1)])
def test_twoshot_copies_nontemporal(B, D, orc, n, per_rank_mib, extra):
    sc = (per_rank_mib << 20) // (16 * n) + extra       # chunks per slice
    k = 8 * n * sc
    say("twoshot nt copies", n, k)
    xs = [synth.normal_bf16(1700 + n, 0, r, k) for r in range(n)]
    want = orc.reduce(xs, threads=THREADS)
    for mode in ("two", "linked"):
        for g in gpu_twoshot(B, D, xs, mode):
            assert np.array_equal(g, want), mode
    torch.cuda.empty_cache()


# From a working set (inputs plus outputs) of 640 MiB with five or more
# ranks, pc_twoshot_fused folds every tile into its owner's output first and
# hands it out afterwards.  Slice sizes just below and past that switch for
# 5..8 ranks, ragged against the tiles, once in place, and four ranks past
# the size (which keep the single fan-out pass).
@pytest.mark.parametrize("n,extra,in_place", [(8, -1, False), (8, 3, False), (8, 5, True), (7, 2, False),
                                              (6, 1, False), (5, 7, False), (4, 9, False)])
def test_twoshot_fused_fold_then_hand_out(B, D, orc, n, extra, in_place):
    switch = 640 << 20
    sc = switch // (32 * n * n) + extra                 # chunks per slice
    k = 8 * n * sc
    split = n >= 5 and 2 * n * (2 * k) >= switch
    assert split == (n >= 5 and extra >= 0)
    say("twoshot fused", n, k, "fold then hand out" if split else "single pass", "in place" if in_place else "")
    xs = [synth.normal_bf16(1750 + n, 0, r, k) for r in range(n)]
    want = orc.reduce(xs, threads=THREADS)
    ins = [D.up(x) for x in xs]
    outs = ins if in_place else [D.filled(k, 0xFFFF) for _ in range(n)]
    B.pc_twoshot_fused(ins, outs, k)
    for r, o in enumerate(outs):
        assert np.array_equal(D.down(o, np.uint16), want), r
    del ins, outs
    torch.cuda.empty_cache()


@pytest.mark.parametrize("mode", TWOSHOT_MODES)
def test_twoshot_in_place(B, D, orc, mode):
    n, k = 4, 8 * 4 * 999
    xs = [synth.normal_bf16(900, 0, r, k) for r in range(n)]
    ins = [D.up(x) for x in xs]
    ws = linked_workspace(B, n, k) if mode == "linked" else None
    run_twoshot(B, ins, ins, k, mode, ws)
    want = orc.reduce(xs)
    for t in ins:
        assert np.array_equal(D.down(t, np.uint16), want)


@pytest.mark.parametrize("n", [1, 2, 3, 4, 5, 6, 7, 8])
def test_bandwidth_regime_every_n(B, D, orc, n):
    """Every rank count in the persistent (bandwidth-regime) kernels: a
    working set just past 64 MiB with ragged slices, for the reduce with a
    permuted order and for all three twoshot forms."""
    sc = -(-(4 << 20) // (n * (n + 1))) + 3          # chunks per slice
    k = 8 * n * sc
    say("bandwidth regime", n, k)
    xs = [synth.normal_bf16(1600 + n, 0, r, k) for r in range(n)]
    order = list(np.random.default_rng(40 + n).permutation(n))
    assert np.array_equal(gpu_reduce(B, D, xs, order=order),
                          orc.reduce(xs, order=order, threads=THREADS))
    want = orc.reduce(xs, threads=THREADS)
    for mode in TWOSHOT_MODES:
        for g in gpu_twoshot(B, D, xs, mode):
            assert np.array_equal(g, want), mode
    torch.cuda.empty_cache()


@pytest.mark.parametrize("n", [2, 3])
def test_short_lived_reduce_few_ranks(B, D, orc, n):
    """Two and three ranks from 128 MiB per rank take short-lived 8 KiB
    workgroups (one rank does throughout the bandwidth regime, as in the
    test above): the oneshot with a permuted order, and twoshot phase 1 on
    ragged slices, each with a ragged last tile."""
    chunks = (8 << 20) + 773                          # 128 MiB + 12,368 B per rank
    k = 8 * chunks
    say("short-lived reduce", n, k)
    xs = [synth.uniform_bf16(1800 + n, 0, r, k) for r in range(n)]
    order = list(np.random.default_rng(80 + n).permutation(n))
    assert np.array_equal(gpu_reduce(B, D, xs, order=order),
                          orc.reduce(xs, order=order, threads=THREADS))
    sc = -(-chunks // n) + 5
    k2 = 8 * n * sc
    xs2 = [synth.uniform_bf16(1810 + n, 0, r, k2) for r in range(n)]
    want = orc.reduce(xs2, threads=THREADS)
    for g in gpu_twoshot(B, D, xs2, "two"):
        assert np.array_equal(g, want)
    torch.cuda.empty_cache()


@pytest.mark.parametrize("n", [4, 5, 8])
def test_staged_reduce_every_batch_remainder(B, D, orc, n):
    """The LDS-staged persistent reduce (four or more ranks, working set of
    64 MiB or more) takes a workgroup's tiles in batches of 8 and the rest
    in batches of 4, 2 and 1.  3,839 tiles of 1,024 chunks (plus a ragged
    tail) on 256 CUs give every workgroup 14 or 15 tiles: 8 + 4 + 2 and
    8 + 4 + 2 + 1.  The oneshot runs it with a permuted order, twoshot
    phase 1 with 3,839 tiles over n slices."""
    chunks = 3838 * 1024 + 517
    k = 8 * chunks
    say("staged reduce remainders", n, k)
    xs = [synth.uniform_bf16(1700 + n, 0, r, k) for r in range(n)]
    order = list(np.random.default_rng(70 + n).permutation(n))
    assert np.array_equal(gpu_reduce(B, D, xs, order=order),
                          orc.reduce(xs, order=order, threads=THREADS))
    sc = -(-3839 * 1024 // n) - 3                     # ragged slices, 128-byte grid
    k2 = 8 * n * sc
    xs2 = [synth.uniform_bf16(1710 + n, 0, r, k2) for r in range(n)]
    want = orc.reduce(xs2, threads=THREADS)
    for g in gpu_twoshot(B, D, xs2, "two"):
        assert np.array_equal(g, want)
    torch.cuda.empty_cache()


@pytest.mark.parametrize("n", [4, 5, 8])
def test_staged_reduce_whole_tiles(B, D, orc, n):
    """Slices that are whole numbers of 1,024-chunk tiles take the staged
    kernel built with a constant tile size: 3,840 whole tiles on 256 CUs,
    15 per workgroup (8 + 4 + 2 + 1), for the oneshot (permuted order) and
    for twoshot phase 1 with slices of whole tiles."""
    chunks = 3840 * 1024
    k = 8 * chunks
    say("staged reduce whole tiles", n, k)
    xs = [synth.uniform_bf16(1800 + n, 0, r, k) for r in range(n)]
    order = list(np.random.default_rng(80 + n).permutation(n))
    assert np.array_equal(gpu_reduce(B, D, xs, order=order),
                          orc.reduce(xs, order=order, threads=THREADS))
    sc = 1024 * -(-3840 // n)                           # whole tiles per slice
    k2 = 8 * n * sc
    xs2 = [synth.uniform_bf16(1810 + n, 0, r, k2) for r in range(n)]
    want = orc.reduce(xs2, threads=THREADS)
    for g in gpu_twoshot(B, D, xs2, "two"):
        assert np.array_equal(g, want)
    torch.cuda.empty_cache()


@pytest.mark.parametrize("n", [4, 7, 8])
@pytest.mark.parametrize("shape", ["whole", "ragged"])
@pytest.mark.parametrize("layout", ["congruent", "skewed"])
def test_staged_reduce_rank_layouts(B, D, orc, n, shape, layout):
    """The staged kernels take the ranks on a diagonal when every rank
    buffer's base agrees with rank 0's modulo 32 KiB, and the plain pipeline
    otherwise.  The rank buffers are carved from one allocation at a stride
    that is a multiple of 32 KiB (congruent) or 4 KiB more (skewed), with
    whole 1,024-chunk tiles or a ragged tail, for the oneshot (permuted order),
    twoshot phase 1 and the flag-linked twoshot's staged phase 1."""
    if shape == "whole":
        chunks = n * 1024 * -(-3840 // n)              # whole tiles, also per twoshot slice
    else:
        chunks = 3838 * 1024 + 517
        chunks -= chunks % n                           # twoshot slices: k a multiple of 8 n
    k = 8 * chunks
    stride = -(-2 * k // 32768) * 32768 // 2 + (2048 if layout == "skewed" else 0)   # elements
    say("staged reduce layouts", n, k, shape, layout)
    base = torch.empty(stride * n, dtype=torch.int16, device="cuda:0")
    views = [base[r * stride:r * stride + k] for r in range(n)]
    congruent = all((v.data_ptr() - views[0].data_ptr()) % 32768 == 0 for v in views)
    assert congruent == (layout == "congruent")
    xs = [synth.uniform_bf16(1900 + n, 0, r, k) for r in range(n)]
    for v, x in zip(views, xs):
        v.copy_(torch.from_numpy(x.view(np.int16)).to("cuda:0"))
    order = list(np.random.default_rng(90 + n).permutation(n))
    out = D.filled(k, 0xFFFF)
    B.pc_reduce(views, out, k, order=order)
    assert np.array_equal(D.down(out, np.uint16), orc.reduce(xs, order=order, threads=THREADS))
    want = orc.reduce(xs, threads=THREADS)
    outs = [D.filled(k, 0xFFFF) for _ in range(n)]
    B.pc_twoshot(views, outs, k)
    for o in outs:
        assert np.array_equal(D.down(o, np.uint16), want)
    ws = linked_workspace(B, n, k)                      # the linked twoshot's staged phase 1
    for o in outs:
        o.fill_(-1)
    B.pc_twoshot_linked(views, outs, k, ws)
    for o in outs:
        assert np.array_equal(D.down(o, np.uint16), want)
    check_linked_workspace(B, D, ws, 1)
    del base, views, outs, ws
    torch.cuda.empty_cache()


def test_twoshot_linked_reuses_workspace_across_sizes(B, D, orc):
    """One workspace, many calls of different n and k (tile geometry changes
    between calls): the flags of earlier calls are never taken as ready, and
    every workgroup's counter advances once per call."""
    shapes = [(8, 8 * 65536), (3, 3 * 8 * 5000), (8, 8 * 65536), (8, 8 * 8 * 1024 * 70),
              (2, 16), (5, 5 * 8 * 256 * 3)]
    nbytes = max(B.pc_twoshot_linked_workspace_bytes(n, k) for n, k in shapes)
    ws = torch.zeros(nbytes // 8, dtype=torch.int64, device="cuda:0")
    for i, (n, k) in enumerate(shapes):
        say("linked reuse", i, n, k)
        xs = [synth.uniform_bf16(1500 + i, 0, r, k) for r in range(n)]
        ins = [D.up(x) for x in xs]
        outs = [D.filled(k, 0xFFFF) for _ in range(n)]
        B.pc_twoshot_linked(ins, outs, k, ws)
        want = orc.reduce(xs, threads=THREADS)
        for o in outs:
            assert np.array_equal(D.down(o, np.uint16), want), (i, n, k)
        check_linked_workspace(B, D, ws, i + 1)


def test_twoshot_linked_first_call_inside_a_capture(B):
    """A fresh process whose first linked call is captured in a graph."""
    import subprocess
    import sys
    here = os.path.dirname(os.path.abspath(__file__))
    r = subprocess.run([sys.executable, os.path.join(here, "linked_capture_first.py")],
                       capture_output=True, text=True, timeout=240)
    assert r.returncode == 0 and "OK" in r.stdout, r.stdout[-2000:] + r.stderr[-2000:]


def test_twoshot_linked_empty_call_leaves_counters(B, D):
    ws = linked_workspace(B, 4, 0)
    B.pc_twoshot_linked([0] * 4, [0] * 4, 0, ws)
    check_linked_workspace(B, D, ws, 0)


# ---- all-gather copy -------------------------------------------------------------

def gpu_allgather(B, D, recs, n, shard_bytes, seq):
    shards = [D.up(r) for r in recs]
    out = D.filled(n * shard_bytes // 2, 0xFFFF)
    bm = torch.full((n * shard_bytes // 128 // 64,), -1, dtype=torch.int64, device="cuda:0")
    B.pc_allgather_copy(shards, out, shard_bytes, seq, bm)
    return D.down(out, np.uint16), D.down(bm, np.uint64)


def test_allgather_2m_stale(B, D, orc):
    case = synth.C5_ALLGATHER_2M
    say(case.name)
    recs, _ = case.records()
    want_out, want_bm = orc.allgather_copy(recs, case.shard_bytes, case.seq)
    got_out, got_bm = gpu_allgather(B, D, recs, case.n, case.shard_bytes, case.seq)
    assert np.array_equal(got_bm, want_bm)
    assert np.array_equal(got_out, want_out)
    assert int(np.unpackbits(got_bm.view(np.uint8)).sum()) == 131072 - 8 * 1638


# The last two move 768 MiB or more (records read plus payloads written),
# where the staging loads carry the non-temporal hint and a workgroup takes
# 32 records (half a bitmap word); the one before sits just below that.
@pytest.mark.parametrize("n,shard_bytes,frac", [(1, 8192, 0.5), (3, 8192 * 3, 0.1),
                                                 (8, 8192 * 17, 0.0), (2, 8192 * 5, 1.0),
                                                 (8, (46 << 20) + 8192 * 7, 0.1),
                                                 (8, (47 << 20) + 8192 * 3, 0.1),
                                                 (3, (125 << 20) + 8192 * 5, 0.05)])
def test_allgather_shapes(B, D, orc, n, shard_bytes, frac):
    say("allgather", n, shard_bytes)
    case = synth.GatherCase("shape", 1000 + n, n, shard_bytes, stale_frac=frac)
    recs, _ = case.records()
    want_out, want_bm = orc.allgather_copy(recs, shard_bytes, case.seq)
    got_out, got_bm = gpu_allgather(B, D, recs, n, shard_bytes, case.seq)
    assert np.array_equal(got_bm, want_bm)
    assert np.array_equal(got_out, want_out)


def test_allgather_header_compared_as_u64(B, D, orc):
    # A header whose low 32 bits match seq but high bits differ is stale.
    case = synth.GatherCase("hi bits", 1100, 2, 8192, stale_frac=0.0)
    recs, _ = case.records()
    recs[1] = recs[1].copy()
    recs[1].view(np.uint64)[17 * 5] = np.uint64((1 << 32) | case.seq)
    want_out, want_bm = orc.allgather_copy(recs, 8192, case.seq)
    got_out, got_bm = gpu_allgather(B, D, recs, 2, 8192, case.seq)
    assert np.array_equal(got_bm, want_bm) and np.array_equal(got_out, want_out)
    assert int(np.unpackbits(got_bm.view(np.uint8)).sum()) == 127


# ---- sentinel readiness -------------------------------------------------------------

def gpu_publish(B, D, x):
    src = D.up(x)
    slot = torch.empty_like(src)
    B.pc_publish_sentinel(src, slot, x.size)
    return slot


def gpu_consume_sentinel(B, D, slots_dev, k, out_fill=0xFFFF):
    out = D.filled(k, out_fill)
    bm = torch.full((k // 512,), -1, dtype=torch.int64, device="cuda:0")
    B.pc_consume_sentinel(slots_dev, out, k, bm)
    return D.down(out, np.uint16), D.down(bm, np.uint64), [D.down(s, np.uint16) for s in slots_dev]


def test_publish_sentinel_bits(B, D, orc):
    allh = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    assert np.array_equal(D.down(gpu_publish(B, D, allh), np.uint16), orc.publish_sentinel(allh))
    x = synth.SentinelCase("pub", 72, 1, 8 * 777).payloads()[0]
    assert np.array_equal(D.down(gpu_publish(B, D, x), np.uint16), orc.publish_sentinel(x))
    t = D.up(x)                                          # in place
    B.pc_publish_sentinel(t, t, x.size)
    assert np.array_equal(D.down(t, np.uint16), orc.publish_sentinel(x))
    # Past 4 MiB per rank (one 4 KiB tile per workgroup), with a ragged tail.
    x = synth.SentinelCase("pub big", 74, 1, 8 * ((1 << 18) + 5)).payloads()[0]
    assert np.array_equal(D.down(gpu_publish(B, D, x), np.uint16), orc.publish_sentinel(x))


@pytest.mark.parametrize("chunks,in_place", [(1 << 21, False), ((1 << 21) + 1, True), ((1 << 24) + 5, False),
                                             ((1 << 24) + 1027, True)])
def test_publish_sentinel_bandwidth_regime(B, D, orc, chunks, in_place):
    # From 4 MiB the publisher takes one 4 KiB tile per workgroup, with
    # default loads up to 32 MiB (the first size is that edge) and
    # non-temporal ones above it (the second, in place, is one chunk past it;
    # the last two are 256 MiB with ragged last tiles, one in place).
    # Uniformly random bit patterns include the sentinel.
    k = 8 * chunks
    say("publish bandwidth regime", k, in_place)
    x = np.random.default_rng(chunks).integers(0, 1 << 16, k, dtype=np.uint32).astype(np.uint16)
    want = orc.publish_sentinel(x)
    if in_place:
        t = D.up(x)
        B.pc_publish_sentinel(t, t, k)
        got = D.down(t, np.uint16)
    else:
        got = D.down(gpu_publish(B, D, x), np.uint16)
    assert np.array_equal(got, want)
    torch.cuda.empty_cache()


def test_consume_sentinel_128k_workload(B, D, orc):
    case = synth.C2S_SENTINEL_128K
    say(case.name)
    xs, ms = case.payloads(), case.masks()
    # Each side publishes with its own code; unarrived/torn packs are then
    # put back to the sentinel by the test.
    dev = [synth.unarrive(D.down(gpu_publish(B, D, x), np.uint16), m, t) for x, (m, t) in zip(xs, ms)]
    host = [synth.unarrive(orc.publish_sentinel(x), m, t) for x, (m, t) in zip(xs, ms)]
    for a, b in zip(dev, host):
        assert np.array_equal(a, b)
    want_out, want_bm, want_slots = orc.consume_sentinel(host, case.k)
    got_out, got_bm, got_slots = gpu_consume_sentinel(B, D, [D.up(s) for s in dev], case.k)
    assert np.array_equal(got_bm, want_bm)
    assert np.array_equal(got_out, want_out)
    for g, w in zip(got_slots, want_slots):
        assert np.array_equal(g, w)
    ready = int(np.unpackbits(got_bm.view(np.uint8)).sum())
    assert 0.6 * case.packs < ready < 0.7 * case.packs


@pytest.mark.parametrize("n,k", [(1, 512), (2, 512 * 3), (3, 512 * 37), (5, 512 * 129), (8, 1 << 20),
                                 (8, (1 << 21) + 512 * 3)])
def test_consume_sentinel_shapes(B, D, orc, n, k):
    case = synth.SentinelCase("shape", 73 + n, n, k, 0.03, 0.01, 0.01)
    slots = [synth.unarrive(orc.publish_sentinel(x), m, t)
             for x, (m, t) in zip(case.payloads(), case.masks())]
    want_out, want_bm, want_slots = orc.consume_sentinel(slots, k)
    got_out, got_bm, got_slots = gpu_consume_sentinel(B, D, [D.up(s) for s in slots], k)
    assert np.array_equal(got_bm, want_bm)
    assert np.array_equal(got_out, want_out)
    assert all(np.array_equal(g, w) for g, w in zip(got_slots, want_slots))


def consume_sentinel_bandwidth_regime(B, D, orc, n, k):
    pick = np.random.default_rng(900 + n)
    slots = []
    for r in range(n):
        slot = orc.publish_sentinel(synth.uniform_bf16(900 + n, 0, r, k))
        if r % 3 == 0:
            roll = pick.random(k // 8)
            slot = synth.unarrive(slot, roll < 0.02, (roll >= 0.02) & (roll < 0.03))
        slots.append(slot)
    want_out, want_bm, want_slots = orc.consume_sentinel(slots, k)
    got_out, got_bm, got_slots = gpu_consume_sentinel(B, D, [D.up(s) for s in slots], k)
    assert np.array_equal(got_bm, want_bm)
    assert np.array_equal(got_out, want_out)
    assert all(np.array_equal(g, w) for g, w in zip(got_slots, want_slots))
    del slots, got_slots, want_slots
    torch.cuda.empty_cache()


@pytest.mark.parametrize("n", [1, 2, 3, 4, 5, 6, 7, 8])
def test_consume_sentinel_bandwidth_regime(B, D, orc, n):
    # From 768 MiB of slots read plus results and re-arms written the call
    # runs as a persistent fold and a separate re-arm pass.  Three 512-element
    # units past that size leave ragged last blocks; ranks 0, 3 and 6 have
    # about 2% of their packs missing and 1% torn (upper half unwritten).
    k = (-(-(768 << 20) // (2 * (2 * n + 1))) // 512 + 3) * 512
    say("consume_sentinel bandwidth regime", n, k)
    consume_sentinel_bandwidth_regime(B, D, orc, n, k)


@pytest.mark.parametrize("n", [4, 8])
def test_consume_sentinel_bandwidth_regime_whole_tiles(B, D, orc, n):
    # The same past the switch with k a multiple of 8,192 elements: every
    # 1,024-pack tile of the fold is whole, with no ragged last tile.
    k = -(-(768 << 20) // (2 * (2 * n + 1) * 8192)) * 8192
    say("consume_sentinel bandwidth regime, whole tiles", n, k)
    consume_sentinel_bandwidth_regime(B, D, orc, n, k)


def test_consume_sentinel_late_arrival(B, D, orc):
    case = synth.SentinelCase("late", 80, 8, 8192)
    xs, ms = case.payloads(), case.masks()
    slots = [D.up(synth.unarrive(orc.publish_sentinel(x), m, t)) for x, (m, t) in zip(xs, ms)]
    out = D.filled(case.k, 0xFFFF)
    bm = torch.empty(case.k // 512, dtype=torch.int64, device="cuda:0")
    B.pc_consume_sentinel(slots, out, case.k, bm)
    first = D.down(bm, np.uint64).copy()
    # The producers now publish everything; packs consumed in the first round
    # are published again into their re-armed storage.
    done = np.repeat(np.unpackbits(first.view(np.uint8), bitorder="little").astype(bool), 8)
    for s, x in zip(slots, xs):
        fresh = D.down(gpu_publish(B, D, x), np.uint16)
        cur = D.down(s, np.uint16)
        s.copy_(D.up(np.where(done, cur, fresh).astype(np.uint16)))
    B.pc_consume_sentinel(slots, out, case.k, bm)
    second = D.down(bm, np.uint64)
    assert np.all((first | second) == np.uint64(0xFFFFFFFFFFFFFFFF)) and np.all((first & second) == 0)
    assert np.array_equal(D.down(out, np.uint16), orc.reduce(xs))
    assert all(np.all(D.down(s, np.uint16) == 0xFFFF) for s in slots)



# ---- speculative reduce with a folded validation flag ---------------------------------

def gpu_validated(B, D, xs, flags, t, flag, max_attempts=1):
    k = xs[0].size
    ins = [D.up(x) for x in xs]
    fl = [torch.from_numpy(f.view(np.int32)).to("cuda:0") for f in flags]
    out = D.filled(k, 0xFFFF)
    at = torch.full((k // t,), -1, dtype=torch.int32, device="cuda:0")
    B.pc_reduce_validated(ins, fl, out, k, t, flag, max_attempts, at)
    return D.down(out, np.uint16), D.down(at, np.uint32)


@pytest.mark.parametrize("n,t,tiles", [(1, 2048, 3), (3, 4096, 5), (5, 6144, 7), (8, 8192, 33),
                                       (8, 2048, 1025)])
def test_reduce_validated_shapes(B, D, orc, n, t, tiles):
    case = synth.ValidatedCase("v", 81 + n, n, t * tiles, t, flag=0x1234, stale_frac=0.1)
    xs, fl = case.payloads(), case.flags()
    want_out, want_ok = orc.reduce_validated(xs, fl, t, case.flag)
    got_out, got_at = gpu_validated(B, D, xs, fl, t, case.flag)
    assert np.array_equal(got_at, want_ok)              # static inputs: attempt 1 or never
    assert np.array_equal(got_out, want_out)


def test_reduce_validated_decode_and_retry_bound(B, D, orc):
    case = synth.C1V_VALIDATED_8K
    xs, fl = case.payloads(), case.flags()
    got_out, got_at = gpu_validated(B, D, xs, fl, case.elems_per_flag, case.flag)
    assert list(got_at) == [1] and np.array_equal(got_out, orc.reduce(xs))
    # A rank that never reaches the call: every attempt fails, the call ends.
    stale = [f.copy() for f in fl]
    stale[3][0] -= 1
    got_out, got_at = gpu_validated(B, D, xs, stale, case.elems_per_flag, case.flag, max_attempts=64)
    assert list(got_at) == [0] and np.all(got_out == 0xFFFF)


def test_reduce_validated_flags_fold_and_wrap(B, D, orc):
    n, t = 3, 2048
    xs = [synth.uniform_bf16(90, 0, r, t) for r in range(n)]
    comp = [np.array([6], np.uint32), np.array([8], np.uint32), np.array([7], np.uint32)]
    got_out, got_at = gpu_validated(B, D, xs, comp, t, 7)
    assert list(got_at) == [1] and np.array_equal(got_out, orc.reduce(xs))
    top = [np.array([0xFFFFFFFF], np.uint32)] * n
    got_out, got_at = gpu_validated(B, D, xs, top, t, 0xFFFFFFFF)
    assert list(got_at) == [1]


def test_reduce_validated_concurrent_arrival(B, D, orc):
    """A rank's flags arrive while the call is retrying: a kernel on a second
    stream rewrites them after a bounded spin.  Retries re-read flags and
    payload past the caches, so every tile validates once the rewrite is
    visible, with the oracle's result; validating after the first attempt
    shows the retry path at work.  All tiles validating at once means the
    rewrite came first (skipped: nothing exercised).  Every tile giving up is
    a failure if the rewrite finished well before the call did (the retries
    then read stale data), and otherwise means the streams did not overlap
    (skipped).  A mix of tiles that gave up and tiles that validated fails."""
    n, epf, tiles, flag = 8, 2048, 64, 41
    k = epf * tiles
    xs = [synth.uniform_bf16(97, 0, r, k) for r in range(n)]
    ins = [D.up(x) for x in xs]
    fl = [torch.full((tiles,), flag, dtype=torch.int32, device="cuda:0") for _ in range(n)]
    fl[3].fill_(flag - 1)                                   # rank 3 has not arrived
    out = D.filled(k, 0xFFFF)
    at = torch.full((tiles,), -1, dtype=torch.int32, device="cuda:0")
    side = torch.cuda.Stream()
    done_call = torch.cuda.Event(enable_timing=True)
    done_flags = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    B.pc_reduce_validated(ins, fl, out, k, epf, flag, 65536, at)
    done_call.record()
    with torch.cuda.stream(side):
        torch.cuda._sleep(100000)
        fl[3].fill_(flag)
        done_flags.record()
    torch.cuda.synchronize()
    lead_ms = done_flags.elapsed_time(done_call)             # > 0: the rewrite finished first
    got_at = D.down(at, np.uint32)
    got = D.down(out, np.uint16)
    say("concurrent arrival: attempts", int(got_at.min()), "to", int(got_at.max()),
        "; rewrite finished", round(lead_ms, 4), "ms before the call")
    if np.all(got_at == 0):
        assert lead_ms < 5.0, "flags rewritten long before the call ended, but no tile validated"
        assert np.all(got == 0xFFFF)
        pytest.skip("the call gave up before the rewrite: the streams did not overlap")
    assert np.all(got_at >= 1), np.unique(got_at)
    assert np.array_equal(got, orc.reduce(xs))
    if np.all(got_at == 1):
        pytest.skip("the rewrite came before the call's first read: no retry was needed")


def test_reduce_validated_in_place(B, D, orc):
    n, t = 4, 4096
    xs = [synth.uniform_bf16(91, 0, r, 4 * t) for r in range(n)]
    ins = [D.up(x) for x in xs]
    fl = [torch.full((4,), 5, dtype=torch.int32, device="cuda:0") for _ in range(n)]
    at = torch.empty(4, dtype=torch.int32, device="cuda:0")
    B.pc_reduce_validated(ins, fl, ins[1], 4 * t, t, 5, 1, at)
    assert np.array_equal(D.down(ins[1], np.uint16), orc.reduce(xs))


# Working sets of 320 MiB and more run on the persistent kernel (two
# workgroups per CU taking batches of 16, 8 or, at 6144 elements per flag, 2
# tiles), or at 8192 elements per flag with four or more ranks on the
# LDS-staged one.  Three tiles past that size leave the last batch of most workgroups
# partly empty.  The flag's multiple wraps mod 2^32, and a tenth of the tiles
# carry a stale flag on some rank.
@pytest.mark.parametrize("n,t,tiles,in_place", [(8, 8192, 2279, False), (8, 2048, 9106, False),
                                                (8, 4096, 4555, False), (2, 4096, 13657, False),
                                                (1, 8192, 10243, False), (5, 6144, 4555, False),
                                                (3, 2048, 20483, False), (6, 4096, 5855, False),
                                                (7, 8192, 2563, False), (4, 8192, 4099, True),
                                                (5, 8192, 3415, False), (6, 8192, 2927, True)])
def test_reduce_validated_bandwidth_regime(B, D, orc, n, t, tiles, in_place):
    k = t * tiles
    say("validated bandwidth regime", n, t, tiles, in_place)
    assert (n + 1) * 2 * k >= 320 << 20
    case = synth.ValidatedCase("vb", 95 + n, n, k, t, flag=0x9E3779B9, stale_frac=0.1)
    xs, fl = case.payloads(), case.flags()
    # A tile that never validates leaves out untouched: prefilled with
    # 0xFFFF, or input 1 when the call runs in place.
    start = xs[1].copy() if in_place else None
    want_out, want_ok = orc.reduce_validated(xs, fl, t, case.flag, out=start)
    assert 0 < int(want_ok.sum()) < tiles
    if not in_place:
        got_out, got_at = gpu_validated(B, D, xs, fl, t, case.flag, max_attempts=3)
    else:
        ins = [D.up(x) for x in xs]
        dev_fl = [torch.from_numpy(f.view(np.int32)).to("cuda:0") for f in fl]
        at = torch.full((tiles,), -1, dtype=torch.int32, device="cuda:0")
        B.pc_reduce_validated(ins, dev_fl, ins[1], k, t, case.flag, 3, at)
        got_out, got_at = D.down(ins[1], np.uint16), D.down(at, np.uint32)
    assert np.array_equal(got_at, want_ok)              # static inputs: attempt 1 or never
    assert np.array_equal(got_out, want_out)


@pytest.mark.parametrize("n,tiles", [(4, 5883), (8, 3835)])
@pytest.mark.parametrize("layout", ["congruent", "skewed"])
def test_reduce_validated_staged_rank_layouts(B, D, orc, n, tiles, layout):
    """At 8192 elements per flag with four or more ranks the bandwidth regime
    folds on the LDS-staged pipeline, on the diagonal when every rank
    buffer's base agrees with rank 0's modulo 32 KiB and plainly otherwise.
    The rank buffers are carved from one allocation at a stride that is a
    multiple of 32 KiB (congruent) or 4 KiB more (skewed).  A tenth of the
    tiles carry a stale flag on some rank and go through the retries.  On
    256 CUs the tile counts give most workgroups 23 (n = 4) or 15 (n = 8)
    tiles, so batches of 8, 4, 2 and 1 tiles all run."""
    t = 8192
    k = t * tiles
    assert (n + 1) * 2 * k >= 320 << 20
    stride = -(-2 * k // 32768) * 32768 // 2 + (2048 if layout == "skewed" else 0)   # elements
    say("validated staged layouts", n, tiles, layout)
    base = torch.empty(stride * n, dtype=torch.int16, device="cuda:0")
    views = [base[r * stride:r * stride + k] for r in range(n)]
    congruent = all((v.data_ptr() - views[0].data_ptr()) % 32768 == 0 for v in views)
    assert congruent == (layout == "congruent")
    case = synth.ValidatedCase("vs", 97 + n, n, k, t, flag=0x7FFFFFFF, stale_frac=0.1)
    xs, fl = case.payloads(), case.flags()
    for v, x in zip(views, xs):
        v.copy_(torch.from_numpy(x.view(np.int16)).to("cuda:0"))
    want_out, want_ok = orc.reduce_validated(xs, fl, t, case.flag)
    assert 0 < int(want_ok.sum()) < tiles
    dev_fl = [torch.from_numpy(f.view(np.int32)).to("cuda:0") for f in fl]
    out = D.filled(k, 0xFFFF)
    at = torch.full((tiles,), -1, dtype=torch.int32, device="cuda:0")
    B.pc_reduce_validated(views, dev_fl, out, k, t, case.flag, 2, at)
    assert np.array_equal(D.down(at, np.uint32), want_ok)
    assert np.array_equal(D.down(out, np.uint16), want_out)
    del base, views, out
    torch.cuda.empty_cache()


# ---- graph capture and concurrent streams ------------------------------------------------

def test_graph_replays_match_oracle(B, D, orc):
    """Calls captured once in a HIP graph and replayed several times, with the
    inputs rewritten eagerly between replays: every replay must equal the
    oracle on the inputs it saw (the library records only kernel launches)."""
    n, k = 8, 8 * 4096
    lines_k = 4096
    ins = [torch.empty(k, dtype=torch.int16, device="cuda:0") for _ in range(n)]
    red = torch.empty(k, dtype=torch.int16, device="cuda:0")
    outs = [torch.empty(k, dtype=torch.int16, device="cuda:0") for _ in range(n)]
    lines = [torch.empty(lines_k // 2, dtype=torch.int64, device="cuda:0") for _ in range(n)]
    ll_out = torch.empty(lines_k, dtype=torch.int16, device="cuda:0")
    ll_bm = torch.empty(lines_k // 128, dtype=torch.int64, device="cuda:0")
    louts = [torch.empty(k, dtype=torch.int16, device="cuda:0") for _ in range(n)]
    ws = linked_workspace(B, n, k)
    for t in ins:
        t.zero_()
    B.pc_twoshot_linked(ins, louts, k, ws)       # one eager call before capture
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            B.pc_reduce(ins, red, k)
            B.pc_twoshot_fused(ins, outs, k)
            for r in range(n):
                B.pc_pack_ll(ins[r], lines[r], lines_k, 9)
            B.pc_consume_ll(lines, ll_out, lines_k, 9, ll_bm)
            B.pc_twoshot_linked(ins, louts, k, ws)   # twice: the epoch advances
            B.pc_twoshot_linked(ins, louts, k, ws)   # on the device, not the host
    torch.cuda.synchronize()
    for rep in range(4):
        xs = [synth.normal_bf16(1200 + rep, 0, r, k) for r in range(n)]
        for t, x in zip(ins, xs):
            t.copy_(D.up(x))                      # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        want = orc.reduce(xs)
        assert np.array_equal(D.down(red, np.uint16), want), rep
        for o in outs:
            assert np.array_equal(D.down(o, np.uint16), want), rep
        wo, wb = orc.consume_ll([orc.pack_ll(x[:lines_k], 9) for x in xs], lines_k, 9)
        assert np.array_equal(D.down(ll_out, np.uint16), wo), rep
        assert np.array_equal(D.down(ll_bm, np.uint64), wb), rep
        for o in louts:
            assert np.array_equal(D.down(o, np.uint16), want), rep
        check_linked_workspace(B, D, ws, 1 + 2 * (rep + 1))
        for o in louts:
            o.fill_(-1)                           # the next replay must rewrite them


def test_graph_replays_bandwidth_regime(B, D, orc):
    """Every large-size path captured once and replayed with new inputs from
    torch's device RNG written eagerly between replays: 8 ranks x 48 MiB takes
    the staged oneshot reduce, the two-launch, flag-linked and fused twoshots
    with their large shapes, the persistent LL and speculative consumers, the
    two-pass sentinel
    consumer and the all-gather with non-temporal staging.  Outputs are
    checked at sampled positions against the oracle run on the sampled
    inputs; bitmaps, re-armed slots, attempts and the linked status word are
    checked whole."""
    n, k = 8, 24 << 20                        # 48 MiB per rank
    nl = k // 2
    dev = "cuda:0"
    gen = torch.Generator(device=dev)
    gen.manual_seed(1950)
    ins = [torch.empty(k, dtype=torch.int16, device=dev) for _ in range(n)]
    outs = [torch.empty(k, dtype=torch.int16, device=dev) for _ in range(n)]
    louts = [torch.empty(k, dtype=torch.int16, device=dev) for _ in range(n)]
    r_out = torch.empty(k, dtype=torch.int16, device=dev)
    ws = linked_workspace(B, n, k)
    lines = [torch.empty(nl, dtype=torch.int64, device=dev) for _ in range(n)]
    ll_out = torch.empty(k, dtype=torch.int16, device=dev)
    ll_bm = torch.empty(nl // 64, dtype=torch.int64, device=dev)
    slots = [torch.full((k,), -1, dtype=torch.int16, device=dev) for _ in range(n)]
    s_out = torch.empty(k, dtype=torch.int16, device=dev)
    s_bm = torch.empty(k // 512, dtype=torch.int64, device=dev)
    flags = [torch.full((k // 8192,), 3, dtype=torch.int32, device=dev) for _ in range(n)]
    v_out = torch.empty(k, dtype=torch.int16, device=dev)
    v_att = torch.empty(k // 8192, dtype=torch.int32, device=dev)
    sb = 2 * k                                 # all-gather shard bytes
    blocks = sb // 128
    recs = [torch.empty(blocks * 17, dtype=torch.int64, device=dev) for _ in range(n)]
    a_out = torch.empty(n * k, dtype=torch.int16, device=dev)
    a_bm = torch.empty(n * blocks // 64, dtype=torch.int64, device=dev)

    def rewrite():
        for t in ins:
            t.copy_(torch.randint(-32768, 32768, (k,), dtype=torch.int32, device=dev, generator=gen))
        for rc in recs:
            rc.copy_(torch.randint(-(1 << 62), 1 << 62, (blocks * 17,), dtype=torch.int64, device=dev,
                                   generator=gen))
            rc.view(blocks, 17)[:, 0] = 11

    rewrite()
    B.pc_twoshot_linked(ins, louts, k, ws)    # one eager call before capture
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            B.pc_reduce(ins, r_out, k)
            B.pc_twoshot(ins, outs, k)
            B.pc_twoshot_fused(ins, outs, k)
            B.pc_twoshot_linked(ins, louts, k, ws)
            for r in range(n):
                B.pc_pack_ll(ins[r], lines[r], k, 9)
            B.pc_consume_ll(lines, ll_out, k, 9, ll_bm)
            for r in range(n):
                B.pc_publish_sentinel(ins[r], slots[r], k)
            B.pc_consume_sentinel(slots, s_out, k, s_bm)
            B.pc_reduce_validated(ins, flags, v_out, k, 8192, 3, 2, v_att)
            B.pc_allgather_copy(recs, a_out, sb, 11, a_bm)
    torch.cuda.synchronize()
    idx_np = np.concatenate([np.arange(0, 4096), np.arange(k - 4096, k),
                             np.random.default_rng(1950).integers(0, k, 1 << 16)])
    idx = torch.from_numpy(idx_np).to(dev)
    blk = torch.from_numpy(np.random.default_rng(1951).integers(0, blocks, 4096)).to(dev)
    for rep in range(3):
        rewrite()
        ll_bm.zero_()
        s_bm.zero_()
        a_bm.zero_()
        g.replay()
        torch.cuda.synchronize()
        say("bandwidth-regime graph replay", rep)
        xs = [D.down(t[idx], np.uint16) for t in ins]
        want = orc.reduce(xs)
        for t in outs + louts + [r_out, ll_out, v_out]:
            assert np.array_equal(D.down(t[idx], np.uint16), want), rep
        assert np.array_equal(D.down(s_out[idx], np.uint16),
                              orc.reduce([orc.publish_sentinel(x) for x in xs])), rep
        assert bool((ll_bm == -1).all()) and bool((s_bm == -1).all()) and bool((a_bm == -1).all())
        assert all(bool((t == -1).all()) for t in slots)
        assert bool((v_att == 1).all())
        assert int(ws[B.PC_LINKED_STATUS_WORD]) == 0
        for r in range(n):
            got = a_out.view(n, blocks, 64)[r][blk]
            src = recs[r].view(blocks, 17)[blk][:, 1:].contiguous().view(torch.int16)
            assert torch.equal(got, src.view(-1, 64)), (rep, r)
    del ins, outs, louts, lines, slots, recs, a_out
    torch.cuda.empty_cache()


def test_graph_replays_of_the_other_calls(B, D, orc):
    """Copy, two-launch twoshot, all-gather, sentinel publish + consume and the
    speculative reduce captured once and replayed with new inputs written
    eagerly between replays; every replay must equal the oracle."""
    n, k = 8, 8 * 4096
    ins = [torch.empty(k, dtype=torch.int16, device="cuda:0") for _ in range(n)]
    cp = torch.empty(k, dtype=torch.int16, device="cuda:0")
    outs = [torch.empty(k, dtype=torch.int16, device="cuda:0") for _ in range(n)]
    slots = [torch.empty(k, dtype=torch.int16, device="cuda:0") for _ in range(n)]
    s_out = torch.empty(k, dtype=torch.int16, device="cuda:0")
    s_bm = torch.empty(k // 512, dtype=torch.int64, device="cuda:0")
    flags = [torch.full((k // 8192,), 3, dtype=torch.int32, device="cuda:0") for _ in range(n)]
    v_out = torch.empty(k, dtype=torch.int16, device="cuda:0")
    v_att = torch.empty(k // 8192, dtype=torch.int32, device="cuda:0")
    ag = synth.GatherCase("graph", 1910, n, 8192 * 2)
    rec_dev = [torch.empty(ag.blocks * 136, dtype=torch.uint8, device="cuda:0") for _ in range(n)]
    a_out = torch.empty(n * ag.shard_bytes // 2, dtype=torch.int16, device="cuda:0")
    a_bm = torch.empty(n * ag.blocks // 64, dtype=torch.int64, device="cuda:0")
    for t in ins + rec_dev:
        t.zero_()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            B.pc_copy(cp, ins[3], 2 * k)
            B.pc_twoshot(ins, outs, k)
            B.pc_allgather_copy(rec_dev, a_out, ag.shard_bytes, ag.seq, a_bm)
            for r in range(n):
                B.pc_publish_sentinel(ins[r], slots[r], k)
            B.pc_consume_sentinel(slots, s_out, k, s_bm)
            B.pc_reduce_validated(ins, flags, v_out, k, 8192, 3, 2, v_att)
    torch.cuda.synchronize()
    for rep in range(3):
        xs = [synth.normal_bf16(1911 + rep, 0, r, k) for r in range(n)]
        for t, x in zip(ins, xs):
            t.copy_(D.up(x))
        recs, _ = synth.GatherCase("graph", 1920 + rep, n, 8192 * 2).records()
        for t, rc in zip(rec_dev, recs):
            t.copy_(D.up(rc))
        a_out.fill_(-1)            # blocks that are not ready keep what is there: 0xFFFF, as in the oracle
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        want = orc.reduce(xs)
        assert np.array_equal(D.down(cp, np.uint16), xs[3]), rep
        assert all(np.array_equal(D.down(o, np.uint16), want) for o in outs), rep
        wo, wb = orc.allgather_copy(recs, ag.shard_bytes, ag.seq)
        assert np.array_equal(D.down(a_out, np.uint16), wo) and np.array_equal(D.down(a_bm, np.uint64), wb), rep
        assert np.array_equal(D.down(s_out, np.uint16), orc.reduce([orc.publish_sentinel(x) for x in xs])), rep
        assert np.all(D.down(s_bm, np.uint64) == np.uint64(0xFFFFFFFFFFFFFFFF)), rep
        assert all(np.all(D.down(sl, np.uint16) == 0xFFFF) for sl in slots), rep   # re-armed
        assert np.array_equal(D.down(v_out, np.uint16), want) and np.all(D.down(v_att, np.uint32) == 1), rep


def test_two_streams_disjoint_buffers(B, D, orc):
    n, k = 4, 8 * 65536
    xa = [synth.uniform_bf16(1300, 0, r, k) for r in range(n)]
    xb = [synth.uniform_bf16(1301, 0, r, k) for r in range(n)]
    ia, ib = [D.up(x) for x in xa], [D.up(x) for x in xb]
    oa = D.filled(k, 0xFFFF)
    ob = [D.filled(k, 0xFFFF) for _ in range(n)]
    sa, sb = torch.cuda.Stream(), torch.cuda.Stream()
    torch.cuda.synchronize()
    for _ in range(20):
        B.pc_reduce(ia, oa, k, stream=sa)
        B.pc_twoshot_fused(ib, ob, k, stream=sb)
    torch.cuda.synchronize()
    assert np.array_equal(D.down(oa, np.uint16), orc.reduce(xa))
    want = orc.reduce(xb)
    assert all(np.array_equal(D.down(o, np.uint16), want) for o in ob)


def test_twoshot_linked_next_to_a_persistent_kernel(B, D, orc):
    """The linked twoshot launched while a bandwidth-regime reduce on another
    stream holds the CUs: some of its workgroups start late, others wait on
    flags meanwhile (bounded).  Results stay exact and no wait is abandoned."""
    n, k = 8, 8 * 65536
    big_k = 8 << 20                                   # 16 MiB per rank: persistent regime
    g = torch.Generator(device="cuda:0")
    g.manual_seed(77)
    big = [torch.randint(-30000, 30000, (big_k,), dtype=torch.int16, device="cuda:0", generator=g)
           for _ in range(n)]
    big_out = torch.empty(big_k, dtype=torch.int16, device="cuda:0")
    xs = [synth.normal_bf16(1700, 0, r, k) for r in range(n)]
    ins = [D.up(x) for x in xs]
    outs = [D.filled(k, 0xFFFF) for _ in range(n)]
    ws = linked_workspace(B, n, k)
    sa, sb = torch.cuda.Stream(), torch.cuda.Stream()
    torch.cuda.synchronize()
    for _ in range(5):
        B.pc_reduce(big, big_out, big_k, stream=sa)
        B.pc_twoshot_linked(ins, outs, k, ws, stream=sb)
    torch.cuda.synchronize()
    want = orc.reduce(xs)
    for o in outs:
        assert np.array_equal(D.down(o, np.uint16), want)
    check_linked_workspace(B, D, ws, 5)
    idx = torch.arange(0, big_k, 4099, device="cuda:0")
    assert np.array_equal(D.down(big_out[idx], np.uint16),
                          orc.reduce([D.down(t[idx], np.uint16) for t in big]))


def test_five_calls_on_five_streams(B, D, orc):
    """Copy, LL consume, all-gather, speculative reduce and linked twoshot,
    each on its own stream with its own buffers, launched together ten times:
    the library keeps no shared state, so every result must be exact."""
    n = 8
    # copy
    csrc = np.random.default_rng(90).integers(0, 256, 3 << 20, dtype=np.uint8)
    c_in, c_out = D.up(csrc), torch.zeros(csrc.size, dtype=torch.uint8, device="cuda:0")
    # LL consume (all current)
    lk = 8 * 65536
    lx = [synth.uniform_bf16(1900, 0, r, lk) for r in range(n)]
    lines = [D.up(orc.pack_ll(x, 7)) for x in lx]
    l_out = D.filled(lk, 0xFFFF)
    l_bm = torch.empty(lk // 128, dtype=torch.int64, device="cuda:0")
    # all-gather
    ag = synth.GatherCase("streams", 1901, n, 8192 * 16, stale_frac=0.1)
    recs, _ = ag.records()
    shards = [D.up(r) for r in recs]
    a_out = D.filled(n * ag.shard_bytes // 2, 0xFFFF)
    a_bm = torch.empty(n * ag.blocks // 64, dtype=torch.int64, device="cuda:0")
    # speculative reduce (all flags current)
    vk = 8192 * 32
    vx = [synth.uniform_bf16(1902, 0, r, vk) for r in range(n)]
    v_in = [D.up(x) for x in vx]
    v_flags = [torch.full((vk // 8192,), 11, dtype=torch.int32, device="cuda:0") for _ in range(n)]
    v_out = D.filled(vk, 0xFFFF)
    v_att = torch.empty(vk // 8192, dtype=torch.int32, device="cuda:0")
    # linked twoshot
    tk = 8 * 8 * 4096
    tx = [synth.normal_bf16(1903, 0, r, tk) for r in range(n)]
    t_in = [D.up(x) for x in tx]
    t_out = [D.filled(tk, 0xFFFF) for _ in range(n)]
    ws = linked_workspace(B, n, tk)
    streams = [torch.cuda.Stream() for _ in range(5)]
    torch.cuda.synchronize()
    for _ in range(10):
        B.pc_copy(c_out, c_in, csrc.size, stream=streams[0])
        B.pc_consume_ll(lines, l_out, lk, 7, l_bm, stream=streams[1])
        B.pc_allgather_copy(shards, a_out, ag.shard_bytes, ag.seq, a_bm, stream=streams[2])
        B.pc_reduce_validated(v_in, v_flags, v_out, vk, 8192, 11, 4, v_att, stream=streams[3])
        B.pc_twoshot_linked(t_in, t_out, tk, ws, stream=streams[4])
    torch.cuda.synchronize()
    assert np.array_equal(D.down(c_out, np.uint8), csrc)
    wo, wb = orc.consume_ll([orc.pack_ll(x, 7) for x in lx], lk, 7)
    assert np.array_equal(D.down(l_out, np.uint16), wo) and np.array_equal(D.down(l_bm, np.uint64), wb)
    wo, wb = orc.allgather_copy(recs, ag.shard_bytes, ag.seq)
    assert np.array_equal(D.down(a_out, np.uint16), wo) and np.array_equal(D.down(a_bm, np.uint64), wb)
    assert np.array_equal(D.down(v_out, np.uint16), orc.reduce(vx))
    assert np.all(D.down(v_att, np.uint32) == 1)
    want = orc.reduce(tx)
    assert all(np.array_equal(D.down(o, np.uint16), want) for o in t_out)
    check_linked_workspace(B, D, ws, 10)


def test_binding_rejects_bad_tensors_before_launch(B, D):
    k = 4096
    x = D.up(synth.uniform_bf16(1310, 0, 0, k))
    out = D.filled(k, 0xFFFF)
    wide = torch.zeros(2 * k, dtype=torch.int16, device="cuda")
    with pytest.raises(ValueError, match="contiguous"):
        B.pc_reduce([wide[::2], x], out, k)
    with pytest.raises(ValueError, match="bytes"):
        B.pc_reduce([x, x], out[: k // 2], k)
    with pytest.raises(ValueError, match="GPU"):
        B.pc_reduce([x, x.cpu()], out, k)
    torch.cuda.synchronize()
    assert np.array_equal(D.down(out, np.uint16), np.full(k, 0xFFFF, np.uint16))
