#!/usr/bin/env python3
"""Benchmark of the MI355X collective datapath (one GPU).

Headline: effective HBM GB/s of the bandwidth-regime oneshot reduce (8 ranks
x 64 MiB bf16, fp32 accumulation in rank order 0..7, bf16 output) with the
inputs resident in HBM, as a fraction of the 8 TB/s HBM peak; beside it the
per-call latency of every datapath call on the decode-shaped workloads and a
latency sweep from 8 KiB to 1 MiB per rank.  Every timed workload is checked
bit for bit against the CPU oracle after timing, and the oracle itself is
timed on the host cores on the headline workload.

Timing:
  * kernel time per launch: HIP events (torch.cuda.Event, recorded on the
    stream the library launches on) around `--steps` back-to-back calls;
  * per-call time in a graph: 128 calls captured in one HIP graph, replayed
    once to warm up, then 8 replays timed with events, divided by 1024;
  * empty-kernel floor: the same two measurements of an empty kernel.

Prints one JSON line on stdout; progress goes to stderr.
"""
from __future__ import annotations

import argparse
import json
import os
import platform
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

HBM_PEAK_GBS = 8000.0

# HBM bytes per launch of the headline kernel from two rocprofv3 counter runs
# (FETCH_SIZE and WRITE_SIZE, each scaled by what it reads for a plain 256 MiB
# copy); profiles/k_reduce_staged_8x64MiB_hbm_counters.md has the commands and
# values.  Reported only while the kernel sources hash to what was profiled.
TRAFFIC = {"bytes": 604560037,
           "sources": ("collective_datapath_amd/csrc/pc_reduce.hip",
                       "collective_datapath_amd/csrc/pc_staged.hpp",
                       "collective_datapath_amd/csrc/pc_device.hpp"),
           "sha256": "fd32a9183144f578c1aa34a98b2311eabbcb5a48e72479786575876a24bb0d2a"}
HEADLINE_KERNEL = "pcdp::k_reduce_staged<8, (pcdp::Out)0, true, true>"
# rocprofv3 kernel-trace statistics of the same kernel over the 1,100
# dispatches of the warm leg that `value` times, and over every dispatch of
# the profiled run (profiles/k_reduce_staged_8x64MiB_trace.md), reported under
# the same source-hash condition as TRAFFIC.
KERNEL_TRACE = {"dispatches": 1100, "leg": "warm", "median_us": 87.849, "mean_us": 88.156,
                "all_dispatches": 4509, "all_median_us": 89.228,
                "profile": "profiles/k_reduce_staged_8x64MiB_trace.md"}
METRIC = "N-way reduce effective HBM GB/s (% of peak) + µs latency at 8 KB–1 MB, 1 GPU"


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200, help="timed calls of the headline workload")
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--only", default="all",
                    choices=["all", "headline", "c1", "c1v", "c2", "c2s", "c3", "c5", "atom_copy", "hbm", "sweep",
                             "sweep_cold", "copy"],
                    help="run one part only (profiling); 'copy' times a plain device copy")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-parity", action="store_true")
    return ap.parse_args()


class Dev:
    """Device plumbing: uploads and timing."""

    def __init__(self):
        import torch
        self.torch = torch
        self.dev = torch.device("cuda:0")

    def up(self, a):
        a = np.ascontiguousarray(a)
        v = {np.dtype(np.uint16): np.int16, np.dtype(np.uint64): np.int64,
             np.dtype(np.uint8): np.uint8}[a.dtype]
        return self.torch.from_numpy(a.view(v)).to(self.dev)

    def down(self, t, dt):
        self.torch.cuda.synchronize()
        return t.cpu().numpy().view(dt)

    def events_ms(self, fn, steps, warmup):
        """Average ms per call over `steps` back-to-back calls (events)."""
        torch = self.torch
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(steps):
            fn()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / steps

    def per_launch_us(self, fn, launches):
        """Each of `launches` calls between its own pair of events (after 3
        untimed calls): median, 10th and 90th percentile in us, and the count."""
        torch = self.torch
        for _ in range(3):
            fn()
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(launches)]
        torch.cuda.synchronize()
        for a, b in evs:
            a.record()
            fn()
            b.record()
        torch.cuda.synchronize()
        t = sorted(a.elapsed_time(b) * 1000.0 for a, b in evs)
        return (statistics.median(t), t[len(t) // 10], t[(9 * len(t)) // 10], len(t))

    def graph_us(self, fn, calls=128, replays=8):
        """Per-call us: `calls` calls in one graph, 1 warm replay, `replays` timed."""
        torch = self.torch
        fn()
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            with torch.cuda.graph(g, stream=s):
                for _ in range(calls):
                    fn()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(replays):
            g.replay()
        b.record()
        torch.cuda.synchronize()
        del g
        return a.elapsed_time(b) * 1000.0 / (calls * replays)


def graph_us_cold(d, fn, flush, calls=128, replays=8):
    """Like Dev.graph_us, but the caches are flushed before each timed replay
    (a 512 MiB read-only pass, outside the timed region, which leaves them
    holding clean unrelated lines), and the caller gives every captured call
    its own inputs."""
    torch = d.torch
    fn()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            for _ in range(calls):
                fn()
    torch.cuda.synchronize()
    g.replay()
    total = 0.0
    for _ in range(replays):
        flush.sum()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        g.replay()
        b.record()
        torch.cuda.synchronize()
        total += a.elapsed_time(b)
    del g
    return total * 1000.0 / (calls * replays)


def timing(d, fn, steps, warmup):
    """graph_us: per-call time inside a HIP graph (device-side latency);
    eager_us: back-to-back eager calls from Python, which for small payloads
    measures the host launch path rather than the GPU."""
    ms = d.events_ms(fn, steps, warmup)
    return {"graph_us": round(d.graph_us(fn), 3), "eager_us": round(ms * 1000.0, 3)}


def gbs(nbytes, us):
    return nbytes / (us * 1e-6) / 1e9


# ---------------------------------------------------------------------------


def run_headline(d, B, synth, args, out):
    """The headline call three ways, all on the same stream:
      * warm: `--steps` back-to-back calls on one input set (the line's value);
      * rotated: `--steps` back-to-back calls cycling three distinct input
        sets of 8 x 64 MiB, so no call finds its inputs in the 256 MiB
        last-level cache (the previous two calls moved 1.1 GiB through it);
        a second rotation also cycles six outputs (384 MiB), so that no call
        overwrites output lines the cache still holds from an earlier call;
      * per launch: 1,100 calls, each between its own pair of events; the
        median is the kernel-time statistic (plus the event overhead).
    Every output of every input set is checked bit for bit against the
    oracle, and the oracle is timed on the host cores on the same call."""
    import dataclasses
    torch = d.torch
    case = synth.C4_ONESHOT_64M
    log("generating", case.name)
    xs = case.inputs()
    # Input sets 1 and 2 hold the same values with the rank order rotated by
    # one and two places: distinct memory, and different fold results.
    sets = [[d.up(x) for x in xs]]
    for j in (1, 2):
        sets.append([sets[0][(r + j) % case.n].clone() for r in range(case.n)])
    host_sets = [[xs[(r + j) % case.n] for r in range(case.n)] for j in range(3)]
    res = [torch.full((case.k,), -1, dtype=torch.int16, device=d.dev) for _ in range(3)]
    nbytes = case.bytes_moved()
    fn = lambda: B.pc_reduce(sets[0], res[0], case.k)  # noqa: E731
    log("timing headline:", args.steps, "calls after", args.warmup, "warm-up")
    ms = d.events_ms(fn, args.steps, args.warmup)
    turn = [0]

    def rotated():
        j = turn[0] % 3
        turn[0] += 1
        B.pc_reduce(sets[j], res[j], case.k)
    ms_rot = d.events_ms(rotated, 3 * max(1, args.steps // 3), 3)
    res_more = [torch.full((case.k,), -1, dtype=torch.int16, device=d.dev) for _ in range(3)]
    outs6 = res + res_more

    def rotated_io():
        m = turn[0] % 6
        turn[0] += 1
        B.pc_reduce(sets[m % 3], outs6[m], case.k)
    turn[0] = 0
    ms_rot_io = d.events_ms(rotated_io, 6 * max(1, args.steps // 6), 6)
    torch.cuda.synchronize()
    for m in range(3):
        if not torch.equal(res_more[m], res[m]):
            raise SystemExit(f"headline: output {m + 3} of the six-output rotation differs from output {m}")
    del res_more, outs6
    med_us, p10_us, p90_us, count = d.per_launch_us(fn, 1100)
    g_us = d.graph_us(fn, calls=16, replays=4)
    ach = gbs(nbytes, ms * 1000.0)
    out["headline"] = {"workload": case.name, "bytes_per_call": nbytes,
                       "event_us_per_launch": round(ms * 1e3, 3), "gbs": round(ach, 1),
                       "rotated_inputs": {"sets": 3, "event_us_per_launch": round(ms_rot * 1e3, 3),
                                          "gbs": round(gbs(nbytes, ms_rot * 1e3), 1),
                                          "frac_of_hbm_peak": round(gbs(nbytes, ms_rot * 1e3) / HBM_PEAK_GBS, 4)},
                       "rotated_inputs_and_outputs": {
                           "sets": 3, "outputs": 6, "event_us_per_launch": round(ms_rot_io * 1e3, 3),
                           "gbs": round(gbs(nbytes, ms_rot_io * 1e3), 1),
                           "frac_of_hbm_peak": round(gbs(nbytes, ms_rot_io * 1e3) / HBM_PEAK_GBS, 4)},
                       "per_launch_events": {"launches": count, "median_us": round(med_us, 3),
                                             "p10_us": round(p10_us, 3), "p90_us": round(p90_us, 3),
                                             "gbs_at_median": round(gbs(nbytes, med_us), 1)},
                       "graph_us": round(g_us, 3)}
    got = [d.down(r, np.uint16) for r in res]
    if not args.no_parity or not args.no_cpu_baseline:
        import oracle
        threads = max(1, min(16, os.cpu_count() or 1))

        def median_of(fn_cpu, runs, seconds):
            fn_cpu()                                   # warm-up, not counted
            times = []
            t_end = time.perf_counter() + seconds
            while len(times) < runs or (time.perf_counter() < t_end and len(times) < 200):
                t0 = time.perf_counter()
                fn_cpu()
                times.append(time.perf_counter() - t0)
            return statistics.median(times), len(times)
        wants = [oracle.reduce(h, threads=threads) for h in host_sets]
        med, nrun = median_of(lambda: oracle.reduce(xs, threads=threads), 5, 8.0)
        med1, nrun1 = median_of(lambda: oracle.reduce(xs, threads=1), 5, 0.0)
        out["cpu_baseline"] = {
            "value": round(nbytes / med / 1e9, 3), "unit": "GB/s", "cores": threads, "kind": "oracle",
            "sample": f"the full headline call (8 x 64 MiB in, 64 MiB out): median of {nrun} runs after "
                      f"1 warm-up on {threads} threads split by element range; single-threaded, median of "
                      f"{nrun1} full runs after 1 warm-up: {nbytes / med1 / 1e9:.3f} GB/s",
            "ms": round(med * 1e3, 2),
            "single_thread": {"value": round(nbytes / med1 / 1e9, 3), "unit": "GB/s", "cores": 1,
                              "ms": round(med1 * 1e3, 1), "runs": nrun1},
            "cpu_model": cpu_model(), "os_cpu_count": os.cpu_count()}
        if not args.no_parity:
            ok = all(bool(np.array_equal(g, w)) for g, w in zip(got, wants))
            out.setdefault("parity", {})["headline"] = ok
            log("headline parity (3 input sets)", ok)
    del sets, res
    torch.cuda.empty_cache()
    return ms, ach


def kernel_sources_sha256():
    import hashlib
    h = hashlib.sha256()
    for rel in TRAFFIC["sources"]:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic():
    if TRAFFIC["bytes"] is None:
        return None
    return TRAFFIC["bytes"] if kernel_sources_sha256() == TRAFFIC["sha256"] else None


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor()


def run_c1(d, B, synth, oracle, args, out):
    case = synth.C1_ONESHOT_8K
    xs = case.inputs()
    ins = [d.up(x) for x in xs]
    res = d.torch.full((case.k,), -1, dtype=d.torch.int16, device=d.dev)
    t = timing(d, lambda: B.pc_reduce(ins, res, case.k), 2000, 100)
    t.update(workload=case.name, bytes_per_call=case.bytes_moved(),
             gbs_cache_resident=round(gbs(case.bytes_moved(), t["graph_us"]), 1))
    out["configs"]["oneshot_8k"] = t
    if oracle is not None:
        out["parity"]["oneshot_8k"] = bool(np.array_equal(d.down(res, np.uint16), oracle.reduce(xs)))


def run_c2(d, B, synth, oracle, args, out):
    torch = d.torch
    case = synth.C2_LL_128K
    pays, stales, masks = case.payloads(), case.stale_payloads(), case.stale_masks()
    src = [d.up(x) for x in pays]
    old_src = [d.up(s) for s in stales]
    cur = [torch.empty(case.lines, dtype=torch.int64, device=d.dev) for _ in range(case.n)]
    old = [torch.empty(case.lines, dtype=torch.int64, device=d.dev) for _ in range(case.n)]
    for r in range(case.n):
        B.pc_pack_ll(src[r], cur[r], case.k, case.seq)
        B.pc_pack_ll(old_src[r], old[r], case.k, case.stale_seq)
    staged = [torch.where(torch.from_numpy(m).to(d.dev), o, c) for m, o, c in zip(masks, old, cur)]
    res = torch.full((case.k,), -1, dtype=torch.int16, device=d.dev)
    bm = torch.empty(case.k // 128, dtype=torch.int64, device=d.dev)
    tc = timing(d, lambda: B.pc_consume_ll(staged, res, case.k, case.seq, bm), 2000, 100)
    tp = timing(d, lambda: B.pc_pack_ll(src[0], cur[0], case.k, case.seq), 2000, 100)
    bits = d.down(bm, np.uint64)
    ready = int(np.unpackbits(bits.view(np.uint8)).sum())
    cbytes = case.n * case.lines * 8 + 4 * ready + case.lines // 8
    tc.update(workload=case.name, ready_lines=ready, bytes_per_call=cbytes,
              gbs_cache_resident=round(gbs(cbytes, tc["graph_us"]), 1))
    tp.update(workload="LL pack of one rank, 128 KiB -> 256 KiB", bytes_per_call=6 * case.k,
              gbs_cache_resident=round(gbs(6 * case.k, tp["graph_us"]), 1))
    out["configs"]["ll_consume_128k"] = tc
    out["configs"]["ll_pack_128k"] = tp
    if oracle is not None:
        for r in range(case.n):
            B.pc_pack_ll(src[r], cur[r], case.k, case.seq)
        host = [np.where(m, oracle.pack_ll(s, case.stale_seq), oracle.pack_ll(x, case.seq))
                for x, s, m in zip(pays, stales, masks)]
        ok_lines = all(np.array_equal(d.down(a, np.uint64), b) for a, b in zip(staged, host))
        res.fill_(-1)
        B.pc_consume_ll(staged, res, case.k, case.seq, bm)
        wo, wb = oracle.consume_ll(host, case.k, case.seq)
        out["parity"]["ll_128k"] = bool(ok_lines and np.array_equal(d.down(res, np.uint16), wo)
                                        and np.array_equal(d.down(bm, np.uint64), wb))


def run_c2s(d, B, synth, oracle, args, out):
    """Sentinel readiness next to LL at the same shape (8 ranks x 128 KiB).

    Consuming re-arms sentinel slots, so a call cycle is timed: every rank
    publishes (or packs), then the consumer consumes.  Parity is checked on
    the workload with unarrived and torn packs and sentinel collisions."""
    torch = d.torch
    case = synth.C2S_SENTINEL_128K
    xs = case.payloads()
    src = [d.up(x) for x in xs]
    slots = [torch.empty(case.k, dtype=torch.int16, device=d.dev) for _ in xs]
    lines = [torch.empty(case.k // 2, dtype=torch.int64, device=d.dev) for _ in xs]
    res = torch.empty(case.k, dtype=torch.int16, device=d.dev)
    bm_s = torch.empty(case.k // 512, dtype=torch.int64, device=d.dev)
    bm_l = torch.empty(case.k // 128, dtype=torch.int64, device=d.dev)

    def sentinel_cycle():
        for r in range(case.n):
            B.pc_publish_sentinel(src[r], slots[r], case.k)
        B.pc_consume_sentinel(slots, res, case.k, bm_s)

    def ll_cycle():
        for r in range(case.n):
            B.pc_pack_ll(src[r], lines[r], case.k, 7)
        B.pc_consume_ll(lines, res, case.k, 7, bm_l)

    ts = timing(d, sentinel_cycle, 300, 20)
    tl = timing(d, ll_cycle, 300, 20)
    k = case.k
    ts.update(workload="8 x publish + consume, all arrived, 8 ranks x 128 KiB",
              staged_bytes_per_rank=2 * k, consume_bytes=case.n * 2 * k + 2 * k + case.n * 2 * k + k // 64)
    tl.update(workload="8 x pack + consume, all current, 8 ranks x 128 KiB",
              staged_bytes_per_rank=4 * k, consume_bytes=case.n * 4 * k + 2 * k + k // 16)
    out["configs"]["sentinel_cycle_128k"] = ts
    out["configs"]["ll_cycle_128k"] = tl
    if oracle is not None:
        ms = case.masks()
        host = [synth.unarrive(oracle.publish_sentinel(x), m, t) for x, (m, t) in zip(xs, ms)]
        for r in range(case.n):
            B.pc_publish_sentinel(src[r], slots[r], case.k)
        dev = [synth.unarrive(d.down(sl, np.uint16), m, t) for sl, (m, t) in zip(slots, ms)]
        ok = all(np.array_equal(a, b) for a, b in zip(dev, host))
        staged = [d.up(x) for x in dev]
        res.fill_(-1)
        B.pc_consume_sentinel(staged, res, case.k, bm_s)
        wo, wb, wsl = oracle.consume_sentinel(host, case.k)
        ok = ok and np.array_equal(d.down(res, np.uint16), wo) and np.array_equal(d.down(bm_s, np.uint64), wb)
        ok = ok and all(np.array_equal(d.down(a, np.uint16), b) for a, b in zip(staged, wsl))
        out["parity"]["sentinel_128k"] = bool(ok)


def run_c1v(d, B, synth, oracle, args, out):
    """Speculative reduce at decode size: validation passes on the first
    attempt; then the cost of one retry, from a flag that never validates."""
    torch = d.torch
    case = synth.C1V_VALIDATED_8K
    xs, fl = case.payloads(), case.flags()
    ins = [d.up(x) for x in xs]
    flags = [torch.from_numpy(f.view(np.int32)).to(d.dev) for f in fl]
    res = torch.full((case.k,), -1, dtype=torch.int16, device=d.dev)
    at = torch.empty(case.tiles, dtype=torch.int32, device=d.dev)
    t = timing(d, lambda: B.pc_reduce_validated(ins, flags, res, case.k, case.elems_per_flag,
                                                case.flag, 1, at), 2000, 100)
    t.update(workload=case.name, bytes_per_call=(case.n + 1) * 2 * case.k + 4 * case.n * case.tiles)
    out["configs"]["validated_8k"] = t
    if oracle is not None:
        wo, wok = oracle.reduce_validated(xs, fl, case.elems_per_flag, case.flag)
        out["parity"]["validated_8k"] = bool(np.array_equal(d.down(res, np.uint16), wo) and
                                             np.array_equal(d.down(at, np.uint32), wok))
    stale = [f.clone() for f in flags]
    stale[0].sub_(1)
    t1 = d.graph_us(lambda: B.pc_reduce_validated(ins, stale, res, case.k, case.elems_per_flag,
                                                  case.flag, 1, at))
    t9 = d.graph_us(lambda: B.pc_reduce_validated(ins, stale, res, case.k, case.elems_per_flag,
                                                  case.flag, 9, at))
    out["configs"]["validated_8k_retry"] = {
        "workload": "same call with one stale flag: 1 vs 9 attempts",
        "graph_us_1_attempt": round(t1, 3), "graph_us_9_attempts": round(t9, 3),
        "us_per_retry": round((t9 - t1) / 8, 3)}


def run_c3(d, B, synth, oracle, args, out):
    case = synth.C3_TWOSHOT_1M
    xs = case.inputs()
    ins = [d.up(x) for x in xs]
    want = oracle.twoshot(xs) if oracle is not None else None
    onev = None
    if oracle is not None:
        one = d.torch.full((case.k,), -1, dtype=d.torch.int16, device=d.dev)
        B.pc_reduce(ins, one, case.k)
        onev = d.down(one, np.uint16)
    # Two launches (slice reduce, then copy-out), the single-launch form, and
    # the single launch whose phases are linked per tile by epoch flags.
    ws = d.torch.zeros(B.pc_twoshot_linked_workspace_bytes(case.n, case.k) // 8,
                       dtype=d.torch.int64, device=d.dev)
    linked = lambda i, o, k: B.pc_twoshot_linked(i, o, k, ws)  # noqa: E731
    for name, fn, nbytes in (("twoshot_1m", B.pc_twoshot, 2 * case.k * (2 * case.n + 1)),
                             ("twoshot_fused_1m", B.pc_twoshot_fused, 2 * case.k * 2 * case.n),
                             ("twoshot_linked_1m", linked, 2 * case.k * (2 * case.n + 1))):
        outs = [d.torch.full((case.k,), -1, dtype=d.torch.int16, device=d.dev) for _ in xs]
        t = timing(d, lambda: fn(ins, outs, case.k), 1000, 50)
        t.update(workload=case.name, bytes_per_call=nbytes,
                 gbs_cache_resident=round(gbs(nbytes, t["graph_us"]), 1))
        out["configs"][name] = t
        if oracle is not None:
            out["parity"][name] = bool(all(np.array_equal(d.down(o, np.uint16), w) and
                                           np.array_equal(w, onev) for o, w in zip(outs, want)))
    out["configs"]["twoshot_linked_1m"]["waits_abandoned"] = int(ws[B.PC_LINKED_STATUS_WORD])


def run_hbm_regime(d, B, synth, oracle, args, out):
    """Every other call at 8 ranks x 64 MiB (HBM-bound; event-timed back to
    back).  Outputs are checked against the oracle at sampled positions, run
    on the sampled inputs; ready bitmaps of all-current data must be full."""
    torch = d.torch
    n, k = 8, 32 << 20
    g = torch.Generator(device=d.dev)
    g.manual_seed(64)

    def rnd(count, dtype=torch.int16):
        return torch.randint(-32768, 32768, (count,), dtype=torch.int32, device=d.dev,
                             generator=g).to(dtype)

    def ev_us(fn, reps=20):
        return d.events_ms(fn, reps, 3) * 1e3

    def isolated_us(setup, fn, reps):
        """Mean us of `fn` alone: `setup` runs untimed before each call."""
        total = 0.0
        for _ in range(reps):
            setup()
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            fn()
            b.record()
            torch.cuda.synchronize()
            total += a.elapsed_time(b) * 1000.0
        return total / reps

    idx_np = np.concatenate([np.arange(0, 4096), np.arange(k - 4096, k),
                             np.random.default_rng(64).integers(0, k, 1 << 14)])
    idx = torch.from_numpy(idx_np).to(d.dev)
    ins = [rnd(k) for _ in range(n)]
    xs = [d.down(t[idx], np.uint16) for t in ins]
    want = oracle.reduce(xs) if oracle is not None else None
    rows = {}

    def row(name, nbytes, us, ok):
        rows[name] = {"event_us_per_launch": round(us, 2), "bytes_per_call": nbytes,
                      "gbs": round(gbs(nbytes, us), 1), "frac_of_hbm_peak": round(gbs(nbytes, us) / HBM_PEAK_GBS, 4)}
        if oracle is not None:
            out["parity"]["hbm_" + name] = bool(ok)

    outs = [torch.empty(k, dtype=torch.int16, device=d.dev) for _ in range(n)]
    ws = torch.zeros(B.pc_twoshot_linked_workspace_bytes(n, k) // 8, dtype=torch.int64, device=d.dev)
    for name, fn, units in (("twoshot", lambda: B.pc_twoshot(ins, outs, k), 2 * n + 1),
                            ("twoshot_fused", lambda: B.pc_twoshot_fused(ins, outs, k), 2 * n),
                            ("twoshot_linked", lambda: B.pc_twoshot_linked(ins, outs, k, ws), 2 * n + 1)):
        for o in outs:
            o.fill_(-1)
        us = ev_us(fn)
        ok = want is not None and all(np.array_equal(d.down(o[idx], np.uint16), want) for o in outs)
        row(name, units * 2 * k, us, ok)
    del outs, ws
    # LL: one rank packed (timed), then all ranks' lines consumed, all current.
    lines = [torch.empty(k // 2, dtype=torch.int64, device=d.dev) for _ in range(n)]
    for r in range(n):
        B.pc_pack_ll(ins[r], lines[r], k, 7)
    us = ev_us(lambda: B.pc_pack_ll(ins[0], lines[0], k, 7))
    pairs = idx[idx % 2 == 0]
    line_idx = pairs // 2
    ok = oracle is not None and np.array_equal(
        d.down(lines[0][line_idx], np.uint64),
        oracle.pack_ll(np.stack([d.down(ins[0][pairs], np.uint16), d.down(ins[0][pairs + 1], np.uint16)], 1).reshape(-1), 7))
    row("pack_ll", 6 * k, us, ok)
    res = torch.full((k,), -1, dtype=torch.int16, device=d.dev)
    bm = torch.empty(k // 128, dtype=torch.int64, device=d.dev)
    us = ev_us(lambda: B.pc_consume_ll(lines, res, k, 7, bm))
    ok = want is not None and np.array_equal(d.down(res[idx], np.uint16), want) and \
        bool((bm == -1).all())
    row("consume_ll", n * 4 * k + 2 * k + k // 16, us, ok)
    del lines
    # Sentinel: publish (timed alone), then publish-and-consume cycles; the
    # consume time is the cycle minus its publishes.
    slots = [torch.empty(k, dtype=torch.int16, device=d.dev) for _ in range(n)]
    us = ev_us(lambda: B.pc_publish_sentinel(ins[0], slots[0], k))
    pub = [d.down(slots[0][idx], np.uint16)]
    ok = oracle is not None and np.array_equal(pub[0], oracle.publish_sentinel(xs[0]))
    row("publish_sentinel", 4 * k, us, ok)
    bms = torch.empty(k // 512, dtype=torch.int64, device=d.dev)

    def publish_all():
        for r in range(n):
            B.pc_publish_sentinel(ins[r], slots[r], k)

    def cycle():
        publish_all()
        B.pc_consume_sentinel(slots, res, k, bms)
    us_publish = ev_us(publish_all, 10)
    us_isolated = isolated_us(publish_all, lambda: B.pc_consume_sentinel(slots, res, k, bms), 10)
    us = ev_us(cycle, 10) - us_publish             # the cycle runs last: slots end re-armed
    ok = oracle is not None and np.array_equal(
        d.down(res[idx], np.uint16), oracle.reduce([oracle.publish_sentinel(x) for x in xs])) and \
        bool((bms == -1).all()) and bool((slots[n - 1][idx] == -1).all())
    sbytes = n * 2 * k + 2 * k + n * 2 * k + k // 64
    row("consume_sentinel", sbytes, us, ok)
    rows["consume_sentinel"]["timing"] = "publish-and-consume cycles minus publish-only runs"
    rows["consume_sentinel"]["isolated"] = {
        "timing": "slots published (untimed), then the consume alone between two events; mean of 10",
        "event_us_per_call": round(us_isolated, 2), "gbs": round(gbs(sbytes, us_isolated), 1),
        "frac_of_hbm_peak": round(gbs(sbytes, us_isolated) / HBM_PEAK_GBS, 4)}
    # Write-only reference on the same eight 64 MiB slots: torch's fill
    # kernel, back to back.  The re-arm pass of the consume (all packs
    # ready) writes exactly these bytes.
    us_fill = ev_us(lambda: [t.fill_(-1) for t in slots], 10)
    rows["write_only_reference"] = {
        "workload": "torch fill_ of 8 x 64 MiB (the bytes a full re-arm writes)",
        "event_us_per_launch": round(us_fill, 2), "bytes_per_call": n * 2 * k,
        "gbs": round(gbs(n * 2 * k, us_fill), 1), "frac_of_hbm_peak": round(gbs(n * 2 * k, us_fill) / HBM_PEAK_GBS, 4)}
    del slots
    # Speculative reduce, one flag per 8192 elements, all flags current.
    flags = [torch.full((k // 8192,), 5, dtype=torch.int32, device=d.dev) for _ in range(n)]
    att = torch.empty(k // 8192, dtype=torch.int32, device=d.dev)
    res.fill_(-1)
    us = ev_us(lambda: B.pc_reduce_validated(ins, flags, res, k, 8192, 5, 1, att))
    ok = want is not None and np.array_equal(d.down(res[idx], np.uint16), want) and bool((att == 1).all())
    row("reduce_validated", 9 * 2 * k + 4 * n * (k // 8192), us, ok)
    del flags, att, res
    # All-gather of 8 shards of 64 MiB payload, every record current.
    sb = 2 * k
    blocks = sb // 128
    recs = []
    for r in range(n):
        rec = torch.empty(blocks * 17, dtype=torch.int64, device=d.dev)
        rv = rec.view(blocks, 17)
        rv[:, 0] = 7
        rv[:, 1:] = rnd(blocks * 64).view(torch.int64).view(blocks, 16)
        recs.append(rec)
    agout = torch.empty(n * sb // 2, dtype=torch.int16, device=d.dev)
    agbm = torch.empty(n * blocks // 64, dtype=torch.int64, device=d.dev)
    us = ev_us(lambda: B.pc_allgather_copy(recs, agout, sb, 7, agbm))
    sample = torch.from_numpy(np.random.default_rng(65).integers(0, blocks, 256)).to(d.dev)
    ok = oracle is not None and bool((agbm == -1).all()) and all(
        torch.equal(agout.view(n, blocks, 64)[r][sample].view(torch.int64), recs[r].view(blocks, 17)[sample][:, 1:])
        for r in range(n))
    row("allgather_copy", n * blocks * 136 + n * sb + n * blocks // 8, us, ok)
    del recs, agout, agbm, ins
    out["hbm_regime"] = {"workload": "8 ranks x 64 MiB per rank (LL: 128 MiB of lines per rank)", **rows}
    torch.cuda.empty_cache()


def run_copy_atom(d, B, synth, oracle, args, out):
    """The Atom copy: 256 MiB (HBM-bound, event-timed) and 1 MiB (per call
    in a graph, cache-resident).  Parity: the destination equals the source."""
    torch = d.torch
    for name, nbytes in (("atom_copy_256m", 256 << 20), ("atom_copy_1m", 1 << 20)):
        g = torch.Generator(device=d.dev)
        g.manual_seed(nbytes % 1000003)
        src = torch.randint(0, 256, (nbytes,), dtype=torch.uint8, device=d.dev, generator=g)
        dst = torch.zeros_like(src)
        fn = lambda: B.pc_copy(dst, src, nbytes)  # noqa: E731
        if nbytes >= (64 << 20):
            ms = d.events_ms(fn, 50, 5)
            t = {"event_us_per_launch": round(ms * 1e3, 3), "bytes_per_call": 2 * nbytes,
                 "gbs": round(gbs(2 * nbytes, ms * 1e3), 1)}
        else:
            t = timing(d, fn, 1000, 50)
            t.update(bytes_per_call=2 * nbytes,
                     gbs_cache_resident=round(gbs(2 * nbytes, t["graph_us"]), 1))
        out["configs"][name] = t
        if oracle is not None:
            torch.cuda.synchronize()
            out["parity"][name] = bool(torch.equal(dst, src))
        del src, dst


def run_c5(d, B, synth, oracle, args, out):
    case = synth.C5_ALLGATHER_2M
    recs, masks = case.records()
    shards = [d.up(r) for r in recs]
    res = d.torch.full((case.n * case.shard_bytes // 2,), -1, dtype=d.torch.int16, device=d.dev)
    bm = d.torch.empty(case.n * case.blocks // 64, dtype=d.torch.int64, device=d.dev)
    t = timing(d, lambda: B.pc_allgather_copy(shards, res, case.shard_bytes, case.seq, bm), 1000, 50)
    ready = int(sum((~m).sum() for m in masks))
    nbytes = case.n * case.blocks * 136 + ready * 128 + case.n * case.blocks // 8
    t.update(workload=case.name, ready_blocks=ready, bytes_per_call=nbytes,
             gbs_cache_resident=round(gbs(nbytes, t["graph_us"]), 1))
    out["configs"]["allgather_2m"] = t
    if oracle is not None:
        wo, wb = oracle.allgather_copy(recs, case.shard_bytes, case.seq)
        out["parity"]["allgather_2m"] = bool(np.array_equal(d.down(res, np.uint16), wo) and
                                             np.array_equal(d.down(bm, np.uint64), wb))


def run_sweep(d, B, synth, oracle, args, out):
    rows = []
    for nbytes in synth.SWEEP_BYTES:
        k = nbytes // 2
        for kind, n in (("reduce", 4), ("reduce", 8), ("twoshot", 8), ("twoshot_fused", 8),
                        ("twoshot_linked", 8)):
            xs = [synth.uniform_bf16(20, 0, r, k) for r in range(n)]
            ins = [d.up(x) for x in xs]
            if kind == "reduce":
                res = d.torch.empty(k, dtype=d.torch.int16, device=d.dev)
                fn = lambda: B.pc_reduce(ins, res, k)  # noqa: E731
                moved = (n + 1) * nbytes
            elif kind == "twoshot":
                outs = [d.torch.empty(k, dtype=d.torch.int16, device=d.dev) for _ in range(n)]
                fn = lambda: B.pc_twoshot(ins, outs, k)  # noqa: E731
                moved = (2 * n + 1) * nbytes
            elif kind == "twoshot_fused":
                outs = [d.torch.empty(k, dtype=d.torch.int16, device=d.dev) for _ in range(n)]
                fn = lambda: B.pc_twoshot_fused(ins, outs, k)  # noqa: E731
                moved = 2 * n * nbytes
            else:
                outs = [d.torch.empty(k, dtype=d.torch.int16, device=d.dev) for _ in range(n)]
                ws = d.torch.zeros(B.pc_twoshot_linked_workspace_bytes(n, k) // 8,
                                   dtype=d.torch.int64, device=d.dev)
                fn = lambda: B.pc_twoshot_linked(ins, outs, k, ws)  # noqa: E731
                moved = (2 * n + 1) * nbytes
            t = timing(d, fn, 500, 50)
            row = {"call": kind, "n": n, "bytes_per_rank": nbytes, **t,
                   "gbs_cache_resident": round(gbs(moved, t["graph_us"]), 1)}
            if oracle is not None:
                want = oracle.reduce(xs)
                got = d.down(res if kind == "reduce" else outs[n - 1], np.uint16)
                row["parity"] = bool(np.array_equal(got, want))
            rows.append(row)
    out["latency_sweep"] = rows


def run_sweep_cold(d, B, synth, oracle, args, out):
    """Cold per-call latency: each of the 128 captured calls reads its own
    region of a 1 GiB arena and the caches are flushed (read-only) before
    each timed replay, so no call finds its inputs in the 256 MiB last-level
    cache (on the pages' systems, peers have just written the inputs)."""
    torch = d.torch
    flush = torch.zeros((512 << 20) // 4, dtype=torch.int32, device=d.dev)
    arena_elems = (1 << 30) // 2
    g = torch.Generator(device=d.dev)
    g.manual_seed(99)
    arena = torch.randint(-32768, 32768, (arena_elems,), dtype=torch.int32, device=d.dev,
                          generator=g).to(torch.int16)
    rows = []
    for nbytes in synth.SWEEP_BYTES:
        k = nbytes // 2
        for kind, n in (("reduce", 8), ("twoshot_fused", 8)):
            per_call = n * k
            calls = 128
            res = [torch.empty(k, dtype=torch.int16, device=d.dev) for _ in range(n)]
            ptr = [0]

            def fn():
                base = (ptr[0] * per_call) % (arena_elems - per_call)
                base -= base % 8
                ptr[0] += 1
                ins = [arena[base + r * k: base + (r + 1) * k] for r in range(n)]
                if kind == "reduce":
                    B.pc_reduce(ins, res[0], k)
                else:
                    B.pc_twoshot_fused(ins, res, k)
            us = graph_us_cold(d, fn, flush, calls=calls, replays=8)
            rows.append({"call": kind, "n": n, "bytes_per_rank": nbytes, "graph_us_cold": round(us, 3)})
    # Parity of one cold call against the oracle.
    if oracle is not None:
        k = 4096
        ins = [arena[(1 << 20) + r * k: (1 << 20) + (r + 1) * k] for r in range(8)]
        res0 = torch.empty(k, dtype=torch.int16, device=d.dev)
        B.pc_reduce(ins, res0, k)
        xs = [d.down(t, np.uint16) for t in ins]
        out["parity"]["sweep_cold"] = bool(np.array_equal(d.down(res0, np.uint16), oracle.reduce(xs)))
    out["latency_sweep_cold"] = rows
    del arena, flush


def run_floor(d, out):
    torch = d.torch
    fn = lambda: torch.cuda._sleep(0)  # noqa: E731
    out["empty_kernel_floor"] = timing(d, fn, 2000, 100)


def run_copy(d, out, steps):
    """Plain device-to-device copy of 256 MiB (calibration for HBM counters)."""
    torch = d.torch
    a = torch.empty(128 << 20, dtype=torch.int16, device=d.dev).fill_(1)
    b = torch.empty_like(a)
    ms = d.events_ms(lambda: b.copy_(a), steps, 5)
    out["copy_256m"] = {"event_us": round(ms * 1e3, 3), "bytes_per_call": 2 * (256 << 20),
                        "gbs": round(gbs(2 * (256 << 20), ms * 1e3), 1)}


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU's share of the datapath on one GPU; runs on several "
              "GPUs are not supported (use --gpus 1).", file=sys.stderr)
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    from collective_datapath_amd import binding as B
    from collective_datapath_amd import synth
    d = Dev()
    out = {"configs": {}, "parity": {}}
    oracle = None
    if not args.no_parity:
        import oracle as _oracle
        oracle = _oracle
    t0 = time.time()

    headline_ms = ach = None
    if args.only in ("all", "headline"):
        headline_ms, ach = run_headline(d, B, synth, args, out)
    if args.only == "copy":
        run_copy(d, out, args.steps)
    for name, fn in (("c1", run_c1), ("c1v", run_c1v), ("c2", run_c2), ("c2s", run_c2s), ("c3", run_c3),
                     ("c5", run_c5), ("atom_copy", run_copy_atom), ("hbm", run_hbm_regime),
                     ("sweep", run_sweep),
                     ("sweep_cold", run_sweep_cold)):
        if args.only in ("all", name):
            log("running", name)
            fn(d, B, synth, oracle, args, out)
    if args.only == "all":
        run_floor(d, out)
    log(f"done in {time.time() - t0:.1f} s")

    line = {"metric": METRIC, "value": round(ach, 1) if ach else None, "unit": "GB/s",
            "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
            "ms_per_step": round(headline_ms, 5) if headline_ms else None,
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
            "dtype": "f32", "data": "synthetic",
            "config": {"workload": "oneshot reduce, N=8 ranks, K=4096x8192 bf16 (64 MiB/rank), "
                                   "normal(0,0.02), fp32 accumulate in rank order 0..7, bf16 RNE output",
                       "n": 8, "k": 4096 * 8192, "bytes_per_call": 9 * 2 * 4096 * 8192}}
    if ach and "headline" in out and measured_traffic() is not None:
        kt = dict(KERNEL_TRACE)
        kt["gbs_at_median"] = round(gbs(out["headline"]["bytes_per_call"], kt["median_us"]), 1)
        kt["frac_at_median"] = round(kt["gbs_at_median"] / HBM_PEAK_GBS, 4)
        out["headline"]["rocprof_kernel_trace"] = kt
    if ach:
        line["roofline"] = {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS,
                            "unit": "GB/s", "frac": round(ach / HBM_PEAK_GBS, 4),
                            "traffic": measured_traffic(),
                            "kernel": HEADLINE_KERNEL}
    if "cpu_baseline" in out:
        line["cpu_baseline"] = out.pop("cpu_baseline")
    line["parity_ok"] = bool(out["parity"]) and all(out["parity"].values())
    line.update(out)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
