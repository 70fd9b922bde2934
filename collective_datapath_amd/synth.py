"""Seeded synthetic inputs for the datapath calls.

This module is shared by the parity tests, the benchmark and the oracle side
of every comparison.  It holds no step of the method: it only draws values,
picks which lines or blocks are stale, and lays records out in memory.  Both
the HIP path and the CPU oracle consume exactly the bytes produced here.

Recipe (one generator per (config, stream, rank)):
  * ``numpy.random.default_rng([cfg, stream, rank])``; stream 0 draws the
    current payload, stream 1 the payload of stale lines/blocks, stream 2 the
    choice of which lines/blocks are stale.
  * Values are drawn as float32 and turned into bf16 bit patterns by keeping
    the upper 16 bits (truncation toward zero).  That is a choice of input
    distribution only; the datapath's own fp32 -> bf16 rounding is never
    used to make inputs.
  * Stale selections take the first ``floor(frac * count)`` entries of a
    seeded permutation, independently per rank.  Stale payloads are drawn
    from uniform[2, 3] so that wrongly accepting a stale line changes the
    result by far more than one bf16 ulp of a fresh value.
"""
from __future__ import annotations

import dataclasses
from typing import List, Tuple

import numpy as np

SEQ_CURRENT = 7
SEQ_STALE = 6
BLOCK_PAYLOAD_BYTES = 128
BLOCK_RECORD_BYTES = 136  # u64 sequence header followed by 128 payload bytes


def rng(cfg: int, stream: int, rank: int) -> np.random.Generator:
    return np.random.default_rng([cfg, stream, rank])


def f32_to_bf16_bits_trunc(x: np.ndarray) -> np.ndarray:
    """Upper half of each float32 (truncation); input-distribution helper."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    return (x.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def uniform_bf16(cfg: int, stream: int, rank: int, n: int,
                 lo: float = -1.0, hi: float = 1.0) -> np.ndarray:
    g = rng(cfg, stream, rank)
    return f32_to_bf16_bits_trunc(g.uniform(lo, hi, size=n).astype(np.float32))


def normal_bf16(cfg: int, stream: int, rank: int, n: int,
                sigma: float = 1.0) -> np.ndarray:
    g = rng(cfg, stream, rank)
    x = g.standard_normal(size=n, dtype=np.float32)
    if sigma != 1.0:
        x *= np.float32(sigma)
    return f32_to_bf16_bits_trunc(x)


def stale_mask(cfg: int, rank: int, count: int, frac: float) -> np.ndarray:
    """Boolean mask over ``count`` items with exactly floor(frac*count) set."""
    g = rng(cfg, 2, rank)
    nstale = int(np.floor(frac * count))
    m = np.zeros(count, dtype=bool)
    m[g.permutation(count)[:nstale]] = True
    return m


# --------------------------------------------------------------------------
# Workloads.  Names say what each one is; sizes are bf16 elements per rank.
# --------------------------------------------------------------------------

@dataclasses.dataclass(frozen=True)
class ReduceCase:
    """N rank-staged bf16 buffers to be reduced elementwise."""
    name: str
    cfg: int
    n: int
    k: int
    dist: str          # "uniform" (uniform[-1,1]) or "normal"
    sigma: float = 1.0

    def inputs(self) -> List[np.ndarray]:
        if self.dist == "uniform":
            return [uniform_bf16(self.cfg, 0, r, self.k) for r in range(self.n)]
        return [normal_bf16(self.cfg, 0, r, self.k, self.sigma) for r in range(self.n)]

    def bytes_moved(self) -> int:
        return (self.n + 1) * 2 * self.k


@dataclasses.dataclass(frozen=True)
class LLCase:
    """Self-synchronizing reduce: per-rank payloads, stale payloads, stale masks."""
    name: str
    cfg: int
    n: int
    k: int
    stale_frac: float = 0.05
    seq: int = SEQ_CURRENT
    stale_seq: int = SEQ_STALE

    @property
    def lines(self) -> int:
        return self.k // 2

    def payloads(self) -> List[np.ndarray]:
        return [uniform_bf16(self.cfg, 0, r, self.k) for r in range(self.n)]

    def stale_payloads(self) -> List[np.ndarray]:
        return [uniform_bf16(self.cfg, 1, r, self.k, 2.0, 3.0) for r in range(self.n)]

    def stale_masks(self) -> List[np.ndarray]:
        return [stale_mask(self.cfg, r, self.lines, self.stale_frac) for r in range(self.n)]


@dataclasses.dataclass(frozen=True)
class GatherCase:
    """All-gather copy: N shards laid out as [u64 seq | 128 B payload] records."""
    name: str
    cfg: int
    n: int
    shard_bytes: int
    stale_frac: float = 0.10
    seq: int = SEQ_CURRENT
    stale_seq: int = SEQ_STALE

    @property
    def blocks(self) -> int:
        return self.shard_bytes // BLOCK_PAYLOAD_BYTES

    def payloads(self) -> List[np.ndarray]:
        return [uniform_bf16(self.cfg, 0, r, self.shard_bytes // 2) for r in range(self.n)]

    def stale_payloads(self) -> List[np.ndarray]:
        return [uniform_bf16(self.cfg, 1, r, self.shard_bytes // 2, 2.0, 3.0)
                for r in range(self.n)]

    def stale_masks(self) -> List[np.ndarray]:
        return [stale_mask(self.cfg, r, self.blocks, self.stale_frac) for r in range(self.n)]

    def records(self) -> Tuple[List[np.ndarray], List[np.ndarray]]:
        """Per-shard record bytes (uint8) and stale masks.

        A stale block carries the stale sequence number and the stale payload
        (what a slot still holds from the previous call); a current block
        carries the current sequence number and the fresh payload.
        """
        out, masks = [], []
        for r, (fresh, stale, m) in enumerate(zip(self.payloads(), self.stale_payloads(),
                                                  self.stale_masks())):
            rec = np.empty((self.blocks, BLOCK_RECORD_BYTES // 8), dtype=np.uint64)
            rec[:, 0] = np.where(m, np.uint64(self.stale_seq), np.uint64(self.seq))
            body = np.where(m[:, None],
                            stale.view(np.uint64).reshape(self.blocks, 16),
                            fresh.view(np.uint64).reshape(self.blocks, 16))
            rec[:, 1:] = body
            out.append(rec.reshape(-1).view(np.uint8))
            masks.append(m)
        return out, masks


SENTINEL = 0xFFFF        # bf16 pattern reserved for "not yet arrived"
PACK_ELEMS = 8           # readiness unit of sentinel storage: 16 bytes


@dataclasses.dataclass(frozen=True)
class SentinelCase:
    """Sentinel readiness: per-rank payloads with some values equal to the
    sentinel (so publication has to substitute them), packs that have not
    arrived yet (still all sentinel) and torn packs (the upper half of the
    pack still sentinel)."""
    name: str
    cfg: int
    n: int
    k: int
    missing_frac: float = 0.05
    torn_frac: float = 0.005
    collision_frac: float = 0.01

    @property
    def packs(self) -> int:
        return self.k // PACK_ELEMS

    def payloads(self) -> List[np.ndarray]:
        out = []
        for r in range(self.n):
            x = uniform_bf16(self.cfg, 0, r, self.k)
            g = rng(self.cfg, 3, r)
            hit = g.permutation(self.k)[: int(np.floor(self.collision_frac * self.k))]
            x[hit] = SENTINEL
            out.append(x)
        return out

    def masks(self) -> List[Tuple[np.ndarray, np.ndarray]]:
        """(missing, torn) boolean masks over packs, disjoint, per rank."""
        res = []
        for r in range(self.n):
            g = rng(self.cfg, 2, r)
            perm = g.permutation(self.packs)
            nm = int(np.floor(self.missing_frac * self.packs))
            nt = int(np.floor(self.torn_frac * self.packs))
            missing = np.zeros(self.packs, dtype=bool)
            torn = np.zeros(self.packs, dtype=bool)
            missing[perm[:nm]] = True
            torn[perm[nm:nm + nt]] = True
            res.append((missing, torn))
        return res


@dataclasses.dataclass(frozen=True)
class ValidatedCase:
    """Speculative reduce: payloads plus one validation flag per tile per rank.
    A stale tile on a rank carries the previous call's flag (flag - 1)."""
    name: str
    cfg: int
    n: int
    k: int
    elems_per_flag: int
    flag: int = 5
    stale_frac: float = 0.05

    @property
    def tiles(self) -> int:
        return self.k // self.elems_per_flag

    def payloads(self) -> List[np.ndarray]:
        return [uniform_bf16(self.cfg, 0, r, self.k) for r in range(self.n)]

    def flags(self) -> List[np.ndarray]:
        out = []
        for r in range(self.n):
            m = stale_mask(self.cfg, r, self.tiles, self.stale_frac)
            f = np.full(self.tiles, self.flag & 0xFFFFFFFF, dtype=np.uint32)
            f[m] = np.uint32((self.flag - 1) & 0xFFFFFFFF)
            out.append(f)
        return out


def unarrive(slot: np.ndarray, missing: np.ndarray, torn: np.ndarray) -> np.ndarray:
    """Put the sentinel back where data has not arrived: whole missing packs,
    and the upper half of torn packs.  Returns a new array."""
    s = np.array(slot, dtype=np.uint16, copy=True).reshape(-1, PACK_ELEMS)
    s[missing] = SENTINEL
    s[torn, PACK_ELEMS // 2:] = SENTINEL
    return s.reshape(-1)


# The five workloads the datapath is measured and checked on.
C1_ONESHOT_8K = ReduceCase("oneshot reduce N=4 K=1x4096 bf16 (8 KiB/rank)", 1, 4, 4096, "uniform")
C2_LL_128K = LLCase("LL self-synchronizing reduce N=8 K=16x4096 bf16 (128 KiB/rank), 5% stale", 2, 8, 16 * 4096)
C3_TWOSHOT_1M = ReduceCase("twoshot N=8 K=64x8192 bf16 (1 MiB/rank)", 3, 8, 64 * 8192, "normal", 1.0)
C4_ONESHOT_64M = ReduceCase("oneshot reduce N=8 K=4096x8192 bf16 (64 MiB/rank)", 4, 8, 4096 * 8192, "normal", 0.02)
C5_ALLGATHER_2M = GatherCase("all-gather copy N=8, 2 MiB shards in 136 B records, 10% stale", 5, 8, 2 * 1024 * 1024)

# Sentinel-readiness consume at the LL workload's shape (compared against it).
C2S_SENTINEL_128K = SentinelCase("sentinel self-synchronizing reduce N=8 K=16x4096 bf16 (128 KiB/rank), "
                                 "5% packs unarrived, 0.5% torn", 6, 8, 16 * 4096)

# Speculative reduce at decode size: 8 ranks x 8 KiB, one flag per 4096 elements.
C1V_VALIDATED_8K = ValidatedCase("speculative reduce N=8 K=1x4096 bf16 (8 KiB/rank), one flag", 7, 8, 4096, 4096,
                                 stale_frac=0.0)

# Per-rank sizes of the latency sweep (bytes).
SWEEP_BYTES = [8 << 10, 16 << 10, 32 << 10, 64 << 10, 128 << 10, 256 << 10, 512 << 10, 1 << 20]
