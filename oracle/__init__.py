"""ctypes view of the CPU oracle (oracle/pc_oracle.c).

TEST INFRASTRUCTURE ONLY: imported by tests/, by the smoke check and by the
benchmark's CPU-baseline leg.  The library's product path never imports it.
The oracle shares no code with the HIP path.  Every function here works on
host numpy arrays of bf16 bit patterns (uint16) and returns new arrays.
"""
from __future__ import annotations

import ctypes
import os
from typing import List, Optional, Sequence, Tuple

import numpy as np

from . import build as _build

_LIB: Optional[ctypes.CDLL] = None


def lib() -> ctypes.CDLL:
    global _LIB
    if _LIB is None:
        # PC_ORACLE_LIB points the pins at a deliberately broken build of the
        # oracle (tests/test_oracle_mutants.py); normal runs never set it.
        path = os.environ.get("PC_ORACLE_LIB", _build.LIB)
        if path == _build.LIB and not os.path.exists(path):
            _build.build()
        L = ctypes.CDLL(path)
        P, S, I = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int
        L.orc_fpenv_ok.restype = I
        L.orc_widen.argtypes = [ctypes.c_uint16]
        L.orc_widen.restype = ctypes.c_float
        L.orc_narrow.argtypes = [ctypes.c_float]
        L.orc_narrow.restype = ctypes.c_uint16
        L.orc_narrow_array.argtypes = [P, P, S]
        L.orc_widen_array.argtypes = [P, P, S]
        L.orc_reduce.argtypes = [P, I, P, S, P, I]
        L.orc_reduce.restype = I
        L.orc_pack_ll.argtypes = [P, P, S, ctypes.c_uint32]
        L.orc_pack_ll.restype = I
        L.orc_consume_ll.argtypes = [P, I, P, S, ctypes.c_uint32, P]
        L.orc_consume_ll.restype = I
        L.orc_twoshot.argtypes = [P, I, P, S]
        L.orc_twoshot.restype = I
        L.orc_allgather_copy.argtypes = [P, I, P, S, ctypes.c_uint64, P]
        L.orc_allgather_copy.restype = I
        L.orc_reduce_validated.argtypes = [P, P, I, P, S, S, ctypes.c_uint32, P]
        L.orc_reduce_validated.restype = I
        L.orc_publish_sentinel.argtypes = [P, P, S]
        L.orc_publish_sentinel.restype = I
        L.orc_consume_sentinel.argtypes = [P, I, P, S, P]
        L.orc_consume_sentinel.restype = I
        _LIB = L
    return _LIB


def _ptr(a: np.ndarray) -> int:
    return a.ctypes.data


def _ptr_array(arrs: Sequence[np.ndarray]):
    return (ctypes.c_void_p * len(arrs))(*[_ptr(a) for a in arrs])


def _check(rc: int, what: str) -> None:
    if rc == -2:
        raise RuntimeError(f"{what}: host float environment is not IEEE (FTZ/DAZ set)")
    if rc != 0:
        raise ValueError(f"{what}: rejected arguments (rc={rc})")


def fpenv_ok() -> bool:
    return bool(lib().orc_fpenv_ok())


def widen(h: np.ndarray) -> np.ndarray:
    h = np.ascontiguousarray(h, dtype=np.uint16)
    out = np.empty(h.shape, dtype=np.float32)
    lib().orc_widen_array(_ptr(h), _ptr(out), h.size)
    return out


def narrow(f: np.ndarray) -> np.ndarray:
    f = np.ascontiguousarray(f, dtype=np.float32)
    out = np.empty(f.shape, dtype=np.uint16)
    lib().orc_narrow_array(_ptr(f), _ptr(out), f.size)
    return out


def reduce(inputs: Sequence[np.ndarray], order: Optional[Sequence[int]] = None,
           threads: int = 1, out: Optional[np.ndarray] = None) -> np.ndarray:
    xs = [np.ascontiguousarray(x, dtype=np.uint16) for x in inputs]
    k = xs[0].size
    assert all(x.size == k for x in xs)
    if out is None:
        out = np.empty(k, dtype=np.uint16)
    ordp = None
    if order is not None:
        ordarr = np.ascontiguousarray(order, dtype=np.int32)
        ordp = _ptr(ordarr)
    _check(lib().orc_reduce(_ptr_array(xs), len(xs), _ptr(out), k, ordp, threads), "orc_reduce")
    return out


def pack_ll(src: np.ndarray, seq: int) -> np.ndarray:
    src = np.ascontiguousarray(src, dtype=np.uint16)
    dst = np.empty(src.size // 2, dtype=np.uint64)
    _check(lib().orc_pack_ll(_ptr(src), _ptr(dst), src.size, seq), "orc_pack_ll")
    return dst


def consume_ll(lines: Sequence[np.ndarray], k: int, seq: int,
               out: Optional[np.ndarray] = None) -> Tuple[np.ndarray, np.ndarray]:
    ls = [np.ascontiguousarray(x, dtype=np.uint64) for x in lines]
    if out is None:
        out = np.full(k, 0xFFFF, dtype=np.uint16)
    bitmap = np.empty(k // 2 // 64, dtype=np.uint64)
    _check(lib().orc_consume_ll(_ptr_array(ls), len(ls), _ptr(out), k, seq, _ptr(bitmap)),
           "orc_consume_ll")
    return out, bitmap


def twoshot(inputs: Sequence[np.ndarray]) -> List[np.ndarray]:
    xs = [np.ascontiguousarray(x, dtype=np.uint16) for x in inputs]
    k = xs[0].size
    outs = [np.full(k, 0xFFFF, dtype=np.uint16) for _ in xs]
    _check(lib().orc_twoshot(_ptr_array(xs), len(xs), _ptr_array(outs), k), "orc_twoshot")
    return outs


def allgather_copy(shards: Sequence[np.ndarray], shard_bytes: int, seq: int,
                   out: Optional[np.ndarray] = None) -> Tuple[np.ndarray, np.ndarray]:
    ss = [np.ascontiguousarray(s, dtype=np.uint8) for s in shards]
    n = len(ss)
    if out is None:
        out = np.full(n * shard_bytes // 2, 0xFFFF, dtype=np.uint16)
    bitmap = np.empty(n * shard_bytes // 128 // 64, dtype=np.uint64)
    _check(lib().orc_allgather_copy(_ptr_array(ss), n, _ptr(out), shard_bytes, seq, _ptr(bitmap)),
           "orc_allgather_copy")
    return out, bitmap


SENTINEL = 0xFFFF


def publish_sentinel(src: np.ndarray) -> np.ndarray:
    src = np.ascontiguousarray(src, dtype=np.uint16)
    dst = np.empty_like(src)
    _check(lib().orc_publish_sentinel(_ptr(src), _ptr(dst), src.size), "orc_publish_sentinel")
    return dst


def consume_sentinel(slots: Sequence[np.ndarray], k: int, out: Optional[np.ndarray] = None):
    """Returns (out, bitmap, slots_after): the slots are copied, consumed and
    re-armed; the caller's arrays are not modified."""
    ss = [np.array(s, dtype=np.uint16, copy=True) for s in slots]
    if out is None:
        out = np.full(k, 0xFFFF, dtype=np.uint16)
    bitmap = np.empty(k // 8 // 64, dtype=np.uint64)
    _check(lib().orc_consume_sentinel(_ptr_array(ss), len(ss), _ptr(out), k, _ptr(bitmap)),
           "orc_consume_sentinel")
    return out, bitmap, ss


def reduce_validated(inputs: Sequence[np.ndarray], flags: Sequence[np.ndarray], elems_per_flag: int,
                     flag: int, out: Optional[np.ndarray] = None) -> Tuple[np.ndarray, np.ndarray]:
    xs = [np.ascontiguousarray(x, dtype=np.uint16) for x in inputs]
    fs = [np.ascontiguousarray(f, dtype=np.uint32) for f in flags]
    k = xs[0].size
    if out is None:
        out = np.full(k, 0xFFFF, dtype=np.uint16)
    ok = np.empty(k // elems_per_flag, dtype=np.uint32)
    _check(lib().orc_reduce_validated(_ptr_array(xs), _ptr_array(fs), len(xs), _ptr(out), k,
                                      elems_per_flag, flag & 0xFFFFFFFF, _ptr(ok)),
           "orc_reduce_validated")
    return out, ok
