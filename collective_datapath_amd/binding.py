"""Thin Python binding of libpcdp.so (the C ABI in include/pc.h).

Argument marshalling only: device buffers are torch tensors (or raw device
addresses as ints), host pointer arrays are built here, and every call goes
straight to the HIP library, which does all the work.  Tensors are checked
to be on the current GPU, contiguous and large enough for the call, so a
wrong tensor raises ValueError here rather than faulting on the device; the
library itself validates everything else (alignment, sizes, overlaps).
There is no fallback: if the built library is missing, importing this
module fails.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence, Union

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libpcdp.so")

PC_OK, PC_EINVAL, PC_EALIGN, PC_EUNSUPPORTED, PC_EHIP = 0, -1, -2, -3, -4
PC_MAX_RANKS = 8
PC_LL_LINE_BYTES = 8
PC_BLOCK_PAYLOAD_BYTES = 128
PC_BLOCK_RECORD_BYTES = 136

# Every symbol include/pc.h declares.
EXPORTS = ("pc_copy", "pc_reduce", "pc_pack_ll", "pc_consume_ll", "pc_twoshot", "pc_twoshot_fused",
           "pc_twoshot_linked", "pc_twoshot_linked_workspace_bytes", "pc_twoshot_linked_static",
           "pc_allgather_copy", "pc_publish_sentinel", "pc_consume_sentinel",
           "pc_reduce_validated", "pc_strerror", "pc_abi_version")
PC_ABI_VERSION = 8          # the include/pc.h this binding is written against
PC_MAX_ATTEMPTS = 65536
PC_LINKED_GROUPS = 256
PC_LINKED_STATUS_WORD = 256       # uint64 words
PC_LINKED_POLL_LIMIT_WORD = 257   # uint64 words
PC_LINKED_STATIC_SCRATCH_BYTES = 1 << 20
PC_SENTINEL = 0xFFFF

if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"{LIB_PATH} is not built; run `python collective_datapath_amd/build.py` first")

# torch owns device memory and streams, so the library must run on torch's HIP
# runtime.  Loading torch first makes the dynamic linker resolve the library's
# libamdhip64.so.7 to the runtime torch already mapped; loading the library
# first would map a second runtime whose view of streams and allocations is
# disjoint from torch's.
import torch  # noqa: E402,F401


def _hip_runtimes():
    paths = set()
    try:
        with open("/proc/self/maps") as f:
            for line in f:
                if "libamdhip64" in line:
                    paths.add(os.path.realpath(line.split()[-1]))
    except OSError:
        pass
    return paths


_lib = ctypes.CDLL(LIB_PATH)
if len(_hip_runtimes()) > 1:
    raise ImportError("two HIP runtimes are mapped in this process "
                      f"({sorted(_hip_runtimes())}); import torch before loading libpcdp.so")
_P, _S, _I = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int
_lib.pc_copy.argtypes = [_P, _P, _S, _P]
_lib.pc_reduce.argtypes = [_P, _I, _P, _S, _P, _P]
_lib.pc_pack_ll.argtypes = [_P, _P, _S, ctypes.c_uint32, _P]
_lib.pc_consume_ll.argtypes = [_P, _I, _P, _S, ctypes.c_uint32, _P, _P]
_lib.pc_twoshot.argtypes = [_P, _I, _P, _S, _P]
_lib.pc_twoshot_fused.argtypes = [_P, _I, _P, _S, _P]
_lib.pc_twoshot_linked.argtypes = [_P, _I, _P, _S, _P, _S, _P]
_lib.pc_twoshot_linked_workspace_bytes.argtypes = [_I, _S]
_lib.pc_twoshot_linked_workspace_bytes.restype = _S
_lib.pc_twoshot_linked_static.argtypes = [_P, _I, _P, _S, _P, _P]
_lib.pc_allgather_copy.argtypes = [_P, _I, _P, _S, ctypes.c_uint64, _P, _P]
_lib.pc_publish_sentinel.argtypes = [_P, _P, _S, _P]
_lib.pc_reduce_validated.argtypes = [_P, _P, _I, _P, _S, _S, ctypes.c_uint32, ctypes.c_uint32, _P, _P]
_lib.pc_consume_sentinel.argtypes = [_P, _I, _P, _S, _P, _P]
for _f in ("pc_copy", "pc_reduce", "pc_pack_ll", "pc_consume_ll", "pc_twoshot", "pc_twoshot_fused",
           "pc_twoshot_linked", "pc_twoshot_linked_static", "pc_allgather_copy", "pc_publish_sentinel",
           "pc_consume_sentinel", "pc_reduce_validated"):
    getattr(_lib, _f).restype = _I
_lib.pc_strerror.argtypes = [_I]
_lib.pc_strerror.restype = ctypes.c_char_p
_lib.pc_abi_version.restype = _I

Buffer = Union[int, "torch.Tensor"]  # noqa: F821


class PCError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn}: {pc_strerror(status)} (status {status})")
        self.status = status


def library() -> ctypes.CDLL:
    return _lib


def _check_tensor(b, nbytes: int, what: str, dev: Optional[int] = None) -> None:
    """A tensor handed to the library must live on the current GPU, be
    contiguous and hold at least `nbytes` bytes (what the call will touch);
    anything else raises here instead of faulting on the device."""
    where = b.get_device()  # -1 for host memory
    if where < 0 or where != (torch.cuda.current_device() if dev is None else dev):
        raise ValueError(f"{what} must be a tensor on the current GPU (got {b.device})")
    if not b.is_contiguous():
        raise ValueError(f"{what} must be contiguous")
    if b.nbytes < nbytes:
        raise ValueError(f"{what} holds {b.nbytes} bytes; the call needs {nbytes}")


def _addr(b: Optional[Buffer], nbytes: int = 0, what: str = "buffer") -> int:
    """Device address of `b` (checked as above when nbytes > 0).  Raw int
    addresses are passed through unchecked."""
    if b is None:
        return 0
    if isinstance(b, int):
        return b
    if nbytes:
        _check_tensor(b, nbytes, what)
    return b.data_ptr()


def _addrs(bs: Sequence[Buffer], nbytes: int = 0, what: str = "buffer"):
    """Host array of device addresses (each tensor checked as in _addr)."""
    ptrs = []
    dev = None
    for i, b in enumerate(bs):
        if b is None:
            ptrs.append(0)
        elif isinstance(b, int):
            ptrs.append(b)
        else:
            if nbytes:
                where = b.get_device()
                if where >= 0 and dev is None:
                    dev = torch.cuda.current_device()
                if where < 0 or where != dev or not b.is_contiguous() or b.nbytes < nbytes:
                    _check_tensor(b, nbytes, f"{what}[{i}]", dev)
            ptrs.append(b.data_ptr())
    return (ctypes.c_void_p * max(len(ptrs), 1))(*ptrs)


# torch's current stream as a raw handle, without building a Stream object
# (the public route costs a few microseconds per call).
_current_raw_stream = getattr(torch._C, "_cuda_getCurrentRawStream", None)


def _stream(stream) -> int:
    if stream is None:
        if _current_raw_stream is not None:
            return _current_raw_stream(torch.cuda.current_device())
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _call(fn: str, status: int, check: bool) -> int:
    if check and status != PC_OK:
        raise PCError(fn, status)
    return status


def pc_strerror(status: int) -> str:
    """Text of a pc_status code."""
    return _lib.pc_strerror(status).decode()


def pc_abi_version() -> int:
    """PC_ABI_VERSION of the loaded library."""
    return _lib.pc_abi_version()


def pc_copy(dst: Buffer, src: Buffer, nbytes: int, stream=None, check: bool = True) -> int:
    """Atom copy: nbytes from src to dst, unchanged (include/pc.h, pc_copy)."""
    st = _lib.pc_copy(_addr(dst, nbytes, "dst"), _addr(src, nbytes, "src"), nbytes, _stream(stream))
    return _call("pc_copy", st, check)


def pc_reduce(inputs: Sequence[Buffer], out: Buffer, k: int, order: Optional[Sequence[int]] = None,
              stream=None, check: bool = True) -> int:
    """out = rank-ordered fold of the n inputs, k bf16 each; `order` permutes the fold order (include/pc.h, pc_reduce)."""
    if order is not None and len(order) != len(inputs):
        raise ValueError("order must list every rank exactly once")
    ordp = (ctypes.c_int32 * len(order))(*order) if order is not None else None
    st = _lib.pc_reduce(_addrs(inputs, 2 * k, "inputs"), len(inputs), _addr(out, 2 * k, "out"), k,
                        ctypes.cast(ordp, ctypes.c_void_p) if ordp is not None else None,
                        _stream(stream))
    return _call("pc_reduce", st, check)


def pc_pack_ll(src: Buffer, dst: Buffer, k: int, seq: int, stream=None, check: bool = True) -> int:
    """Pack k bf16 of src into k/2 LL lines stamped with seq (include/pc.h, pc_pack_ll)."""
    st = _lib.pc_pack_ll(_addr(src, 2 * k, "src"), _addr(dst, 4 * k, "dst"), k, seq, _stream(stream))
    return _call("pc_pack_ll", st, check)


def pc_consume_ll(lines: Sequence[Buffer], out: Buffer, k: int, seq: int, ready_bitmap: Buffer,
                  stream=None, check: bool = True) -> int:
    """Fold the lines every rank stamped with seq into out; one ready bit per line (include/pc.h, pc_consume_ll)."""
    st = _lib.pc_consume_ll(_addrs(lines, 4 * k, "lines"), len(lines), _addr(out, 2 * k, "out"), k,
                            seq, _addr(ready_bitmap, k // 128 * 8, "ready_bitmap"), _stream(stream))
    return _call("pc_consume_ll", st, check)


def pc_twoshot(inputs: Sequence[Buffer], outs: Sequence[Buffer], k: int, stream=None,
               check: bool = True) -> int:
    """Twoshot in two launches: slice s folded into outs[s], then copied to every outs[r] (include/pc.h, pc_twoshot)."""
    if len(outs) != len(inputs):
        raise ValueError("pc_twoshot needs one output per input")
    st = _lib.pc_twoshot(_addrs(inputs, 2 * k, "inputs"), len(inputs), _addrs(outs, 2 * k, "outs"),
                         k, _stream(stream))
    return _call("pc_twoshot", st, check)


def pc_twoshot_fused(inputs: Sequence[Buffer], outs: Sequence[Buffer], k: int, stream=None,
                     check: bool = True) -> int:
    """Twoshot in one launch: the folding workgroup writes every output (include/pc.h, pc_twoshot_fused)."""
    if len(outs) != len(inputs):
        raise ValueError("pc_twoshot_fused needs one output per input")
    st = _lib.pc_twoshot_fused(_addrs(inputs, 2 * k, "inputs"), len(inputs),
                               _addrs(outs, 2 * k, "outs"), k, _stream(stream))
    return _call("pc_twoshot_fused", st, check)


def pc_twoshot_linked_workspace_bytes(n: int, k: int) -> int:
    """Workspace bytes pc_twoshot_linked needs for (n, k); 0 if n or k is invalid."""
    return _lib.pc_twoshot_linked_workspace_bytes(n, k)


def pc_twoshot_linked(inputs: Sequence[Buffer], outs: Sequence[Buffer], k: int, workspace: Buffer,
                      workspace_bytes: Optional[int] = None, stream=None, check: bool = True) -> int:
    """Twoshot in one launch, phases linked per tile by epoch flags kept in
    `workspace` (include/pc.h, pc_twoshot_linked).
    `workspace`: zero-filled before its first use (uint64 words; a torch
    int64 tensor), then reused unchanged across calls.  `workspace_bytes` defaults to the size of a workspace
    tensor and must be given for a raw address."""
    if len(outs) != len(inputs):
        raise ValueError("pc_twoshot_linked needs one output per input")
    if workspace_bytes is None:
        if isinstance(workspace, int):
            raise ValueError("workspace_bytes is needed with a raw workspace address")
        workspace_bytes = workspace.numel() * workspace.element_size()
    need = pc_twoshot_linked_workspace_bytes(len(inputs), k) if k else 0
    st = _lib.pc_twoshot_linked(_addrs(inputs, 2 * k, "inputs"), len(inputs),
                                _addrs(outs, 2 * k, "outs"), k,
                                _addr(workspace, min(need, workspace_bytes), "workspace"),
                                workspace_bytes, _stream(stream))
    return _call("pc_twoshot_linked", st, check)


def pc_twoshot_linked_static(inputs: Sequence[Buffer], outs: Sequence[Buffer], k: int,
                             gave_up: Optional[Buffer] = None, stream=None, check: bool = True) -> int:
    """pc_twoshot_linked with the library's static workspace: allocates
    nothing (include/pc.h, pc_twoshot_linked_static).  `gave_up`: optional
    device word (int64 tensor) to which abandoned tiles are added."""
    if len(outs) != len(inputs):
        raise ValueError("pc_twoshot_linked_static needs one output per input")
    st = _lib.pc_twoshot_linked_static(_addrs(inputs, 2 * k, "inputs"), len(inputs),
                                       _addrs(outs, 2 * k, "outs"), k,
                                       _addr(gave_up, 8, "gave_up"), _stream(stream))
    return _call("pc_twoshot_linked_static", st, check)


def pc_allgather_copy(shards: Sequence[Buffer], out: Buffer, shard_bytes: int, seq: int,
                      ready_bitmap: Buffer, stream=None, check: bool = True) -> int:
    """Copy the payload of every record whose header equals seq; one ready bit per block (include/pc.h, pc_allgather_copy)."""
    blocks = shard_bytes // PC_BLOCK_PAYLOAD_BYTES
    st = _lib.pc_allgather_copy(_addrs(shards, blocks * PC_BLOCK_RECORD_BYTES, "shards"), len(shards),
                                _addr(out, len(shards) * shard_bytes, "out"), shard_bytes, seq,
                                _addr(ready_bitmap, len(shards) * blocks // 64 * 8, "ready_bitmap"),
                                _stream(stream))
    return _call("pc_allgather_copy", st, check)


def pc_publish_sentinel(src: Buffer, slot: Buffer, k: int, stream=None, check: bool = True) -> int:
    """Publish k bf16 into sentinel-armed storage, sentinel values made canonical NaN (include/pc.h, pc_publish_sentinel)."""
    st = _lib.pc_publish_sentinel(_addr(src, 2 * k, "src"), _addr(slot, 2 * k, "slot"), k,
                                  _stream(stream))
    return _call("pc_publish_sentinel", st, check)


def pc_consume_sentinel(slots: Sequence[Buffer], out: Buffer, k: int, ready_bitmap: Buffer,
                        stream=None, check: bool = True) -> int:
    """Fold the packs no rank still holds the sentinel in, then re-arm them (include/pc.h, pc_consume_sentinel)."""
    st = _lib.pc_consume_sentinel(_addrs(slots, 2 * k, "slots"), len(slots), _addr(out, 2 * k, "out"),
                                  k, _addr(ready_bitmap, k // 512 * 8, "ready_bitmap"), _stream(stream))
    return _call("pc_consume_sentinel", st, check)


def pc_reduce_validated(inputs: Sequence[Buffer], flags: Sequence[Buffer], out: Buffer, k: int,
                        elems_per_flag: int, flag: int, max_attempts: int, attempts: Buffer,
                        stream=None, check: bool = True) -> int:
    """Speculative reduce accepted per tile when the folded flags equal n * flag (include/pc.h, pc_reduce_validated)."""
    if len(flags) != len(inputs):
        raise ValueError("pc_reduce_validated needs one flag buffer per input")
    tiles = k // elems_per_flag if elems_per_flag else 0
    st = _lib.pc_reduce_validated(_addrs(inputs, 2 * k, "inputs"), _addrs(flags, 4 * tiles, "flags"),
                                  len(inputs), _addr(out, 2 * k, "out"), k, elems_per_flag,
                                  flag & 0xFFFFFFFF, max_attempts, _addr(attempts, 4 * tiles, "attempts"),
                                  _stream(stream))
    return _call("pc_reduce_validated", st, check)
