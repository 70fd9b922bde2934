"""The C-ABI library loads, exports what include/pc.h declares, and rejects
bad arguments before launching anything (no GPU needed: the addresses used
here are never dereferenced, because validation fails or k == 0)."""
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "pc.h")

from collective_datapath_amd import binding as B  # noqa: E402

A = 0x7F0000000000        # 16-byte aligned fake device addresses, never touched
MB = 1 << 20


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^PC_API\s+[\w\s\*]+?\b(pc_\w+)\s*\(", text, re.M)))


def test_header_and_binding_agree():
    assert declared_functions() == sorted(B.EXPORTS)


def test_library_exports_every_declared_symbol():
    out = subprocess.run(["nm", "-D", "--defined-only", B.LIB_PATH], check=True,
                         capture_output=True, text=True).stdout
    syms = {line.split()[-1] for line in out.splitlines() if line.strip()}
    for name in declared_functions():
        assert name in syms, name
        assert getattr(B.library(), name) is not None
    # No other C entry point of ours is exported (host helpers are hidden;
    # HIP keeps kernel handle symbols visible, which are C++-mangled).
    ours = {s for s in syms if s.startswith("pc_")}
    assert ours == set(declared_functions())


def test_version_and_strerror():
    header = int(re.search(r"#define PC_ABI_VERSION (\d+)", open(HEADER).read()).group(1))
    assert B.pc_abi_version() == header == B.PC_ABI_VERSION
    assert B.pc_strerror(B.PC_OK) == "success"
    for st in (B.PC_EINVAL, B.PC_EALIGN, B.PC_EUNSUPPORTED, B.PC_EHIP, 12345):
        assert isinstance(B.pc_strerror(st), str) and B.pc_strerror(st)


def ptrs(n, stride=64 * MB, base=A):
    return [base + r * stride for r in range(n)]


OUT = A + 1024 * MB


@pytest.mark.parametrize("args,want", [
    (dict(inputs=ptrs(0), out=OUT, k=8), B.PC_EINVAL),
    (dict(inputs=ptrs(9), out=OUT, k=8), B.PC_EINVAL),
    (dict(inputs=ptrs(2) + [0], out=OUT, k=8), B.PC_EINVAL),
    (dict(inputs=ptrs(2), out=0, k=8), B.PC_EINVAL),
    (dict(inputs=ptrs(2), out=OUT, k=12), B.PC_EALIGN),
    (dict(inputs=[A, A + 8], out=OUT, k=8), B.PC_EALIGN),
    (dict(inputs=ptrs(2), out=OUT + 2, k=8), B.PC_EALIGN),
    (dict(inputs=ptrs(3), out=OUT, k=8, order=[0, 0, 1]), B.PC_EINVAL),
    (dict(inputs=ptrs(3), out=OUT, k=8, order=[0, 1, 3]), B.PC_EINVAL),
    (dict(inputs=ptrs(3), out=OUT, k=8, order=[-1, 0, 1]), B.PC_EINVAL),
    (dict(inputs=ptrs(2), out=A + 16, k=64), B.PC_EINVAL),          # partial overlap
    (dict(inputs=ptrs(2), out=OUT, k=(1 << 34) + 8), B.PC_EINVAL),   # above the maximum
    (dict(inputs=ptrs(2), out=OUT, k=0), B.PC_OK),                   # empty: no-op
    (dict(inputs=[0, 0], out=0, k=0), B.PC_OK),                      # empty tensors
])
def test_reduce_validation(args, want):
    assert B.pc_reduce(stream=0, check=False, **args) == want


def test_reduce_binding_checks_order_length():
    with pytest.raises(ValueError):
        B.pc_reduce(ptrs(3), OUT, 8, order=[0, 1], stream=0)


def test_error_raises_with_status():
    with pytest.raises(B.PCError) as e:
        B.pc_reduce(ptrs(9), OUT, 8, stream=0)
    assert e.value.status == B.PC_EINVAL


@pytest.mark.parametrize("args,want", [
    (dict(src=A, dst=OUT, k=8, seq=0), B.PC_EINVAL),
    (dict(src=A, dst=OUT, k=12, seq=1), B.PC_EALIGN),
    (dict(src=A + 8, dst=OUT, k=8, seq=1), B.PC_EALIGN),
    (dict(src=0, dst=OUT, k=8, seq=1), B.PC_EINVAL),
    (dict(src=A, dst=A + 16, k=64, seq=1), B.PC_EINVAL),
    (dict(src=A, dst=OUT, k=0, seq=1), B.PC_OK),
])
def test_pack_validation(args, want):
    assert B.pc_pack_ll(stream=0, check=False, **args) == want


@pytest.mark.parametrize("args,want", [
    (dict(lines=ptrs(2), out=OUT, k=128, seq=0, ready_bitmap=OUT + MB), B.PC_EINVAL),
    (dict(lines=ptrs(9), out=OUT, k=128, seq=1, ready_bitmap=OUT + MB), B.PC_EINVAL),
    (dict(lines=ptrs(2), out=OUT, k=64, seq=1, ready_bitmap=OUT + MB), B.PC_EALIGN),
    (dict(lines=ptrs(2), out=OUT, k=128, seq=1, ready_bitmap=0), B.PC_EINVAL),
    (dict(lines=ptrs(2), out=OUT, k=128, seq=1, ready_bitmap=OUT + 8), B.PC_EALIGN),
    (dict(lines=ptrs(2), out=OUT, k=128, seq=1, ready_bitmap=OUT + 128), B.PC_EINVAL),
    (dict(lines=ptrs(2), out=A + 64, k=128, seq=1, ready_bitmap=OUT + MB), B.PC_EINVAL),
    (dict(lines=ptrs(2), out=OUT, k=0, seq=1, ready_bitmap=0), B.PC_OK),
])
def test_consume_validation(args, want):
    assert B.pc_consume_ll(stream=0, check=False, **args) == want


@pytest.mark.parametrize("args,want", [
    (dict(inputs=ptrs(4), outs=ptrs(4, base=OUT), k=8 * 4 + 8), B.PC_EALIGN),
    (dict(inputs=ptrs(4), outs=ptrs(4, base=OUT, stride=16), k=64 * 4), B.PC_EINVAL),
    (dict(inputs=ptrs(4), outs=ptrs(4, base=A + 32), k=64 * 4), B.PC_EINVAL),
    (dict(inputs=ptrs(4), outs=ptrs(4, base=OUT), k=0), B.PC_OK),
    (dict(inputs=ptrs(9), outs=ptrs(9, base=OUT), k=72), B.PC_EINVAL),
])
def test_twoshot_validation(args, want):
    assert B.pc_twoshot(stream=0, check=False, **args) == want
    assert B.pc_twoshot_fused(stream=0, check=False, **args) == want
    ws = A + 4096 * MB
    assert B.pc_twoshot_linked(workspace=ws, workspace_bytes=64 * MB, stream=0, check=False,
                               **args) == want


WS = A + 4096 * MB


def linked_need(n, k):
    return B.pc_twoshot_linked_workspace_bytes(n, k)


def test_linked_workspace_bytes():
    fixed = 8 * (B.PC_LINKED_GROUPS + 64)   # uint64 words
    assert linked_need(8, 0) == fixed
    # 1 MiB per rank, n = 8: slices of 8192 chunks, 512-chunk tiles -> 128 tiles.
    assert linked_need(8, 8 * 65536) == fixed + 8 * 128
    # 256 KiB per rank: 256-chunk tiles -> 8 slices of 8 tiles.
    assert linked_need(8, 8 * 16384) == fixed + 8 * 64
    # A ragged slice rounds its tile count up: 3 slices of 257 chunks -> 2 tiles each.
    assert linked_need(3, 3 * 8 * 257) == fixed + 8 * 6
    # Tiles lie on a grid of 8-chunk (128-byte) lines of the buffer.  Two
    # slices of 509 chunks: slice 1 starts 5 chunks into a line, so its tiles
    # cover [509, 760), [760, 1016) and [1016, 1018) -> 3 tiles per slice.
    assert linked_need(2, 2 * 8 * 509) == fixed + 8 * 2 * 3
    # Slices that start on a line keep ceil(chunks / tile) tiles: 2 x 512.
    assert linked_need(2, 2 * 8 * 512) == fixed + 8 * 2 * 2
    # From 4 MiB per rank the tiles hold 1024 chunks: 8 slices of 32768 chunks.
    assert linked_need(8, 1 << 21) == fixed + 8 * 8 * 32
    for bad in [(0, 64), (9, 72), (4, 8 * 4 + 8), (2, (1 << 34) + 16)]:
        assert linked_need(*bad) == 0


@pytest.mark.parametrize("ws,ws_bytes,want", [
    (0, 64 * MB, B.PC_EINVAL),                 # no workspace
    (WS + 4, 64 * MB, B.PC_EALIGN),            # misaligned
    (WS, None, B.PC_EINVAL),                   # one word too small
    (OUT + 16, 64 * MB, B.PC_EINVAL),          # overlaps outs[0]
    (A + 64 * MB - 64, 64 * MB, B.PC_EINVAL),  # overlaps inputs[0]'s tail and inputs[1]
])
def test_twoshot_linked_workspace_validation(ws, ws_bytes, want):
    n, k = 4, 4 * 8 * 300
    if ws_bytes is None:
        ws_bytes = linked_need(n, k) - 4
    assert B.pc_twoshot_linked(ptrs(n), ptrs(n, base=OUT), k, ws, workspace_bytes=ws_bytes,
                               stream=0, check=False) == want


def test_twoshot_linked_binding_needs_size_for_raw_workspace():
    with pytest.raises(ValueError):
        B.pc_twoshot_linked(ptrs(2), ptrs(2, base=OUT), 16, WS, stream=0)


@pytest.mark.parametrize("args,want", [
    (dict(shards=ptrs(2), out=OUT, shard_bytes=8192, seq=0, ready_bitmap=OUT + MB), B.PC_EINVAL),
    (dict(shards=ptrs(2), out=OUT, shard_bytes=4096, seq=1, ready_bitmap=OUT + MB), B.PC_EALIGN),
    (dict(shards=[A, A + 8 + 64 * MB], out=OUT, shard_bytes=8192, seq=1, ready_bitmap=OUT + MB), B.PC_EALIGN),
    (dict(shards=ptrs(2), out=OUT, shard_bytes=8192, seq=1, ready_bitmap=OUT + 64), B.PC_EINVAL),
    (dict(shards=ptrs(2), out=A + 4096, shard_bytes=8192, seq=1, ready_bitmap=OUT + MB), B.PC_EINVAL),
    (dict(shards=ptrs(2), out=OUT, shard_bytes=0, seq=1, ready_bitmap=0), B.PC_OK),
])
def test_allgather_validation(args, want):
    assert B.pc_allgather_copy(stream=0, check=False, **args) == want


def test_one_hip_runtime_in_process():
    # The library must share torch's HIP runtime (streams, allocations).
    assert len(B._hip_runtimes()) == 1


@pytest.mark.parametrize("args,want", [
    (dict(src=A, slot=OUT, k=12), B.PC_EALIGN),
    (dict(src=A + 8, slot=OUT, k=8), B.PC_EALIGN),
    (dict(src=0, slot=OUT, k=8), B.PC_EINVAL),
    (dict(src=A, slot=A + 16, k=64), B.PC_EINVAL),
    (dict(src=A, slot=OUT, k=(1 << 34) + 8), B.PC_EINVAL),
    (dict(src=A, slot=OUT, k=0), B.PC_OK),
])
def test_publish_sentinel_validation(args, want):
    assert B.pc_publish_sentinel(stream=0, check=False, **args) == want


@pytest.mark.parametrize("args,want", [
    (dict(slots=ptrs(9), out=OUT, k=512, ready_bitmap=OUT + MB), B.PC_EINVAL),
    (dict(slots=ptrs(2), out=OUT, k=256, ready_bitmap=OUT + MB), B.PC_EALIGN),
    (dict(slots=ptrs(2), out=OUT, k=512, ready_bitmap=0), B.PC_EINVAL),
    (dict(slots=ptrs(2), out=OUT + 8, k=512, ready_bitmap=OUT + MB), B.PC_EALIGN),
    (dict(slots=ptrs(2, stride=512), out=OUT, k=512, ready_bitmap=OUT + MB), B.PC_EINVAL),
    (dict(slots=ptrs(2), out=A + 512, k=512, ready_bitmap=OUT + MB), B.PC_EINVAL),
    (dict(slots=ptrs(2), out=OUT, k=512, ready_bitmap=OUT + 512), B.PC_EINVAL),
    (dict(slots=ptrs(2), out=OUT, k=0, ready_bitmap=0), B.PC_OK),
])
def test_consume_sentinel_validation(args, want):
    assert B.pc_consume_sentinel(stream=0, check=False, **args) == want


FL = A + 2048 * MB


@pytest.mark.parametrize("args,want", [
    (dict(inputs=ptrs(2), flags=ptrs(2, base=FL), out=OUT, k=2048, elems_per_flag=2048, flag=1,
          max_attempts=0, attempts=OUT + MB), B.PC_EINVAL),
    (dict(inputs=ptrs(2), flags=ptrs(2, base=FL), out=OUT, k=2048, elems_per_flag=2048, flag=1,
          max_attempts=65537, attempts=OUT + MB), B.PC_EINVAL),
    (dict(inputs=ptrs(2), flags=ptrs(2, base=FL), out=OUT, k=4096, elems_per_flag=1024, flag=1,
          max_attempts=1, attempts=OUT + MB), B.PC_EINVAL),
    (dict(inputs=ptrs(2), flags=ptrs(2, base=FL), out=OUT, k=4096, elems_per_flag=16384, flag=1,
          max_attempts=1, attempts=OUT + MB), B.PC_EINVAL),
    (dict(inputs=ptrs(2), flags=ptrs(2, base=FL), out=OUT, k=6144, elems_per_flag=4096, flag=1,
          max_attempts=1, attempts=OUT + MB), B.PC_EALIGN),
    (dict(inputs=ptrs(2), flags=[FL, FL + 2], out=OUT, k=2048, elems_per_flag=2048, flag=1,
          max_attempts=1, attempts=OUT + MB), B.PC_EALIGN),
    (dict(inputs=ptrs(2), flags=[FL, 0], out=OUT, k=2048, elems_per_flag=2048, flag=1,
          max_attempts=1, attempts=OUT + MB), B.PC_EINVAL),
    (dict(inputs=ptrs(2), flags=ptrs(2, base=FL), out=OUT, k=2048, elems_per_flag=2048, flag=1,
          max_attempts=1, attempts=OUT + 64), B.PC_EINVAL),
    (dict(inputs=ptrs(2), flags=ptrs(2, base=FL), out=OUT, k=2048, elems_per_flag=2048, flag=1,
          max_attempts=1, attempts=FL), B.PC_EINVAL),
    (dict(inputs=ptrs(2), flags=ptrs(2, base=FL), out=OUT, k=0, elems_per_flag=2048, flag=1,
          max_attempts=1, attempts=0), B.PC_OK),
])
def test_reduce_validated_validation(args, want):
    assert B.pc_reduce_validated(stream=0, check=False, **args) == want


def test_binding_rejects_host_and_short_tensors():
    import torch
    cpu = torch.zeros(64, dtype=torch.int16)
    with pytest.raises(ValueError):
        B.pc_reduce([cpu, cpu], cpu, 64, stream=0)
    with pytest.raises(ValueError):
        B.pc_publish_sentinel(cpu, cpu, 64, stream=0)


@pytest.mark.parametrize("args,want", [
    (dict(dst=0, src=A, nbytes=16), B.PC_EINVAL),
    (dict(dst=OUT, src=0, nbytes=16), B.PC_EINVAL),
    (dict(dst=OUT + 8, src=A, nbytes=16), B.PC_EALIGN),
    (dict(dst=OUT, src=A + 4, nbytes=16), B.PC_EALIGN),
    (dict(dst=OUT, src=A, nbytes=24), B.PC_EALIGN),
    (dict(dst=A + 16, src=A, nbytes=64), B.PC_EINVAL),            # partial overlap
    (dict(dst=A, src=A + 48, nbytes=64), B.PC_EINVAL),
    (dict(dst=OUT, src=A, nbytes=(1 << 35) + 16), B.PC_EINVAL),   # above the maximum
    (dict(dst=A, src=A, nbytes=4096), B.PC_OK),                    # onto itself: no-op
    (dict(dst=0, src=0, nbytes=0), B.PC_OK),                       # empty
])
def test_copy_validation(args, want):
    assert B.pc_copy(stream=0, check=False, **args) == want


def static_limit(n):
    """The largest k (a multiple of 8 * n) whose linked workspace fits in the
    static scratch of pc_twoshot_linked_static."""
    unit = 8 * n
    lo, hi = unit, unit
    while B.pc_twoshot_linked_workspace_bytes(n, hi) <= B.PC_LINKED_STATIC_SCRATCH_BYTES:
        lo, hi = hi, 2 * hi
    while hi - lo > unit:
        mid = (lo + hi) // 2 // unit * unit
        if B.pc_twoshot_linked_workspace_bytes(n, mid) <= B.PC_LINKED_STATIC_SCRATCH_BYTES:
            lo = mid
        else:
            hi = mid
    return lo


@pytest.mark.parametrize("n", [1, 3, 8])
def test_twoshot_linked_static_rejects_calls_beyond_its_scratch(n):
    k = static_limit(n) + 8 * n
    assert B.pc_twoshot_linked_workspace_bytes(n, k) > B.PC_LINKED_STATIC_SCRATCH_BYTES
    # About 2 GiB per rank at 8 ranks: far-apart fake addresses, never touched.
    big = 64 << 30
    assert B.pc_twoshot_linked_static(ptrs(n, stride=big), ptrs(n, stride=big, base=A + 16 * big), k,
                                      stream=0, check=False) == B.PC_EINVAL


@pytest.mark.parametrize("gave_up,want", [
    (A + 4096 * MB + 4, B.PC_EALIGN),          # not 8-byte aligned
    (OUT + 8, B.PC_EINVAL),                    # inside outs[0]
    (A + 8, B.PC_EINVAL),                      # inside inputs[0]
])
def test_twoshot_linked_static_gave_up_word_validation(gave_up, want):
    n, k = 4, 4 * 8 * 300
    assert B.pc_twoshot_linked_static(ptrs(n), ptrs(n, base=OUT), k, gave_up, stream=0,
                                      check=False) == want


def test_twoshot_linked_static_shares_twoshot_validation():
    assert B.pc_twoshot_linked_static(ptrs(4), ptrs(4, base=OUT), 64 * 4 + 8, stream=0,
                                      check=False) == B.PC_EALIGN
    assert B.pc_twoshot_linked_static(ptrs(4), ptrs(4, base=A + 32), 64 * 4, stream=0,
                                      check=False) == B.PC_EINVAL
    assert B.pc_twoshot_linked_static([0] * 4, [0] * 4, 0, stream=0, check=False) == B.PC_OK
