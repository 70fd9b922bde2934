// pc_launch.hpp -- host-side launchers of the datapath kernels.
//
// Arguments reaching a launcher have been validated by the C ABI layer
// (pc_api.hip): pointers non-null and 16-byte aligned, sizes in range and
// multiples of the kernel's unit, n in 1..8.  Each launcher enqueues its
// kernel(s) on `stream` and returns the HIP launch status.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace pcdp {

// Compute units of the current device, cached per device.
uint32_t device_cus();

// Atom copy of nchunks 16-byte chunks, bytes unchanged.
hipError_t launch_copy(const void* src, void* dst, size_t nchunks, hipStream_t stream);

// out[c] = fold over ranks of src[r][c], for 16-byte chunks c < nchunks.
// src has n pointers already permuted into fold order.
hipError_t launch_reduce(const void* const* src, int n, void* out, size_t nchunks,
                         hipStream_t stream);

// Twoshot: slice s (nchunks_slice 16-byte chunks) folded into outs[s], then
// copied from outs[s] into every outs[r], r != s.
hipError_t launch_twoshot(const void* const* src, int n, void* const* outs,
                          size_t nchunks_slice, hipStream_t stream);

// Single-launch twoshot: slice s folded once, in rank order, and written by
// the same workgroup to every outs[r].
hipError_t launch_twoshot_fused(const void* const* src, int n, void* const* outs,
                                size_t nchunks_slice, hipStream_t stream);

// Flag-linked single-launch twoshot on a fixed grid of kLinkGroups
// workgroups.  The workspace holds kLinkGroups 64-bit call counters, a
// header of kLinkHeaderWords 64-bit words (word 0: give-up count, word 1:
// poll limit, 0 = default) and linked_tiles() 64-bit flags.  Abandoned
// waits are counted at `status` (NULL: the workspace's header word 0).
// Returns hipErrorCooperativeLaunchTooLarge, launching nothing, when the
// grid cannot be resident on the device at once.
constexpr uint32_t kLinkGroups = 256;
constexpr uint32_t kLinkHeaderWords = 64;
size_t linked_tiles(int n, size_t nchunks_slice);
hipError_t launch_twoshot_linked(const void* const* src, int n, void* const* outs,
                                 size_t nchunks_slice, void* workspace, void* status, hipStream_t stream);

// The library's own workspace for the flag-linked twoshot, in static device
// memory (kStaticScratchBytes per GPU): its address on the current device.
constexpr size_t kStaticScratchBytes = (size_t)1 << 20;
hipError_t static_workspace(void** ptr);

// LL lines: 16-byte chunks of src -> 4 lines each.
hipError_t launch_pack_ll(const void* src, void* dst, size_t nchunks, uint32_t seq,
                          hipStream_t stream);

// LL consume over nlines lines (a multiple of 64).
hipError_t launch_consume_ll(const void* const* lines, int n, void* out, size_t nlines,
                             uint32_t seq, void* bitmap, hipStream_t stream);

// Sentinel readiness: publish 16-byte chunks with substitution; consume
// npacks 16-byte packs (a multiple of 64) from n slots, re-arming them.
hipError_t launch_publish_sentinel(const void* src, void* dst, size_t nchunks, hipStream_t stream);
hipError_t launch_consume_sentinel(void* const* slots, int n, void* out, size_t npacks,
                                   void* bitmap, hipStream_t stream);

// Speculative reduce, one workgroup per validation tile of elems_per_flag
// (2048, 4096, 6144 or 8192) elements.
hipError_t launch_reduce_validated(const void* const* src, const void* const* flags, int n,
                                   void* out, size_t k, size_t elems_per_flag, uint32_t flag,
                                   uint32_t max_attempts, void* attempts, hipStream_t stream);

// All-gather of n shards of `groups` 64-record groups each.
hipError_t launch_allgather(const void* const* shards, int n, void* out, size_t groups,
                            uint64_t seq, void* bitmap, hipStream_t stream);

}  // namespace pcdp
