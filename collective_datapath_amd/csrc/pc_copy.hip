// pc_copy.hip -- the Atom's copy: one contiguous byte range, moved in 16-byte
// units, bytes unchanged.
//
// "Purlin: Separating Orchestration from the Datapath of Collectives",
// Section 3.3: the Atom offers two datapath primitives, a copy of one
// contiguous range and a typed reduce of n sources; both run through the same
// transfer pipeline, where the per-element step of a copy is just a store.
// The copy-outs of the twoshot and all-gather calls are this primitive with a
// fan-out or a readiness test added; this entry point is the bare form.
//
// One shape serves every size: short-lived workgroups of 256 lanes that each
// load one 4 KiB tile, one 16-byte chunk per lane, and store it.  A stream of
// copies is written fastest by many workgroups that write a few KiB each and
// end, so this beats a persistent grid that walks tiles in batches (at
// 1 GiB: 324 vs 360 us; 512 MiB: 163 vs 173; 256 MiB: 74.6 vs 75.0 warm and
// 82.4 vs 84.7 us with the buffers rotated past the last-level cache).  The
// stores are device-scope at every size (32 MiB: 7.9 vs 9.7 us with the
// default policy; 8 MiB: 2.8 vs 3.1; 1 MiB in a graph: 1.57 vs 1.85), and
// above 32 MiB the loads are non-temporal (64 MiB: 17.7 vs 19.4 us; 1 GiB:
// 324 vs 342), while up to 32 MiB the source still benefits from the caches
// (32 MiB: 7.9 vs 9.2 us).  A tile-sized buffer resource clamps the ragged
// last tile, so no lane needs a bounds branch.
#include "pc_device.hpp"
#include "pc_launch.hpp"

namespace pcdp {

constexpr int kCopyBlock = 256;

template <int kLoadPolicy, int kStorePolicy>
__global__ __launch_bounds__(kCopyBlock) void k_copy(const u32x4* src, u32x4* dst, size_t nchunks) {
    const size_t first = (size_t)blockIdx.x * kCopyBlock;
    const size_t left = nchunks - first;
    const uint32_t bytes = (uint32_t)(left < kCopyBlock ? left : kCopyBlock) * 16u;
    const uint32_t off = threadIdx.x * 16u;
    const u32x4 v = load16_rsrc<kLoadPolicy>(tile_rsrc(src + first, bytes), off);
    store16_rsrc<kStorePolicy>(tile_rsrc(dst + first, bytes), off, v);
}

hipError_t launch_copy(const void* src, void* dst, size_t nchunks, hipStream_t stream) {
    const u32x4* s = static_cast<const u32x4*>(src);
    u32x4* d = static_cast<u32x4*>(dst);
    const size_t bytes = nchunks * 16;
    const void* k = bytes <= ((size_t)32 << 20) ? (const void*)&k_copy<0, kPolicyDeviceScope>
                                                : (const void*)&k_copy<kPolicyNonTemporal, kPolicyDeviceScope>;
    // At most 2^31 chunks (the largest copy), so the grid stays below 2^23.
    dim3 grid((unsigned)((nchunks + kCopyBlock - 1) / kCopyBlock));
    void* args[] = {&s, &d, &nchunks};
    return hipLaunchKernel(k, grid, dim3(kCopyBlock), args, 0, stream);
}

}  // namespace pcdp
