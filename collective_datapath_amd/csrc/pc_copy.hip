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
// Shapes follow the reduce kernels: one workgroup per tile of 256*U chunks
// for cache-resident payloads, and for working sets of 64 MiB or more a
// persistent grid of two workgroups per CU whose workgroups load a batch of
// 16 KiB tiles, pass a barrier, and then store the batch.  Unlike the
// reduce's 8:1 mix, this 1:1 stream is fastest with one tile per batch
// (256 MiB: 75.1 us with 1 tile, 76.7 with 2, 77.2 with 4, 78.7 with 8 and
// 91.2 us for one workgroup per tile).  Tile-sized buffer resources clamp
// every ragged tile, so no lane needs a bounds branch.
#include "pc_device.hpp"
#include "pc_launch.hpp"

namespace pcdp {

constexpr int kCopyBlock = 256;

template <int U>
__global__ __launch_bounds__(kCopyBlock) void k_copy(const u32x4* src, u32x4* dst, size_t nchunks) {
    constexpr uint32_t kTile = kCopyBlock * U;
    const size_t first = (size_t)blockIdx.x * kTile;
    const size_t left = nchunks - first;
    const uint32_t bytes = (uint32_t)(left < kTile ? left : kTile) * 16u;
    const uint32_t t = threadIdx.x;
    const __amdgpu_buffer_rsrc_t rs = tile_rsrc(src + first, bytes);
    const __amdgpu_buffer_rsrc_t rd = tile_rsrc(dst + first, bytes);
    u32x4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = load16_rsrc<0>(rs, (u * kCopyBlock + t) * 16u);
#pragma unroll
    for (int u = 0; u < U; ++u) store16_rsrc<0>(rd, (u * kCopyBlock + t) * 16u, v[u]);
}

// Bandwidth regime.  Workgroup w takes tiles w, w + grid, ... in batches of
// kBatch; tile g covers chunks [g*1024, (g+1)*1024) clamped to nchunks.
template <int kBatch>
__global__ __launch_bounds__(kCopyBlock) __attribute__((amdgpu_waves_per_eu(2)))
void k_copy_persistent(const u32x4* src, u32x4* dst, size_t nchunks, uint32_t ntiles) {
    constexpr int U = 4;
    constexpr uint32_t kTile = kCopyBlock * U;
    const uint32_t t = threadIdx.x, stride = gridDim.x;
    for (uint32_t g0 = blockIdx.x; g0 < ntiles; g0 += stride * kBatch) {
        u32x4 v[kBatch][U];
#pragma unroll
        for (int j = 0; j < kBatch; ++j) {
            const uint32_t g = g0 + j * stride;
            const size_t first = (size_t)g * kTile;
            // A tile past the end gets a zero-length resource: its loads
            // return zero and its stores are dropped.
            const size_t left = g < ntiles ? nchunks - first : 0;
            const uint32_t bytes = (uint32_t)(left < kTile ? left : kTile) * 16u;
            const __amdgpu_buffer_rsrc_t rs = tile_rsrc(src + (g < ntiles ? first : 0), bytes);
#pragma unroll
            for (int u = 0; u < U; ++u) v[j][u] = load16_rsrc<kPolicyNonTemporal>(rs, (u * kCopyBlock + t) * 16u);
        }
        __syncthreads();
#pragma unroll
        for (int j = 0; j < kBatch; ++j) {
            const uint32_t g = g0 + j * stride;
            const size_t first = (size_t)g * kTile;
            const size_t left = g < ntiles ? nchunks - first : 0;
            const uint32_t bytes = (uint32_t)(left < kTile ? left : kTile) * 16u;
            const __amdgpu_buffer_rsrc_t rd = tile_rsrc(dst + (g < ntiles ? first : 0), bytes);
#pragma unroll
            for (int u = 0; u < U; ++u) store16_rsrc<kPolicyDeviceScope>(rd, (u * kCopyBlock + t) * 16u, v[j][u]);
        }
    }
}

hipError_t launch_copy(const void* src, void* dst, size_t nchunks, hipStream_t stream) {
    const u32x4* s = static_cast<const u32x4*>(src);
    u32x4* d = static_cast<u32x4*>(dst);
    if (nchunks * 16 * 2 >= ((size_t)64 << 20)) {
        constexpr int kBatch = 1;
        constexpr uint32_t kTile = kCopyBlock * 4;
        uint32_t ntiles = (uint32_t)((nchunks + kTile - 1) / kTile);
        const uint32_t slots = 2 * device_cus();
        const uint32_t rounds = (ntiles + slots - 1) / slots;
        const uint32_t grid = (ntiles + rounds - 1) / rounds;
        void* args[] = {&s, &d, &nchunks, &ntiles};
        return hipLaunchKernel((const void*)&k_copy_persistent<kBatch>, dim3(grid), dim3(kCopyBlock),
                               args, 0, stream);
    }
    const int u = nchunks * 16 < ((size_t)4 << 20) ? 1 : 4;
    const size_t tile = (size_t)kCopyBlock * u;
    dim3 grid((unsigned)((nchunks + tile - 1) / tile));
    void* args[] = {&s, &d, &nchunks};
    return hipLaunchKernel(u == 1 ? (const void*)&k_copy<1> : (const void*)&k_copy<4>, grid,
                           dim3(kCopyBlock), args, 0, stream);
}

}  // namespace pcdp
