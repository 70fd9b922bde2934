// pc_linked.hip -- single-launch twoshot whose two phases are linked per tile
// by epoch-stamped readiness flags, with the epoch kept on the device.
//
// "flash-comm: Self-Synchronizing Collective Communication for LLM
// Decoding", Section 4.3 (sharded two-hop: readiness checks join the
// reduce-scatter and the result distribution tile by tile, so a finished
// owner tile is distributed while other tiles are still being reduced) and
// Section 4.2 (each thread group derives its state from a call counter kept
// on the device, because launch arguments are frozen once a graph is
// captured; one family runs on one fixed grid so that the counters stay in
// step; every rank issues the same sequence of calls).  "Purlin: Separating
// Orchestration from the Datapath of Collectives", Section 4.2 (every
// thread block keeps a persistent epoch that it advances after each call,
// and that epoch is the value a producer writes to signal readiness) and
// Section 3.2 (the consumer waits on the notification, then moves the data).
//
// Workspace (caller-owned, zero before its first use, uint64 words):
//   [0, G)          call counter of workgroup w (G = kLinkGroups)
//   [G]             number of tiles whose wait gave up (sticky)
//   [G + 1]         polls per wait before giving up; 0 = kMaxPolls
//   [G + 64, ...)   flag of tile t: the epoch of the call that last
//                   finished reducing it
// Workgroup w runs call number ctr[w] + 1 as its epoch and stores it back
// when it is done.  Every call launches all G workgroups, so all counters
// agree and a stale flag (an earlier epoch, or zero) never equals the
// current one; no flag has to be cleared between calls, and a graph replay
// advances the epoch by itself.  Epochs are 64-bit, so they never wrap.
//
// Tile t = (slice s, tile j of the slice) covers up to 256*U chunks of 16
// bytes of slice s.  Phase 1: workgroup t mod G folds tile t from the n
// inputs into outs[s] (the owner's copy), at 4 MiB per rank and above with
// four or more ranks through the LDS stages of pc_staged.hpp; once all of
// its tiles are stored it publishes their flags behind one release at agent
// scope.  Phase 2:
// workgroup (t + G/2) mod G waits for the flags of its tiles, acquires once
// at agent scope, reads each owner tile and writes it to every other
// outs[r].  Every workgroup finishes phase 1 before it waits on any flag,
// and the grid is small enough to be resident at once (checked before
// launch), so every awaited flag is eventually published.  The wait is
// still bounded: a workgroup that gives up adds the number of its tiles to
// the status word and skips them, so the kernel always ends.
//
// Measured floor (one MI355X, 8 ranks, per call inside a graph): the
// cross-workgroup hand-off costs more than a kernel boundary.  At 8 KiB per
// rank this kernel takes 4.6 us, 4.2 us with its fences removed (timing
// only), against 3.5 us for the two-launch form and 1.9 us for the
// single-launch form without flags; at 1 MiB, 8.0 / 6.8 against 4.9 / 3.4.
// A grid sized to the tile count with one device epoch advanced by the last
// workgroup to finish was slower still (5.0 us at 8 KiB, 8.9 at 1 MiB).
//
// Built with PC_LINKED_DELAY_STRESS defined (a test-only variant), every
// wave sleeps a pseudo-random time, seeded by workgroup, wave and epoch,
// before its phase-1 stores, before the flags are published and before its
// phase-2 reads, so that the flag hand-off is exercised at timings the
// natural schedule does not produce.
#include "pc_device.hpp"
#include "pc_launch.hpp"
#include "pc_staged.hpp"

#include <atomic>

namespace pcdp {

constexpr int kLinkBlock = 256;
constexpr uint32_t kMaxPolls = 1u << 20;
constexpr uint32_t kLinkPollLimitWord = 1;  // after the status word

// Pseudo-random sleep of up to ~0.15 ms in the stress variant; nothing
// otherwise.
__device__ __forceinline__ void stress_delay(uint64_t epoch, uint32_t who, uint32_t where) {
#ifdef PC_LINKED_DELAY_STRESS
    uint32_t x = (uint32_t)epoch * 0x9E3779B1u ^ who * 0x85EBCA77u ^ where * 0xC2B2AE3Du;
    x ^= x >> 15;
    x *= 0x2C1B3C6Du;
    x ^= x >> 13;
    for (uint32_t i = x % 48u; i; --i) __builtin_amdgcn_s_sleep(127);
#else
    (void)epoch;
    (void)who;
    (void)where;
#endif
}

// kStaged (tiles of 1024 chunks, four or more ranks): phase 1 runs the
// LDS-staged fold of pc_staged.hpp, which fits this kernel's shape of one
// 256-lane workgroup per CU; kDiagonal: with the ranks on a diagonal
// (rank buffers whose bases agree modulo 32 KiB, as for the reduce).
template <int N, int U, bool kStream, bool kNtCopies, bool kStaged, bool kDiagonal = false>
__global__ __launch_bounds__(kLinkBlock) void k_twoshot_linked(Ptrs<const u32x4*> src,
                                                                Ptrs<u32x4*> outs, uint64_t* ws,
                                                                uint64_t* status,
                                                                size_t slice_chunks,
                                                                size_t tiles_per_slice) {
    constexpr uint32_t kTile = kLinkBlock * U;  // chunks per tile
    constexpr int kLoadPolicy = kStream ? kPolicyNonTemporal : 0;
    __shared__ uint64_t shared_epoch;
    __shared__ uint32_t shared_limit, ready;
    const uint32_t w = blockIdx.x, tid = threadIdx.x;
    uint64_t* const ctr = ws;
    uint64_t* const flags = ws + kLinkGroups + kLinkHeaderWords;

    if (tid == 0) {
        shared_epoch = ctr[w] + 1u;
        const uint64_t limit = ws[kLinkGroups + kLinkPollLimitWord];
        shared_limit = limit == 0 || limit > kMaxPolls ? kMaxPolls : (uint32_t)limit;
    }
    __syncthreads();
    const uint64_t epoch = shared_epoch;
    const size_t ntiles = (size_t)N * tiles_per_slice;

    // ---- phase 1: fold this workgroup's owner tiles, then publish them -----------
    // One release per workgroup: after the barrier, lane 0's agent-scope fence
    // orders every wave's stores before the flags (the barrier-then-lane-0
    // pattern of a grid-wide barrier).  Fences are few on purpose: each one
    // writes back or invalidates a whole L2 and they queue up per XCD.
    if (w < ntiles) {
        if constexpr (kStaged) {
            static_assert(kTile == kStageTileChunks && N >= kStageMinRanks, "staged tile shape");
            PC_STAGE_ARRAYS(N)
            const uint32_t lane = tid & (kWave - 1), wave = tid / kWave;
            for_each_stage_batch([&](auto tiles, uint32_t g0) {
                constexpr int kTiles = decltype(tiles)::value;
                StageTile tile[kTiles];
                uint32_t slice[kTiles];
#pragma unroll
                for (int j = 0; j < kTiles; ++j) {
                    const size_t t = g0 + (size_t)j * kLinkGroups;
                    const size_t s = t / tiles_per_slice;
                    const SliceTile st = slice_tile((uint32_t)s, (uint32_t)(t % tiles_per_slice), slice_chunks, kTile);
                    tile[j] = {st.first, st.chunks * 16u};
                    slice[j] = (uint32_t)s;
                }
                std::conditional_t<kDiagonal, DiagonalBatch<N, kTiles>, StagedBatch<N, false, kTiles>> b{
                    src, tile, {PC_STAGE_LIST}, wave, lane};
                b.run();
                __syncthreads();
                stress_delay(epoch, w * 4 + wave, g0);
#pragma unroll
                for (int j = 0; j < 4 * kTiles; ++j) {
                    const StageTile tl = tile[j / 4];
                    store16_tile(tile_rsrc(outs.p[slice[j / 4]] + tl.first, tl.bytes), stage_row_offset(j, wave, lane),
                                 b.res[j]);
                }
            }, (uint32_t)ntiles);
        } else {
            for (size_t t = w; t < ntiles; t += kLinkGroups) {
                const size_t s = t / tiles_per_slice;
                const SliceTile st = slice_tile((uint32_t)s, (uint32_t)(t % tiles_per_slice), slice_chunks, kTile);
                const size_t c0 = st.first;
                const uint32_t bytes = st.chunks * 16u;
                u32x4 v[U][N];
#pragma unroll
                for (int r = 0; r < N; ++r) {
                    const __amdgpu_buffer_rsrc_t rs = tile_rsrc(src.p[r] + c0, bytes);
#pragma unroll
                    for (int u = 0; u < U; ++u)
                        v[u][r] = load16_rsrc<kLoadPolicy>(rs, (u * kLinkBlock + tid) * 16u);
                }
                stress_delay(epoch, w * 4 + tid / kWave, (uint32_t)t);
                const __amdgpu_buffer_rsrc_t ro = tile_rsrc(outs.p[s] + c0, bytes);
#pragma unroll
                for (int u = 0; u < U; ++u) store16_tile(ro, (u * kLinkBlock + tid) * 16u, fold_chunk<N>(v[u]));
            }
        }
        __syncthreads();
        if (tid == 0) {
            stress_delay(epoch, w, 0x10000u);
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
            for (size_t t = w; t < ntiles; t += kLinkGroups)
                __hip_atomic_store(flags + t, epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }

    // ---- phase 2: wait for the flags of this workgroup's tiles, copy them out -----
    // Lane 0 waits for every flag in turn (bounded), acquires once, and the
    // barrier hands the go-ahead to the other waves.  A workgroup that gives
    // up copies none of its tiles and adds their number to the status word.
    const size_t first = (w + kLinkGroups / 2) % kLinkGroups;
    if (first < ntiles) {
        if (tid == 0) {
            const uint32_t limit = shared_limit;
            bool ok = true;
            uint64_t mine = 0;
            for (size_t t = first; t < ntiles; t += kLinkGroups) {
                ++mine;
                uint32_t polls = 0;
                while (ok && __hip_atomic_load(flags + t, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != epoch) {
                    if (++polls >= limit) ok = false;
                    else __builtin_amdgcn_s_sleep(1);
                }
            }
            if (ok) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
            else __hip_atomic_fetch_add(status, mine, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            ready = ok;
        }
        __syncthreads();
        if (ready) {
            stress_delay(epoch, w * 4 + tid / kWave, 0x20000u);
            for (size_t t = first; t < ntiles; t += kLinkGroups) {
                const size_t s = t / tiles_per_slice;
                const SliceTile st = slice_tile((uint32_t)s, (uint32_t)(t % tiles_per_slice), slice_chunks, kTile);
                const size_t c0 = st.first;
                const uint32_t bytes = st.chunks * 16u;
                const __amdgpu_buffer_rsrc_t rs = tile_rsrc(outs.p[s] + c0, bytes);
                u32x4 v[U];
#pragma unroll
                for (int u = 0; u < U; ++u) v[u] = load16_rsrc<0>(rs, (u * kLinkBlock + tid) * 16u);
                // The owner's own range gets a zero-length resource, so its
                // stores are dropped without a branch.
#pragma unroll
                for (int r = 0; r < N; ++r) {
                    const __amdgpu_buffer_rsrc_t rd = tile_rsrc(outs.p[r] + c0, (size_t)r == s ? 0u : bytes);
#pragma unroll
                    for (int u = 0; u < U; ++u) {
                        if constexpr (kNtCopies) store16_rsrc<kPolicyNonTemporal>(rd, (u * kLinkBlock + tid) * 16u, v[u]);
                        else store16_tile(rd, (u * kLinkBlock + tid) * 16u, v[u]);
                    }
                }
            }
        }
    }
    if (tid == 0) ctr[w] = epoch;
}

// Chunks per lane per tile, from a sweep at 8 ranks: one below 512 KiB per
// rank (the most tiles in flight), two below 4 MiB (half the tiles, and
// half the fences, at 1 MiB), four above.
static int linked_unroll(size_t nchunks_slice, int n) {
    const size_t per_rank = nchunks_slice * (size_t)n * 16;
    return per_rank < ((size_t)512 << 10) ? 1 : per_rank < ((size_t)4 << 20) ? 2 : 4;
}

size_t linked_tiles(int n, size_t nchunks_slice) {
    const uint32_t tile = kLinkBlock * linked_unroll(nchunks_slice, n);
    return (size_t)n * slice_tiles(nchunks_slice, (uint32_t)n, tile);
}

// Workgroups of `kernel` that fit on the device at once, cached per device
// and kernel (the answer does not change while the process runs).
static hipError_t resident_capacity(const void* kernel, int* capacity) {
    int dev = 0, cus = 0, per_cu = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, kLinkBlock, 0);
    if (e != hipSuccess) return e;
    *capacity = cus * per_cu;
    return hipSuccess;
}

// Workgroups of kernel K that fit on the current device at once, looked up
// once per device.
template <const void* (*K)()>
static hipError_t cached_capacity(int* cap) {
    // 0 = not yet known, else capacity + 1, per device.
    static std::atomic<int> known[64];
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    *cap = dev >= 0 && dev < 64 ? known[dev].load(std::memory_order_relaxed) - 1 : -1;
    if (*cap < 0) {
        e = resident_capacity(K(), cap);
        if (e != hipSuccess) return e;
        if (dev >= 0 && dev < 64) known[dev].store(*cap + 1, std::memory_order_relaxed);
    }
    return hipSuccess;
}

template <int N, int U, bool kStream, bool kNtCopies, bool kStaged, bool kDiagonal = false>
static const void* linked_kernel() {
    return (const void*)&k_twoshot_linked<N, U, kStream, kNtCopies, kStaged, kDiagonal>;
}

// The staged phase 1 takes over half of a CU's LDS, so only one workgroup of
// it fits per CU: it is launched where the whole grid still fits at once
// (every MI355X CU in one partition), else the kernel that loads into
// registers is.  At 8 ranks, interleaved on one MI355X: 187.9 vs 192.7 us at
// 64 MiB per rank, 144.1 vs 147.2 at 48, 275.8 vs 286.8 at 96; 4 ranks
// 99.2 vs 103.1 at 64 MiB and 29.0 vs 29.9 at 16.
template <int N, int U, bool kStream, bool kNtCopies>
static hipError_t go_linked(Ptrs<const u32x4*> s, Ptrs<u32x4*> o, uint64_t* ws, uint64_t* status,
                            size_t slice_chunks, hipStream_t stream) {
    constexpr bool kCanStage = kStream && U * kLinkBlock == (int)kStageTileChunks && N >= kStageMinRanks;
    int cap = 0;
    const void* kernel = linked_kernel<N, U, kStream, kNtCopies, false>();
    hipError_t e;
    if constexpr (kCanStage) {
        const bool diagonal = bases_congruent((const void* const*)s.p, N);
        e = diagonal ? cached_capacity<linked_kernel<N, U, kStream, kNtCopies, true, true>>(&cap)
                     : cached_capacity<linked_kernel<N, U, kStream, kNtCopies, true, false>>(&cap);
        if (e != hipSuccess) return e;
        if (cap >= (int)kLinkGroups)
            kernel = diagonal ? linked_kernel<N, U, kStream, kNtCopies, true, true>()
                              : linked_kernel<N, U, kStream, kNtCopies, true, false>();
    }
    if (cap < (int)kLinkGroups) {
        e = cached_capacity<linked_kernel<N, U, kStream, kNtCopies, false>>(&cap);
        if (e != hipSuccess) return e;
    }
    if (cap < (int)kLinkGroups) return hipErrorCooperativeLaunchTooLarge;
    size_t tiles_per_slice = slice_tiles(slice_chunks, N, kLinkBlock * U);
    void* args[] = {&s, &o, &ws, &status, &slice_chunks, &tiles_per_slice};
    return hipLaunchKernel(kernel, dim3(kLinkGroups), dim3(kLinkBlock), args, 0, stream);
}

template <int N>
static hipError_t go_linked_n(Ptrs<const u32x4*> s, Ptrs<u32x4*> o, uint64_t* ws, uint64_t* status,
                              size_t slice_chunks, hipStream_t stream) {
    // From 48 MiB per rank the copies carry the non-temporal hint: at 8 ranks
    // 195 vs 218 us at 64 MiB per rank, 286 vs 333 us at 96 MiB and 149 vs
    // 153 us at 48 MiB; below it the default policy is 1-3% faster.
    if (slice_chunks * N * 16 >= ((size_t)48 << 20))
        return go_linked<N, 4, true, true>(s, o, ws, status, slice_chunks, stream);
    switch (linked_unroll(slice_chunks, N)) {
        case 1: return go_linked<N, 1, false, false>(s, o, ws, status, slice_chunks, stream);
        case 2: return go_linked<N, 2, false, false>(s, o, ws, status, slice_chunks, stream);
        default: return go_linked<N, 4, true, false>(s, o, ws, status, slice_chunks, stream);
    }
}

// ---- the same call with its workspace in static device memory --------------------
// For callers that cannot allocate.  `scratch` is this library's workspace
// of fixed size in every GPU's memory (zero when the code object is
// loaded, as every static device variable); host code never uses the
// array's name, only the per-device address hipGetSymbolAddress returns,
// looked up on the first call on each device.  Calls on one device share
// it, so calls that may overlap in time on one device race.
__device__ __align__(256) uint64_t scratch[kStaticScratchBytes / sizeof(uint64_t)];

hipError_t static_workspace(void** ptr) {
    static std::atomic<void*> known[64];
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
    void* p = known[dev].load(std::memory_order_acquire);
    if (!p) {
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        known[dev].store(p, std::memory_order_release);
    }
    *ptr = p;
    return hipSuccess;
}

hipError_t launch_twoshot_linked(const void* const* src, int n, void* const* outs,
                                 size_t nchunks_slice, void* workspace, void* status, hipStream_t stream) {
    Ptrs<const u32x4*> s;
    Ptrs<u32x4*> o;
    for (int r = 0; r < kMaxRanks; ++r) {
        s.p[r] = r < n ? static_cast<const u32x4*>(src[r]) : nullptr;
        o.p[r] = r < n ? static_cast<u32x4*>(outs[r]) : nullptr;
    }
    uint64_t* ws = static_cast<uint64_t*>(workspace);
    uint64_t* st = status ? static_cast<uint64_t*>(status) : ws + kLinkGroups;
    switch (n) {
        case 1: return go_linked_n<1>(s, o, ws, st, nchunks_slice, stream);
        case 2: return go_linked_n<2>(s, o, ws, st, nchunks_slice, stream);
        case 3: return go_linked_n<3>(s, o, ws, st, nchunks_slice, stream);
        case 4: return go_linked_n<4>(s, o, ws, st, nchunks_slice, stream);
        case 5: return go_linked_n<5>(s, o, ws, st, nchunks_slice, stream);
        case 6: return go_linked_n<6>(s, o, ws, st, nchunks_slice, stream);
        case 7: return go_linked_n<7>(s, o, ws, st, nchunks_slice, stream);
        case 8: return go_linked_n<8>(s, o, ws, st, nchunks_slice, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace pcdp
