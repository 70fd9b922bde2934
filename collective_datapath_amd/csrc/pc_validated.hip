// pc_validated.hip -- speculative reduce with a folded validation flag.
//
// "SiFAR: Synchronization-Free All-Reduce for Low-Latency LLM Inference",
// Section 4 (the paragraphs on eliminating flag exchange, on the
// verification logic with Figure 14, and on speculative reduction): instead
// of a barrier before the reduction, every rank writes the call's flag into a
// validation buffer; the consumer reduces the validation buffers next to the
// payload, accepts the result iff the folded flag equals n * flag, and
// otherwise reruns the reduction, re-reading flags and payload past the
// caches.  As on the pages, flags and payload are read in the same attempt
// with no ordering between them; the check is sound when ranks progress
// monotonically (SiFAR, Section 8.1).
//
// Tile b (elems_per_flag elements) is validated by flag word b of every
// rank.  Below a 320 MiB working set each tile has a workgroup of
// elems_per_flag / 8 lanes; from there a persistent grid takes the tiles in
// batches, folding on the LDS-staged pipeline when a tile is that
// pipeline's 16 KiB per rank (8192 elements per flag, four or more ranks).  The retry loop is bounded by max_attempts so every kernel ends;
// attempts[b] receives the attempt that validated (1-based) or 0.
#include "pc_device.hpp"
#include "pc_launch.hpp"
#include "pc_staged.hpp"

#include <type_traits>

namespace pcdp {

constexpr int kBlock = 256;

// One attempt's reads.  The first attempt reads payload and flags the
// default way, so they may come from the caches; a stale cached flag holds
// an earlier call's value, which only makes the check fail.  A retry must
// not be served stale data, so it reads both device-coherently.  Policy and
// scope are template parameters, so each attempt is one straight block of
// loads.
template <int N, int kPolicy>
__device__ __forceinline__ void load_payload(u32x4 (&v)[N], const Ptrs<const u32x4*>& src,
                                             size_t first, uint32_t tile_chunks, uint32_t t) {
#pragma unroll
    for (int r = 0; r < N; ++r) {
        const __amdgpu_buffer_rsrc_t rs = tile_rsrc(src.p[r] + first, tile_chunks * 16u);
        v[r] = load16_rsrc<kPolicy>(rs, t * 16u);
    }
}

template <int N, int kScope>
__device__ __forceinline__ void load_flags(uint32_t (&f)[N], const Ptrs<const uint32_t*>& flags,
                                           uint32_t b) {
#pragma unroll
    for (int r = 0; r < N; ++r) f[r] = __hip_atomic_load(flags.p[r] + b, __ATOMIC_RELAXED, kScope);
}

// The validation fold: the uint32 sum (mod 2^32) of every rank's flag.
template <int N>
__device__ __forceinline__ uint32_t fold_flags(const uint32_t (&f)[N]) {
    uint32_t folded = 0;
#pragma unroll
    for (int r = 0; r < N; ++r) folded += f[r];
    return folded;
}

// One workgroup per tile, one 16-byte chunk per lane: kLanes = elems_per_flag
// / 8 (256, 512, 768 or 1024).  The first attempt is straight-line code, and
// lane 0 issues its flag loads ahead of the payload loads so both are in
// flight together; only a tile that fails the check enters the retry loop.
template <int N, int kLanes>
__global__ __launch_bounds__(kLanes) void k_reduce_validated(Ptrs<const u32x4*> src,
                                                              Ptrs<const uint32_t*> flags,
                                                              u32x4* out, uint32_t flag,
                                                              uint32_t max_attempts,
                                                              uint32_t* attempts) {
    __shared__ uint32_t verdict;
    const uint32_t b = blockIdx.x, t = threadIdx.x;
    const size_t first = (size_t)b * kLanes;
    const uint32_t expect = (uint32_t)N * flag;
    uint32_t f[N];
    u32x4 v[N];
    if (t == 0) load_flags<N, __HIP_MEMORY_SCOPE_WORKGROUP>(f, flags, b);
    load_payload<N, 0>(v, src, first, kLanes, t);
    if (t == 0) verdict = fold_flags<N>(f) == expect;
    __syncthreads();
    uint32_t accepted = 0;
    if (verdict) {
        out[first + t] = fold_chunk<N>(v);
        accepted = 1;
    } else {
        for (uint32_t a = 2; a <= max_attempts; ++a) {
            __syncthreads();  // every wave has read the previous verdict
            if (t == 0) load_flags<N, __HIP_MEMORY_SCOPE_AGENT>(f, flags, b);
            load_payload<N, kPolicyDeviceScope>(v, src, first, kLanes, t);
            if (t == 0) verdict = fold_flags<N>(f) == expect;
            __syncthreads();
            if (verdict) {  // one decision for the whole workgroup
                out[first + t] = fold_chunk<N>(v);
                accepted = a;
                break;
            }
        }
    }
    if (t == 0) attempts[b] = accepted;
}

// Bandwidth regime (working sets of 320 MiB and more): a persistent grid of
// two 256-lane workgroups per CU, the structure of the persistent reduce.
// Workgroup w takes tiles w, w + grid, ... in batches of kBatch; lane t holds
// chunks t, t + 256, ... (U = elems_per_flag / 2048 of them) of each tile.
// Lane j < kBatch loads and folds the flags of the batch's tile j ahead of
// the payload loads, as lane 0 does above.  The folded payload of the whole
// batch waits in registers until a barrier, then every tile that passed the
// check is stored (a failing tile gets a zero-length resource, so the stores
// carry no branch).  A tile that failed then goes through the same bounded
// retry as in the kernel above, one tile at a time.
template <int N, int U>
__global__ __launch_bounds__(kBlock) __attribute__((amdgpu_waves_per_eu(2)))
void k_reduce_validated_persistent(Ptrs<const u32x4*> src, Ptrs<const uint32_t*> flags, u32x4* out,
                                   uint32_t flag, uint32_t max_attempts, uint32_t* attempts,
                                   uint32_t ntiles) {
    // Tiles per batch, from a sweep at 8 ranks x 64 MiB: 16 for one or two
    // chunks per lane, 8 for four (32 chunks, as in the persistent reduce),
    // and 2 for three (the only batch that compiled without spilling).
    constexpr int kBatch = U == 4 ? 8 : (U == 3 ? 2 : 16);
    constexpr uint32_t kTile = kBlock * U;
    static_assert(kBatch <= 32, "one bit per tile of a batch");
    __shared__ uint32_t passed_lds, again_lds;
    const uint32_t t = threadIdx.x, stride = gridDim.x;
    const uint32_t expect = (uint32_t)N * flag;
    for (uint32_t g0 = blockIdx.x; g0 < ntiles; g0 += stride * kBatch) {
        // The first wave checks the batch: bit j of `passed` is set iff tile
        // j exists and its folded flags equal N * flag.
        if (t < 64) {
            bool ok = false;
            const uint32_t g = g0 + t * stride;
            if (t < (uint32_t)kBatch && g < ntiles) {
                uint32_t f[N];
                load_flags<N, __HIP_MEMORY_SCOPE_WORKGROUP>(f, flags, g);
                ok = fold_flags<N>(f) == expect;
            }
            const uint64_t m = __ballot(ok);
            if (t == 0) passed_lds = (uint32_t)m;
        }
        u32x4 o[kBatch][U];
#pragma unroll
        for (int j = 0; j < kBatch; ++j) {
            // A tile past the end gets a zero-length resource: its loads
            // return zero and its stores are dropped.
            const uint32_t g = g0 + j * stride;
            const size_t first = g < ntiles ? (size_t)g * kTile : 0;
            const uint32_t bytes = g < ntiles ? kTile * 16u : 0u;
            u32x4 v[U][N];
#pragma unroll
            for (int r = 0; r < N; ++r) {
                const __amdgpu_buffer_rsrc_t rs = tile_rsrc(src.p[r] + first, bytes);
#pragma unroll
                for (int u = 0; u < U; ++u) v[u][r] = load16_tile(rs, (u * kBlock + t) * 16u);
            }
#pragma unroll
            for (int u = 0; u < U; ++u) o[j][u] = fold_chunk<N>(v[u]);
        }
        __syncthreads();
        // Read through readfirstlane, so the mask, the store resources and
        // every branch on them stay scalar (a value read from LDS is taken as
        // varying across lanes, which would put the resources in vector
        // registers behind a loop over lanes).
        const uint32_t passed = __builtin_amdgcn_readfirstlane(passed_lds);
#pragma unroll
        for (int j = 0; j < kBatch; ++j) {
            const uint32_t g = g0 + j * stride;
            const bool keep = g < ntiles && ((passed >> j) & 1u);
            const __amdgpu_buffer_rsrc_t ro = tile_rsrc(out + (keep ? (size_t)g * kTile : 0),
                                                        keep ? kTile * 16u : 0u);
#pragma unroll
            for (int u = 0; u < U; ++u) store16_tile(ro, (u * kBlock + t) * 16u, o[j][u]);
        }
        if (t < (uint32_t)kBatch && g0 + t * stride < ntiles && ((passed >> t) & 1u)) attempts[g0 + t * stride] = 1;
        // The rare path: retry each failing tile of the batch, one at a time.
        // Every branch below is uniform for the workgroup.
#pragma unroll 1
        for (int j = 0; j < kBatch; ++j) {
            const uint32_t g = g0 + j * stride;
            if (g >= ntiles) break;
            if ((passed >> j) & 1u) continue;
            const size_t first = (size_t)g * kTile;
            uint32_t accepted = 0;
            for (uint32_t a = 2; a <= max_attempts; ++a) {
                __syncthreads();  // every wave has read the previous verdict
                uint32_t f[N] = {};
                if (t == 0) load_flags<N, __HIP_MEMORY_SCOPE_AGENT>(f, flags, g);
                u32x4 v[U][N];
#pragma unroll
                for (int r = 0; r < N; ++r) {
                    const __amdgpu_buffer_rsrc_t rs = tile_rsrc(src.p[r] + first, kTile * 16u);
#pragma unroll
                    for (int u = 0; u < U; ++u)
                        v[u][r] = load16_rsrc<kPolicyDeviceScope>(rs, (u * kBlock + t) * 16u);
                }
                if (t == 0) again_lds = fold_flags<N>(f) == expect;
                __syncthreads();
                if (__builtin_amdgcn_readfirstlane(again_lds)) {
                    const __amdgpu_buffer_rsrc_t ro = tile_rsrc(out + first, kTile * 16u);
#pragma unroll
                    for (int u = 0; u < U; ++u) store16_tile(ro, (u * kBlock + t) * 16u, fold_chunk<N>(v[u]));
                    accepted = a;
                    break;
                }
            }
            if (t == 0) attempts[g] = accepted;
        }
        __syncthreads();  // passed_lds is rewritten by the next batch
    }
}

// Bandwidth regime with 8192 elements per flag and four or more ranks: a
// tile is then 16 KiB per rank, the tile of the LDS-staged pipeline in
// pc_staged.hpp, so the payload is folded by that pipeline (one workgroup
// per CU, batches of 8, 4, 2 and 1 tiles, on the diagonal for rank buffers
// whose bases agree modulo 32 KiB).  The first wave checks the batch's
// flags while the stages fill; after the barrier every row of a tile that
// passed is stored (a failing tile gets a zero-length resource) and failing
// tiles go through the bounded retry one at a time, as above.  Lane t of
// wave w holds chunk 256u + 64w + t of a tile in both paths.  At 64 MiB per
// rank, against the register-batched kernel above, interleaved in a graph:
// 8 ranks 90.1 - 90.3 vs 91.9 - 92.0 us, 4 ranks 50.9 - 51.1 vs 51.4.
template <int N, bool kDiagonal>
__global__ __launch_bounds__(kStageBlock) __attribute__((amdgpu_waves_per_eu(1, 1)))
void k_reduce_validated_staged(Ptrs<const u32x4*> src, Ptrs<const uint32_t*> flags, u32x4* out,
                               uint32_t flag, uint32_t max_attempts, uint32_t* attempts,
                               uint32_t ntiles) {
    static_assert(N >= kStageMinRanks, "staged fold shape");
    constexpr int U = 4;
    constexpr uint32_t kTile = kStageTileChunks;
    PC_STAGE_ARRAYS(N)
    __shared__ uint32_t passed_lds, again_lds;
    const uint32_t t = threadIdx.x, lane = t & (kWave - 1), w = t / kWave, stride = gridDim.x;
    const uint32_t expect = (uint32_t)N * flag;
    for_each_stage_batch([&](auto tiles, uint32_t g0) {
        constexpr int kTiles = decltype(tiles)::value;
        // Every tile of a batch exists (the batches are cut to the tiles left).
        if (t < kWave) {
            bool ok = false;
            if (t < (uint32_t)kTiles) {
                uint32_t f[N];
                load_flags<N, __HIP_MEMORY_SCOPE_WORKGROUP>(f, flags, g0 + t * stride);
                ok = fold_flags<N>(f) == expect;
            }
            const uint64_t m = __ballot(ok);
            if (t == 0) passed_lds = (uint32_t)m;
        }
        StageTile tile[kTiles];
#pragma unroll
        for (int j = 0; j < kTiles; ++j) tile[j] = {(size_t)(g0 + j * stride) * kTile, kTile * 16u};
        std::conditional_t<kDiagonal, DiagonalBatch<N, kTiles>, StagedBatch<N, false, kTiles>> b{
            src, tile, {PC_STAGE_LIST}, w, lane};
        b.run();
        __syncthreads();
        const uint32_t passed = __builtin_amdgcn_readfirstlane(passed_lds);
#pragma unroll
        for (int j = 0; j < 4 * kTiles; ++j) {
            const StageTile tl = tile[j / 4];
            const bool keep = (passed >> (j / 4)) & 1u;
            store16_tile(tile_rsrc(out + tl.first, keep ? tl.bytes : 0u), stage_row_offset(j, w, lane), b.res[j]);
        }
        if (t < (uint32_t)kTiles && ((passed >> t) & 1u)) attempts[g0 + t * stride] = 1;
        // The rare path: retry each failing tile, one at a time.  Every
        // branch below is uniform for the workgroup.
#pragma unroll 1
        for (int j = 0; j < kTiles; ++j) {
            if ((passed >> j) & 1u) continue;
            const uint32_t g = g0 + j * stride;
            const size_t first = (size_t)g * kTile;
            uint32_t accepted = 0;
            for (uint32_t a = 2; a <= max_attempts; ++a) {
                __syncthreads();  // every wave has read the previous verdict
                uint32_t f[N] = {};
                if (t == 0) load_flags<N, __HIP_MEMORY_SCOPE_AGENT>(f, flags, g);
                u32x4 v[U][N];
#pragma unroll
                for (int r = 0; r < N; ++r) {
                    const __amdgpu_buffer_rsrc_t rs = tile_rsrc(src.p[r] + first, kTile * 16u);
#pragma unroll
                    for (int u = 0; u < U; ++u)
                        v[u][r] = load16_rsrc<kPolicyDeviceScope>(rs, (u * kStageBlock + t) * 16u);
                }
                if (t == 0) again_lds = fold_flags<N>(f) == expect;
                __syncthreads();
                if (__builtin_amdgcn_readfirstlane(again_lds)) {
                    const __amdgpu_buffer_rsrc_t ro = tile_rsrc(out + first, kTile * 16u);
#pragma unroll
                    for (int u = 0; u < U; ++u) store16_tile(ro, (u * kStageBlock + t) * 16u, fold_chunk<N>(v[u]));
                    accepted = a;
                    break;
                }
            }
            if (t == 0) attempts[g] = accepted;
        }
        __syncthreads();  // passed_lds is rewritten by the next batch
    }, ntiles);
}

template <int N, int kLanes>
static hipError_t go_validated(Ptrs<const u32x4*> s, Ptrs<const uint32_t*> f, u32x4* out,
                               uint32_t flag, uint32_t max_attempts, uint32_t* attempts,
                               size_t tiles, hipStream_t stream) {
    void* args[] = {&s, &f, &out, &flag, &max_attempts, &attempts};
    return hipLaunchKernel((const void*)&k_reduce_validated<N, kLanes>, dim3((unsigned)tiles),
                           dim3(kLanes), args, 0, stream);
}

template <int N>
static hipError_t go_validated_u(int u, Ptrs<const u32x4*> s, Ptrs<const uint32_t*> f, u32x4* out,
                                 uint32_t flag, uint32_t max_attempts, uint32_t* attempts,
                                 size_t tiles, hipStream_t stream) {
    switch (u) {
        case 1: return go_validated<N, 256>(s, f, out, flag, max_attempts, attempts, tiles, stream);
        case 2: return go_validated<N, 512>(s, f, out, flag, max_attempts, attempts, tiles, stream);
        case 3: return go_validated<N, 768>(s, f, out, flag, max_attempts, attempts, tiles, stream);
        case 4: return go_validated<N, 1024>(s, f, out, flag, max_attempts, attempts, tiles, stream);
        default: return hipErrorInvalidValue;
    }
}

template <int N, int U>
static hipError_t go_validated_persistent(Ptrs<const u32x4*> s, Ptrs<const uint32_t*> f, u32x4* out,
                                          uint32_t flag, uint32_t max_attempts, uint32_t* attempts,
                                          size_t tiles, hipStream_t stream) {
    // Whole rounds of at most two workgroups per CU, then as few workgroups
    // as give that many rounds.
    uint32_t ntiles = (uint32_t)tiles;
    const uint32_t slots = 2 * device_cus();
    const uint32_t rounds = (ntiles + slots - 1) / slots;
    const uint32_t grid = (ntiles + rounds - 1) / rounds;
    void* args[] = {&s, &f, &out, &flag, &max_attempts, &attempts, &ntiles};
    return hipLaunchKernel((const void*)&k_reduce_validated_persistent<N, U>, dim3(grid), dim3(kBlock),
                           args, 0, stream);
}

template <int N>
static hipError_t go_validated_staged(Ptrs<const u32x4*> s, Ptrs<const uint32_t*> f, u32x4* out,
                                      uint32_t flag, uint32_t max_attempts, uint32_t* attempts,
                                      size_t tiles, hipStream_t stream) {
    // Whole rounds of one workgroup per CU, then as few workgroups as give
    // that many rounds (at most one per tile).
    uint32_t ntiles = (uint32_t)tiles;
    const uint32_t cus = device_cus();
    const uint32_t rounds = (ntiles + cus - 1) / cus;
    const uint32_t grid = (ntiles + rounds - 1) / rounds;
    const void* k = bases_congruent((const void* const*)s.p, N) ? (const void*)&k_reduce_validated_staged<N, true>
                                                                : (const void*)&k_reduce_validated_staged<N, false>;
    void* args[] = {&s, &f, &out, &flag, &max_attempts, &attempts, &ntiles};
    return hipLaunchKernel(k, dim3(grid), dim3(kStageBlock), args, stage_pad_bytes<N>(), stream);
}

template <int N>
static hipError_t go_validated_persistent_u(int u, Ptrs<const u32x4*> s, Ptrs<const uint32_t*> f,
                                            u32x4* out, uint32_t flag, uint32_t max_attempts,
                                            uint32_t* attempts, size_t tiles, hipStream_t stream) {
    if constexpr (N >= kStageMinRanks)
        if (u == 4) return go_validated_staged<N>(s, f, out, flag, max_attempts, attempts, tiles, stream);
    switch (u) {
        case 1: return go_validated_persistent<N, 1>(s, f, out, flag, max_attempts, attempts, tiles, stream);
        case 2: return go_validated_persistent<N, 2>(s, f, out, flag, max_attempts, attempts, tiles, stream);
        case 3: return go_validated_persistent<N, 3>(s, f, out, flag, max_attempts, attempts, tiles, stream);
        case 4: return go_validated_persistent<N, 4>(s, f, out, flag, max_attempts, attempts, tiles, stream);
        default: return go_validated_u<N>(u, s, f, out, flag, max_attempts, attempts, tiles, stream);
    }
}

hipError_t launch_reduce_validated(const void* const* src, const void* const* flags, int n,
                                   void* out, size_t k, size_t elems_per_flag, uint32_t flag,
                                   uint32_t max_attempts, void* attempts, hipStream_t stream) {
    Ptrs<const u32x4*> s;
    Ptrs<const uint32_t*> f;
    for (int r = 0; r < kMaxRanks; ++r) {
        s.p[r] = r < n ? static_cast<const u32x4*>(src[r]) : nullptr;
        f.p[r] = r < n ? static_cast<const uint32_t*>(flags[r]) : nullptr;
    }
    u32x4* o = static_cast<u32x4*>(out);
    uint32_t* at = static_cast<uint32_t*>(attempts);
    const int u = (int)(elems_per_flag / 2048);
    const size_t tiles = k / elems_per_flag;
    // Inputs read plus the result written.  From 320 MiB the persistent kernel
    // is ahead (8 ranks, one flag per 8192 elements: 60 vs 72 us at 40 MiB per
    // rank = 360 MiB, 92 vs 116 us at 64 MiB); below it the one-tile kernel is
    // (50 vs 53 us at 32 MiB = 288 MiB, 14 vs 30 us at 8 MiB, where most
    // batches are part-empty).
    if ((size_t)(n + 1) * k * 2 >= ((size_t)320 << 20)) {
        switch (n) {
            case 1: return go_validated_persistent_u<1>(u, s, f, o, flag, max_attempts, at, tiles, stream);
            case 2: return go_validated_persistent_u<2>(u, s, f, o, flag, max_attempts, at, tiles, stream);
            case 3: return go_validated_persistent_u<3>(u, s, f, o, flag, max_attempts, at, tiles, stream);
            case 4: return go_validated_persistent_u<4>(u, s, f, o, flag, max_attempts, at, tiles, stream);
            case 5: return go_validated_persistent_u<5>(u, s, f, o, flag, max_attempts, at, tiles, stream);
            case 6: return go_validated_persistent_u<6>(u, s, f, o, flag, max_attempts, at, tiles, stream);
            case 7: return go_validated_persistent_u<7>(u, s, f, o, flag, max_attempts, at, tiles, stream);
            case 8: return go_validated_persistent_u<8>(u, s, f, o, flag, max_attempts, at, tiles, stream);
            default: return hipErrorInvalidValue;
        }
    }
    switch (n) {
        case 1: return go_validated_u<1>(u, s, f, o, flag, max_attempts, at, tiles, stream);
        case 2: return go_validated_u<2>(u, s, f, o, flag, max_attempts, at, tiles, stream);
        case 3: return go_validated_u<3>(u, s, f, o, flag, max_attempts, at, tiles, stream);
        case 4: return go_validated_u<4>(u, s, f, o, flag, max_attempts, at, tiles, stream);
        case 5: return go_validated_u<5>(u, s, f, o, flag, max_attempts, at, tiles, stream);
        case 6: return go_validated_u<6>(u, s, f, o, flag, max_attempts, at, tiles, stream);
        case 7: return go_validated_u<7>(u, s, f, o, flag, max_attempts, at, tiles, stream);
        case 8: return go_validated_u<8>(u, s, f, o, flag, max_attempts, at, tiles, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace pcdp
