// pc_sentinel.hip -- sentinel readiness: publish into sentinel-armed storage,
// then validate, fold and re-arm on the consumer side.
//
// "flash-comm: Self-Synchronizing Collective Communication for LLM
// Decoding", Section 3.1 (sentinel readiness: receive storage is prefilled
// with a reserved bit pattern; a producer overwrites it, so a pack that no
// longer holds the pattern has arrived; the consumer restores the pattern
// after capturing the value; a real value equal to the pattern is replaced by
// a canonical quiet NaN before publication, and so are partial sums) and
// Section 4.3 (one-hop: receive slots indexed by source rank, the fold waits
// for every source and resets each slot after capturing it, then folds in
// rank order).
//
// Sentinel: the bf16 pattern 0xFFFF (a NaN).  Readiness unit: a pack of 8
// bf16 = 16 bytes, published with one 16-byte store.  Because every NaN
// result of the fold is narrowed to the canonical 0x7FC0, no fold result can
// equal the sentinel, so results can be republished without a further check.
// The consumer is one kernel up to 768 MiB moved, and from there a fold pass
// and a re-arm pass ordered by the stream.
#include "pc_device.hpp"
#include "pc_launch.hpp"
#include "pc_staged.hpp"

namespace pcdp {

// Bytes per rank below which the publisher takes one chunk per lane.
constexpr size_t kSentinelSmallBytes = (size_t)4 << 20;
constexpr uint32_t kSentinelWord = 0xFFFFFFFFu;  // two sentinel elements

// 1 if neither bf16 half of `w` is the sentinel.  Bitwise, not short
// circuit: the readiness test of a pack combines 4 * N of these, and a
// short-circuit chain compiled to a branch per term.
__device__ __forceinline__ bool no_sentinel(uint32_t w) {
    return ((w & 0xFFFFu) != 0xFFFFu) & ((w >> 16) != 0xFFFFu);
}

// Replace each sentinel half of `w` by the canonical quiet NaN.
__device__ __forceinline__ uint32_t sanitize(uint32_t w) {
    const uint32_t lo = (w & 0xFFFFu) == 0xFFFFu ? 0x7FC0u : (w & 0xFFFFu);
    const uint32_t hi = (w >> 16) == 0xFFFFu ? 0x7FC0u : (w >> 16);
    return lo | (hi << 16);
}

// ---- publish: copy with substitution, 16 bytes per lane ---------------------------
// Device-scope stores through a workgroup-tile resource: eight 128 KiB
// publishes and a consume in a graph took 15.55 vs 16.60 us (the consume's
// own stores measured level either way and keep the default policy).
template <int W, int U>
__global__ __launch_bounds__(W * kWave) void k_publish_sentinel(const u32x4* src, u32x4* dst,
                                                                 size_t nchunks) {
    constexpr int kBlk = W * kWave;
    const size_t tile0 = (size_t)blockIdx.x * (kBlk * U);
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const size_t c = tile0 + u * kBlk + threadIdx.x;
        if (c < nchunks) {
            u32x4 v = src[c];
#pragma unroll
            for (int e = 0; e < 4; ++e) v[e] = sanitize(v[e]);
            store16_rsrc<kPolicyDeviceScope>(tile_rsrc(dst + tile0, kBlk * U * 16u), (uint32_t)(c - tile0) * 16u, v);
        }
    }
}

// From 4 MiB: the Atom copy's shape.  Short-lived workgroups of 256 lanes
// each publish one 4 KiB tile with device-scope stores; above 32 MiB the
// loads are non-temporal.  Against the persistent grid that walked 16 KiB
// tiles, at one rank: 1 GiB 324 vs 360 us, 512 MiB 163 vs 174, 64 MiB 17.9
// vs 19.6 (and 20.6 vs 24.4 with the buffers rotated past the last-level
// cache); against the 8 KiB-per-workgroup kernel above with default
// policies, 32 MiB 7.8 vs 10.2 us and 16 MiB 4.2 vs 4.7.  Publishing in
// place is safe: each lane reads its chunk and then writes that chunk.
template <int kLoadPolicy>
__global__ __launch_bounds__(4 * kWave) void k_publish_sentinel_tile(const u32x4* src, u32x4* dst,
                                                                      size_t nchunks) {
    constexpr uint32_t kTile = 4 * kWave;
    const size_t first = (size_t)blockIdx.x * kTile;
    const size_t left = nchunks - first;
    const uint32_t bytes = (uint32_t)(left < kTile ? left : kTile) * 16u;
    const uint32_t off = threadIdx.x * 16u;
    u32x4 v = load16_rsrc<kLoadPolicy>(tile_rsrc(src + first, bytes), off);
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] = sanitize(v[e]);
    store16_rsrc<kPolicyDeviceScope>(tile_rsrc(dst + first, bytes), off, v);
}

// ---- consume: every wave owns U groups of 64 consecutive packs --------------------
// Lane l of group u takes pack base + 64u + l from every rank's slot; the
// wave's ballot over "no rank holds the sentinel anywhere in the pack" is the
// group's bitmap word.  A ready pack is folded in rank order, stored, and its
// slots are re-armed with the sentinel; other packs are left as they are.
template <int N, int W, int U>
__global__ __launch_bounds__(W * kWave) void k_consume_sentinel(Ptrs<u32x4*> slots, u32x4* out,
                                                                 uint64_t* bitmap, size_t npacks) {
    const uint32_t lane = threadIdx.x & (kWave - 1);
    const uint32_t wave = threadIdx.x / kWave;
    const size_t base = ((size_t)blockIdx.x * W + wave) * (kWave * U);
    if (base >= npacks) return;  // whole wave past the end
    u32x4 v[U][N];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        if (base + (size_t)u * kWave < npacks) {
#pragma unroll
            for (int r = 0; r < N; ++r) v[u][r] = slots.p[r][base + u * kWave + lane];
        }
    }
    const u32x4 armed = {kSentinelWord, kSentinelWord, kSentinelWord, kSentinelWord};
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const size_t g = base + (size_t)u * kWave;
        if (g >= npacks) break;
        bool ready = true;
#pragma unroll
        for (int r = 0; r < N; ++r)
#pragma unroll
            for (int e = 0; e < 4; ++e) ready &= no_sentinel(v[u][r][e]);
        const uint64_t word = __ballot(ready);
        if (ready) {
            out[g + lane] = fold_chunk<N>(v[u]);
#pragma unroll
            for (int r = 0; r < N; ++r) slots.p[r][g + lane] = armed;
        }
        if (lane == 0) bitmap[g / kWave] = word;
    }
}

// ---- consume in two passes, from 768 MiB moved ----------------------------------------
// Pass 1 folds: the LDS-staged persistent fold of pc_staged.hpp over tiles of
// 1024 packs, one workgroup per CU.  Readiness is evaluated per pack as the
// rows leave LDS; the ballot of each 64-pack row is its bitmap word, and a
// wave's 32 words of a batch wait in lanes 0..31 until the batch's store
// phase, where they leave together with the ready results (a pack that is
// not ready gets an out-of-range offset, which its tile's resource drops).
// Pass 2 re-arms: workgroup (x, r) covers 256 packs of slot r, one per lane;
// each wave reads the bitmap word of its 64 packs with a scalar load and
// writes the sentinel over the ready ones with non-temporal stores.  Small
// workgroups keep many short-lived store streams in flight, which HBM
// writes best.  The two passes are ordered by the stream; no pack is
// re-armed before its value is captured.
// At 8 ranks x 64 MiB on one MI355X, interleaved against the previous
// register-batched fold and 1024-pack re-arm blocks: fold 90.7 - 91.3 us
// against 97.6 - 98.6; re-arm 79.0 - 79.5 us against 101.2 - 101.4.
// Device-scope re-arm stores took 75.2 against 79.4 us alone, but left the
// re-armed lines for the next cycle's publishes to write back: eight
// publishes and a consume then took 366 against 357 us.
constexpr uint32_t kSDrop = 0x80000000u;  // past every tile resource

template <int N>
__global__ __launch_bounds__(kStageBlock) __attribute__((amdgpu_waves_per_eu(1, 1)))
void k_sentinel_fold_staged(Ptrs<const u32x4*> slots, u32x4* out, uint64_t* bitmap, size_t npacks,
                            uint32_t ntiles) {
    PC_STAGE_ARRAYS(N)
    const uint32_t lane = threadIdx.x & 63, w = threadIdx.x >> 6, stride = gridDim.x;
    for_each_stage_batch([&](auto tiles, uint32_t g0) {
        constexpr int kTiles = decltype(tiles)::value;
        StageTile tile[kTiles];
#pragma unroll
        for (int j = 0; j < kTiles; ++j) {
            const size_t first = (size_t)(g0 + j * stride) * kStageTileChunks;
            const size_t left = npacks - first;
            tile[j] = {first, (uint32_t)(left < kStageTileChunks ? left : kStageTileChunks) * 16u};
        }
        StagedBatch<N, true, kTiles> b{slots, tile, {PC_STAGE_LIST}, w, lane};
        b.run();
        __syncthreads();
        // Lane j < 4 * kTiles holds the word of row j: tile j / 4, row j % 4,
        // i.e. word 16 * g + 4 * (j % 4) + w.  Packs come in whole 64-pack
        // words, so a word is either wholly inside npacks or wholly outside,
        // and a resource over the whole bitmap drops the words past its end.
        // (A branch around this store instead made the compiler spill the
        // batch's results.)
        {
            const uint32_t g = g0 + (lane / 4) * stride;
            const uint32_t word = g * 16 + (lane % 4) * 4 + w;
            const __amdgpu_buffer_rsrc_t rb = tile_rsrc(bitmap, (uint32_t)(npacks / kWave) * 8u);
            u32x2 words;
            words[0] = b.words_lo;
            words[1] = b.words_hi;
            __builtin_amdgcn_raw_buffer_store_b64(words, rb, lane < 4u * kTiles ? word * 8u : kSDrop, 0,
                                                  kPolicyDeviceScope);
        }
#pragma unroll
        for (int j = 0; j < 4 * kTiles; ++j) {
            const StageTile t = tile[j / 4];
            const __amdgpu_buffer_rsrc_t ro = tile_rsrc(out + t.first, t.bytes);
            const bool ready = (b.ready_bits >> j) & 1u;
            store16_tile(ro, ready ? stage_row_offset(j, w, lane) : kSDrop, b.res[j]);
        }
    }, ntiles);
}

// Pass 2.  Grid: x = block of 256 packs, y = slot r.
constexpr uint32_t kRearmPacks = 256;
__global__ __launch_bounds__(4 * kWave) void k_sentinel_rearm(Ptrs<u32x4*> slots, const uint64_t* bitmap,
                                                              size_t npacks) {
    const uint32_t lane = threadIdx.x & (kWave - 1);
    const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const size_t group = (size_t)blockIdx.x * 4 + wave;  // this wave's 64 packs = bitmap word
    if (group * kWave >= npacks) return;                 // wave past the end
    const __attribute__((address_space(4))) uint64_t* words =
        (const __attribute__((address_space(4))) uint64_t*)bitmap;
    const uint64_t word = words[group];
    const bool ready = (word >> lane) & 1u;
    const __amdgpu_buffer_rsrc_t rs = tile_rsrc(slots.p[blockIdx.y] + group * kWave, kWave * 16u);
    const u32x4 armed = {kSentinelWord, kSentinelWord, kSentinelWord, kSentinelWord};
    store16_rsrc<kPolicyNonTemporal>(rs, ready ? lane * 16u : kSDrop, armed);
}

template <int W, int U>
static hipError_t go_publish(const u32x4* s, u32x4* d, size_t nchunks, hipStream_t stream) {
    const size_t tile = (size_t)W * kWave * U;
    dim3 grid((unsigned)((nchunks + tile - 1) / tile));
    void* args[] = {&s, &d, &nchunks};
    return hipLaunchKernel((const void*)&k_publish_sentinel<W, U>, grid, dim3(W * kWave), args, 0,
                           stream);
}

hipError_t launch_publish_sentinel(const void* src, void* dst, size_t nchunks, hipStream_t stream) {
    const u32x4* s = static_cast<const u32x4*>(src);
    u32x4* d = static_cast<u32x4*>(dst);
    if (nchunks * 16 < kSentinelSmallBytes) return go_publish<4, 1>(s, d, nchunks, stream);
    const void* k = nchunks * 16 <= ((size_t)32 << 20) ? (const void*)&k_publish_sentinel_tile<0>
                                                       : (const void*)&k_publish_sentinel_tile<kPolicyNonTemporal>;
    // At most 2^31 chunks, so the grid stays below 2^23.
    dim3 grid((unsigned)((nchunks + 4 * kWave - 1) / (4 * kWave)));
    void* args[] = {&s, &d, &nchunks};
    return hipLaunchKernel(k, grid, dim3(4 * kWave), args, 0, stream);
}

template <int N, int W, int U>
static hipError_t go_consume_sentinel_shape(Ptrs<u32x4*> p, u32x4* out, uint64_t* bitmap,
                                            size_t npacks, hipStream_t stream) {
    const size_t per_block = (size_t)W * kWave * U;
    dim3 grid((unsigned)((npacks + per_block - 1) / per_block));
    void* args[] = {&p, &out, &bitmap, &npacks};
    return hipLaunchKernel((const void*)&k_consume_sentinel<N, W, U>, grid, dim3(W * kWave), args, 0,
                           stream);
}

template <int N>
static hipError_t go_consume_sentinel_two_pass(Ptrs<u32x4*> p, u32x4* out, uint64_t* bitmap,
                                               size_t npacks, hipStream_t stream) {
    uint32_t ntiles = (uint32_t)((npacks + kStageTileChunks - 1) / kStageTileChunks);
    const uint32_t cus = device_cus();
    const uint32_t rounds = (ntiles + cus - 1) / cus;
    const uint32_t grid = (ntiles + rounds - 1) / rounds;
    Ptrs<const u32x4*> cp;
    for (int r = 0; r < kMaxRanks; ++r) cp.p[r] = p.p[r];
    void* args[] = {&cp, &out, &bitmap, &npacks, &ntiles};
    hipError_t e = hipLaunchKernel((const void*)&k_sentinel_fold_staged<N>, dim3(grid), dim3(kStageBlock), args,
                                   stage_pad_bytes<N>(), stream);
    if (e != hipSuccess) return e;
    dim3 rgrid((unsigned)((npacks + kRearmPacks - 1) / kRearmPacks), (unsigned)N);
    const uint64_t* b = bitmap;
    void* rargs[] = {&p, &b, &npacks};
    return hipLaunchKernel((const void*)&k_sentinel_rearm, rgrid, dim3(4 * kWave), rargs, 0, stream);
}

template <int N>
static hipError_t go_consume_sentinel(Ptrs<u32x4*> p, u32x4* out, uint64_t* bitmap, size_t npacks,
                                      hipStream_t stream) {
    // Slots read plus results and re-arms written.  From 768 MiB, three times
    // the last-level cache, the two passes are faster (8 ranks: 197 vs 226 us
    // at 64 MiB per rank, 147 vs 165 at 48, 294 vs 333 at 96); below it the
    // single kernel keeps more in the caches (101 vs 104 us at 32 MiB) and a
    // second launch costs more than it saves at decode sizes.
    if (npacks * 16 * (2 * (size_t)N + 1) >= ((size_t)768 << 20))
        return go_consume_sentinel_two_pass<N>(p, out, bitmap, npacks, stream);
    return go_consume_sentinel_shape<N, 4, 1>(p, out, bitmap, npacks, stream);
}

hipError_t launch_consume_sentinel(void* const* slots, int n, void* out, size_t npacks,
                                   void* bitmap, hipStream_t stream) {
    Ptrs<u32x4*> p;
    for (int r = 0; r < kMaxRanks; ++r) p.p[r] = r < n ? static_cast<u32x4*>(slots[r]) : nullptr;
    u32x4* o = static_cast<u32x4*>(out);
    uint64_t* b = static_cast<uint64_t*>(bitmap);
    switch (n) {
        case 1: return go_consume_sentinel<1>(p, o, b, npacks, stream);
        case 2: return go_consume_sentinel<2>(p, o, b, npacks, stream);
        case 3: return go_consume_sentinel<3>(p, o, b, npacks, stream);
        case 4: return go_consume_sentinel<4>(p, o, b, npacks, stream);
        case 5: return go_consume_sentinel<5>(p, o, b, npacks, stream);
        case 6: return go_consume_sentinel<6>(p, o, b, npacks, stream);
        case 7: return go_consume_sentinel<7>(p, o, b, npacks, stream);
        case 8: return go_consume_sentinel<8>(p, o, b, npacks, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace pcdp
