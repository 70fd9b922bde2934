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
#include "pc_device.hpp"
#include "pc_launch.hpp"

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
            dst[c] = v;
        }
    }
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
    return go_publish<4, 2>(s, d, nchunks, stream);
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

// The consumer keeps one 64-pack group per lane at every size: a second group
// per lane would hold 2*N 16-byte packs in registers for the re-arm pass.
template <int N>
static hipError_t go_consume_sentinel(Ptrs<u32x4*> p, u32x4* out, uint64_t* bitmap, size_t npacks,
                                      hipStream_t stream) {
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
