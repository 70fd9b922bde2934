// pc_ll.hip -- sequence-number ("LL") lines: pack on the producer side,
// validate-and-fold on the consumer side.
//
// "flash-comm: Self-Synchronizing Collective Communication for LLM
// Decoding", Section 3.1 (sequence-number readiness: payload and call number
// share one store, so a line whose number is the current call's has fully
// arrived and any other line is stale), Section 4.3 (16-byte
// packet = 8 payload bytes + two copies of the sequence number; one-hop
// reduce only after every source is ready, folded by source rank in rank
// order) and Section 3.3 (fold order 0..N-1).  "Purlin: Separating
// Orchestration from the Datapath of Collectives", Section 3.2 (latency path:
// payload packed with a flag so the consumer polls the data itself).
//
// Line j (8 bytes, little-endian): bytes 0..3 = bf16 elements 2j (low half)
// and 2j+1 (high half), bytes 4..7 = sequence number.  Two lines make one of
// flash-comm's 16-byte packets.  Each line is read with one 8-byte load, so
// its data and its sequence number are observed together.
#include "pc_device.hpp"
#include "pc_launch.hpp"

namespace pcdp {

// Launch shapes: W waves per workgroup, U 64-line groups (consume) or
// 16-byte chunks (pack) per lane.  Payloads under 4 MiB per rank take one
// group or chunk per lane, so a 128 KiB call still spreads over more
// workgroups (the two-per-lane shape measured 0.5 us slower per call there).

// ---- pack: 8 bf16 (16 bytes) in -> 4 lines (32 bytes) out -----------------------
// Device-scope stores through a workgroup-tile resource: 1.62-1.63 vs
// 1.64-1.66 us per call in a graph at 128 KiB.
template <int W, int U>
__global__ __launch_bounds__(W * kWave) void k_pack_ll(const u32x4* src, u32x4* dst, uint32_t seq,
                                                        size_t nchunks) {
    constexpr int kBlk = W * kWave;
    const size_t tile0 = (size_t)blockIdx.x * (kBlk * U);
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const size_t c = tile0 + u * kBlk + threadIdx.x;
        if (c < nchunks) {
            const u32x4 v = src[c];
            u32x4 a, b;
            a[0] = v[0]; a[1] = seq; a[2] = v[1]; a[3] = seq;
            b[0] = v[2]; b[1] = seq; b[2] = v[3]; b[3] = seq;
            const __amdgpu_buffer_rsrc_t rd = tile_rsrc(dst + 2 * tile0, 2u * kBlk * U * 16u);
            store16_rsrc<kPolicyDeviceScope>(rd, (uint32_t)(2 * (c - tile0)) * 16u, a);
            store16_rsrc<kPolicyDeviceScope>(rd, (uint32_t)(2 * (c - tile0) + 1) * 16u, b);
        }
    }
}

// From 4 MiB per rank: a lane takes 8 input bytes (4 bf16) and writes the two
// lines they make as one 16-byte store, so a wave reads 512 B and writes
// 1 KiB, both contiguous.  (The kernel above writes two 16-byte chunks per
// lane, so each of its store instructions covers every other chunk of the
// output.)  A workgroup of 256 lanes takes one 2 KiB piece of the input and
// ends, as the Atom copy's workgroups do, with device-scope stores; above
// 64 MiB per rank its loads are non-temporal.  At one rank, against the
// same lane mapping with two pieces per lane and default policies: 5.9 vs
// 8.3 us at 16 MiB, 28.9 vs 29.3 at 64 MiB (33.9 vs 37.1 with the buffers
// rotated past the last-level cache), 123 vs 137 at 256 MiB and 244 vs 270
// at 512 MiB.  The grid is capped for the largest calls (2^32 pieces would
// not fit the launch's 32-bit work-item count), and its workgroups then
// loop over the pieces.
constexpr uint32_t kPackGridCap = 1u << 22;

template <int kLoadPolicy>
__global__ __launch_bounds__(4 * kWave) void k_pack_ll_half(const u32x2* src, u32x4* dst, uint32_t seq,
                                                             size_t nhalf) {
    constexpr uint32_t kTile = 4 * kWave;
    const uint32_t off = threadIdx.x;
    for (size_t first = (size_t)blockIdx.x * kTile; first < nhalf; first += (size_t)gridDim.x * kTile) {
        const size_t left = nhalf - first;
        const uint32_t n = (uint32_t)(left < kTile ? left : kTile);
        const u32x2 v = __builtin_bit_cast(
            u32x2, __builtin_amdgcn_raw_buffer_load_b64(tile_rsrc(src + first, n * 8u), off * 8u, 0, kLoadPolicy));
        const u32x4 a = {v[0], seq, v[1], seq};
        store16_rsrc<kPolicyDeviceScope>(tile_rsrc(dst + first, n * 16u), off * 16u, a);
    }
}

// ---- consume: every wave owns U groups of 64 consecutive lines ------------------
// Lane l of group u takes line base + 64u + l from every rank.  The wave's
// ballot over "all ranks carry seq" is exactly the 64-bit bitmap word of the
// group (bit l = line base + 64u + l), so no bit shuffling is needed.  Lines
// that are ready are folded in rank order and stored; the rest are skipped,
// leaving their output as it was.
template <int N, int W, int U>
__global__ __launch_bounds__(W * kWave) void k_consume_ll(Ptrs<const u32x2*> lines, uint32_t* out,
                                                           uint64_t* bitmap, uint32_t seq,
                                                           size_t nlines) {
    const uint32_t lane = threadIdx.x & (kWave - 1);
    const uint32_t wave = threadIdx.x / kWave;
    const size_t base = ((size_t)blockIdx.x * W + wave) * (kWave * U);
    if (base >= nlines) return;  // whole wave past the end
    u32x2 l[U][N];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        if (base + (size_t)u * kWave < nlines) {
#pragma unroll
            for (int r = 0; r < N; ++r) l[u][r] = lines.p[r][base + u * kWave + lane];
        }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const size_t g = base + (size_t)u * kWave;
        if (g >= nlines) break;
        bool ready = true;
#pragma unroll
        for (int r = 0; r < N; ++r) ready &= l[u][r][1] == seq;
        const uint64_t word = __ballot(ready);
        if (ready) {
            float lo = -0.0f, hi = -0.0f;
#pragma unroll
            for (int r = 0; r < N; ++r) {
                lo = lo + widen_lo(l[u][r][0]);
                hi = hi + widen_hi(l[u][r][0]);
            }
            out[g + lane] = narrow_pair(lo, hi);
        }
        if (lane == 0) bitmap[g / kWave] = word;
    }
}

// ---- consume, bandwidth regime (working sets of 512 MiB and more) -----------------
// A persistent grid of two 256-lane workgroups per CU.  Tile g holds lines
// [2048 g, 2048 g + 2048): wave w owns its groups 8w .. 8w + 7 of 64 lines,
// and lane l line l of each group, as above.  Workgroup b takes tiles b,
// b + grid, ... in batches of 8.  Every line of a batch is loaded (one
// non-temporal 8-byte buffer load per line and rank, so data and sequence
// number still arrive together), checked and folded into registers; after a
// barrier the batch's results and bitmap words are stored.  A line that is
// not ready gets an out-of-range store offset, which the tile's buffer
// resource drops, so no store sits behind a branch.
constexpr int kLLGroups = 8;                                     // per wave per tile
constexpr uint32_t kLLTileLines = 4 * kWave * kLLGroups;         // 2048
constexpr int kLLBatch = 8;                                      // tiles per batch
constexpr uint32_t kDropOffset = 0x80000000u;                    // past every tile resource

__device__ __forceinline__ u32x2 load8_nt(__amdgpu_buffer_rsrc_t rs, uint32_t byte_off) {
    return __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(rs, byte_off, 0, kPolicyNonTemporal));
}

// One batch: tiles g0, g0 + stride, ... (kBatch of them).  kAllValid: every
// tile of the batch exists, so no tile needs a test; otherwise (a
// workgroup's last batch) the missing tiles are skipped, so they issue no
// loads at all.
template <int N, int kBatch, bool kAllValid>
__device__ __forceinline__ void consume_ll_batch(const Ptrs<const u32x2*>& lines, uint32_t* out,
                                                 uint64_t* bitmap, uint32_t seq, size_t nlines,
                                                 uint32_t ntiles, uint32_t g0, uint32_t stride) {
    static_assert(kBatch * kLLGroups <= 64, "one readiness bit per line of a batch");
    const uint32_t lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
    uint32_t o[kBatch][kLLGroups];
    uint64_t ready_bits = 0;  // bit j * kLLGroups + u: this lane's line of tile j, group u
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
        const uint32_t g = g0 + j * stride;
        if (!kAllValid && g >= ntiles) continue;  // uniform for the workgroup
        const size_t first = (size_t)g * kLLTileLines;
        const size_t left = nlines - first;
        const uint32_t nl = (uint32_t)(left < kLLTileLines ? left : kLLTileLines);
        u32x2 l[kLLGroups][N];
        uint32_t words_lo = 0, words_hi = 0;
#pragma unroll
        for (int r = 0; r < N; ++r) {
            const __amdgpu_buffer_rsrc_t rs = tile_rsrc(lines.p[r] + first, nl * 8u);
#pragma unroll
            for (int u = 0; u < kLLGroups; ++u)
                l[u][r] = load8_nt(rs, ((wave * kLLGroups + u) * kWave + lane) * 8u);
        }
#pragma unroll
        for (int u = 0; u < kLLGroups; ++u) {
            bool ready = true;
            float lo = -0.0f, hi = -0.0f;
#pragma unroll
            for (int r = 0; r < N; ++r) {
                ready &= l[u][r][1] == seq;  // no short circuit: no branch per rank
                lo = lo + widen_lo(l[u][r][0]);
                hi = hi + widen_hi(l[u][r][0]);
            }
            o[j][u] = narrow_pair(lo, hi);
            ready_bits |= (uint64_t)ready << (j * kLLGroups + u);
            // Lane u of `words` takes the group's bitmap word.
            const uint64_t word = __ballot(ready);
            words_lo = lane == (uint32_t)u ? (uint32_t)word : words_lo;
            words_hi = lane == (uint32_t)u ? (uint32_t)(word >> 32) : words_hi;
        }
        // The wave's words leave in one 64-byte store by lanes 0..7 (one
        // store per word wrote about four times the bitmap's bytes to HBM).
        const __amdgpu_buffer_rsrc_t rb = tile_rsrc(bitmap + first / kWave, nl / kWave * 8u);
        u32x2 words;
        words[0] = words_lo;
        words[1] = words_hi;
        __builtin_amdgcn_raw_buffer_store_b64(words, rb,
                                              lane < (uint32_t)kLLGroups ? (wave * kLLGroups + lane) * 8u
                                                                         : kDropOffset,
                                              0, kPolicyDeviceScope);
        // Keep the next tile's address and descriptor set-up behind this
        // fold; computing all of them up front spilled registers.
        __builtin_amdgcn_sched_barrier(0);
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
        const uint32_t g = g0 + j * stride;
        if (!kAllValid && g >= ntiles) continue;
        const size_t first = (size_t)g * kLLTileLines;
        const size_t left = nlines - first;
        const uint32_t nl = (uint32_t)(left < kLLTileLines ? left : kLLTileLines);
        const __amdgpu_buffer_rsrc_t ro = tile_rsrc(out + first, nl * 4u);
#pragma unroll
        for (int u = 0; u < kLLGroups; ++u) {
            const bool ready = (ready_bits >> (j * kLLGroups + u)) & 1u;
            const uint32_t line = (wave * kLLGroups + u) * kWave + lane;
            __builtin_amdgcn_raw_buffer_store_b32(o[j][u], ro, ready ? line * 4u : kDropOffset, 0,
                                                  kPolicyDeviceScope);
        }
    }
}

template <int N, int kBatch>
__global__ __launch_bounds__(4 * kWave) __attribute__((amdgpu_waves_per_eu(2)))
void k_consume_ll_persistent(Ptrs<const u32x2*> lines, uint32_t* out, uint64_t* bitmap, uint32_t seq,
                             size_t nlines, uint32_t ntiles) {
    const uint32_t stride = gridDim.x;
    for (uint32_t g0 = blockIdx.x; g0 < ntiles; g0 += stride * kBatch) {
        if (g0 + (kBatch - 1) * stride < ntiles)
            consume_ll_batch<N, kBatch, true>(lines, out, bitmap, seq, nlines, ntiles, g0, stride);
        else
            consume_ll_batch<N, kBatch, false>(lines, out, bitmap, seq, nlines, ntiles, g0, stride);
    }
}

// Bytes per rank below which the one-wave shapes are used.
constexpr size_t kSmallBytes = (size_t)4 << 20;

template <int W, int U>
static hipError_t go_pack(const u32x4* s, u32x4* d, uint32_t seq, size_t nchunks, hipStream_t stream) {
    const size_t tile = (size_t)W * kWave * U;
    dim3 grid((unsigned)((nchunks + tile - 1) / tile));
    void* args[] = {&s, &d, &seq, &nchunks};
    return hipLaunchKernel((const void*)&k_pack_ll<W, U>, grid, dim3(W * kWave), args, 0, stream);
}

hipError_t launch_pack_ll(const void* src, void* dst, size_t nchunks, uint32_t seq,
                          hipStream_t stream) {
    const u32x4* s = static_cast<const u32x4*>(src);
    u32x4* d = static_cast<u32x4*>(dst);
    if (nchunks * 16 < kSmallBytes) return go_pack<4, 1>(s, d, seq, nchunks, stream);
    const u32x2* h = reinterpret_cast<const u32x2*>(src);
    size_t nhalf = nchunks * 2;
    const size_t pieces = (nhalf + 4 * kWave - 1) / (4 * kWave);
    dim3 grid((unsigned)(pieces < kPackGridCap ? pieces : kPackGridCap));
    void* args[] = {&h, &d, &seq, &nhalf};
    const void* k = nchunks * 16 <= ((size_t)64 << 20) ? (const void*)&k_pack_ll_half<0>
                                                       : (const void*)&k_pack_ll_half<kPolicyNonTemporal>;
    return hipLaunchKernel(k, grid, dim3(4 * kWave), args, 0, stream);
}

template <int N, int W, int U>
static hipError_t go_consume_shape(Ptrs<const u32x2*> p, uint32_t* out, uint64_t* bitmap,
                                   uint32_t seq, size_t nlines, hipStream_t stream) {
    const size_t per_block = (size_t)W * kWave * U;
    dim3 grid((unsigned)((nlines + per_block - 1) / per_block));
    void* args[] = {&p, &out, &bitmap, &seq, &nlines};
    return hipLaunchKernel((const void*)&k_consume_ll<N, W, U>, grid, dim3(W * kWave), args, 0,
                           stream);
}

template <int N, int kBatch>
static hipError_t go_consume_persistent(Ptrs<const u32x2*> p, uint32_t* out, uint64_t* bitmap,
                                        uint32_t seq, size_t nlines, hipStream_t stream) {
    // Whole rounds of at most two workgroups per CU, then as few workgroups
    // as give that many rounds.
    uint32_t ntiles = (uint32_t)((nlines + kLLTileLines - 1) / kLLTileLines);
    const uint32_t slots = 2 * device_cus();
    const uint32_t rounds = (ntiles + slots - 1) / slots;
    const uint32_t grid = (ntiles + rounds - 1) / rounds;
    void* args[] = {&p, &out, &bitmap, &seq, &nlines, &ntiles};
    return hipLaunchKernel((const void*)&k_consume_ll_persistent<N, kBatch>, dim3(grid), dim3(4 * kWave),
                           args, 0, stream);
}

template <int N>
static hipError_t go_consume(Ptrs<const u32x2*> p, uint32_t* out, uint64_t* bitmap, uint32_t seq,
                             size_t nlines, hipStream_t stream) {
    // Lines read plus results written.  From 512 MiB, twice the last-level
    // cache, the persistent kernel is ahead (8 ranks: 172 vs 207 us at 64 MiB
    // per rank, 88 vs 102 at 32 MiB); below it, the kernel above keeps more
    // of its inputs in the cache between calls (44 vs 46 us at 16 MiB).
    if (nlines * (8 * (size_t)N + 4) >= ((size_t)512 << 20))
        return go_consume_persistent<N, kLLBatch>(p, out, bitmap, seq, nlines, stream);
    // Below 4 MiB per rank: two waves per workgroup (1.85 vs 1.91 us per
    // call at 8 ranks x 128 KiB; one, eight and sixteen waves were slower).
    if (nlines * 4 < kSmallBytes)
        return go_consume_shape<N, 2, 1>(p, out, bitmap, seq, nlines, stream);
    return go_consume_shape<N, 4, 2>(p, out, bitmap, seq, nlines, stream);
}

hipError_t launch_consume_ll(const void* const* lines, int n, void* out, size_t nlines,
                             uint32_t seq, void* bitmap, hipStream_t stream) {
    Ptrs<const u32x2*> p;
    for (int r = 0; r < kMaxRanks; ++r) p.p[r] = r < n ? static_cast<const u32x2*>(lines[r]) : nullptr;
    uint32_t* o = static_cast<uint32_t*>(out);
    uint64_t* b = static_cast<uint64_t*>(bitmap);
    switch (n) {
        case 1: return go_consume<1>(p, o, b, seq, nlines, stream);
        case 2: return go_consume<2>(p, o, b, seq, nlines, stream);
        case 3: return go_consume<3>(p, o, b, seq, nlines, stream);
        case 4: return go_consume<4>(p, o, b, seq, nlines, stream);
        case 5: return go_consume<5>(p, o, b, seq, nlines, stream);
        case 6: return go_consume<6>(p, o, b, seq, nlines, stream);
        case 7: return go_consume<7>(p, o, b, seq, nlines, stream);
        case 8: return go_consume<8>(p, o, b, seq, nlines, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace pcdp
