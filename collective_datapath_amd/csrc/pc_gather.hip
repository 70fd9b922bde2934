// pc_gather.hip -- all-gather copy of sequence-stamped 128-byte blocks.
//
// "flash-comm: Self-Synchronizing Collective Communication for LLM
// Decoding", Section 4.3 (the all-gather is the distribution half of the
// all-reduce: shards pass through the same readiness check and are placed,
// not folded) and Section 3.1 (sequence-number readiness: a stale number
// means "not yet arrived"); Appendix A, Table 8 discussion (128-byte
// writes were never observed torn).  "Purlin: Separating Orchestration from
// the Datapath of Collectives", Section 3.1 (AllGather places the gathered
// partitions in rank order).
//
// A shard is an array of 136-byte records: a u64 sequence header followed by
// 128 payload bytes.  136 is not a multiple of 16, so every other payload
// starts 8 bytes off a 16-byte boundary.  A workgroup therefore stages 64
// records (8704 bytes = 544 aligned 16-byte pieces, one bitmap word) in LDS
// with coalesced 16-byte loads, then writes the accepted payloads to the
// output with coalesced 16-byte stores; LDS does the repacking.  In the
// bandwidth regime a workgroup takes 32 records (4352 bytes in, 4 KiB out,
// half a bitmap word, written as its own 32-bit half): many short-lived
// workgroups that each write a few KiB keep HBM writing fastest, 159.3 vs
// 164.2 us at 8 x 64 MiB shards with 10% stale records; with 2 MiB shards
// the 64-record groups are faster (3.97 vs 4.29 us).
#include "pc_device.hpp"
#include "pc_launch.hpp"

namespace pcdp {

constexpr int kGBlock = 256;
constexpr int kGroup = 64;                      // records per bitmap word (the API's group)
constexpr int kRecBytes = 136;

// Grid: x = workgroup within a shard, y = shard; a workgroup takes G records
// (64, one bitmap word, or 32, half of one).  The LDS tile is held as u64
// words (a record is 17 of them) and filled with 16-byte copies, so the
// header and the payload halves are read back as whole words.  Every lane
// issues its staging loads (three for 64 records, two for 32) before the
// first LDS write, through a buffer resource sized to the workgroup's
// records: loads past them return zero and land in the tile's padding, so
// the staging needs no branch (a loop of load, wait, write had serialised
// them).  Output stores carry the non-temporal hint: the gathered output is
// written once here and read by a later operation, and keeping it from
// displacing the shards in the caches measured 22% faster on the 8 x 2 MiB
// workload.  kLoadPolicy is the staging loads' cache policy: default, or
// non-temporal for calls far larger than the last-level cache (chosen at
// launch).
template <int kLoadPolicy, int G>
__global__ __launch_bounds__(kGBlock) void k_allgather(Ptrs<const u32x4*> shards, u32x4* out,
                                                        uint64_t* bitmap, uint64_t seq,
                                                        uint32_t per_shard) {
    static_assert(G == 64 || G == 32, "a workgroup covers one bitmap word or half of one");
    constexpr int kRecWords = kRecBytes / 8;                       // 17
    constexpr int kPieces = G * kRecBytes / 16;                    // 544 or 272
    constexpr int kLoads = (kPieces + kGBlock - 1) / kGBlock;      // 3 or 2 per lane
    __shared__ __attribute__((aligned(16))) uint64_t tile[kLoads * kGBlock * 2];
    const uint32_t g = blockIdx.x, r = blockIdx.y, t = threadIdx.x;
    const __amdgpu_buffer_rsrc_t rs = tile_rsrc(shards.p[r] + (size_t)g * kPieces, kPieces * 16u);
    u32x4 v[kLoads];
#pragma unroll
    for (int j = 0; j < kLoads; ++j) v[j] = load16_rsrc<kLoadPolicy>(rs, (j * kGBlock + t) * 16u);
#pragma unroll
    for (int j = 0; j < kLoads; ++j) __builtin_memcpy(&tile[2 * (j * kGBlock + t)], &v[j], sizeof v[j]);
    __syncthreads();

    const size_t item0 = ((size_t)r * per_shard + g) * G;  // first output block of the workgroup
    u32x4* dst = out + item0 * 8;
    // G records x 8 pieces of 16 bytes; consecutive lanes take consecutive pieces.
#pragma unroll
    for (int k = 0; k < G * 8 / kGBlock; ++k) {
        const uint32_t q = k * kGBlock + t;
        const uint32_t i = q >> 3, piece = q & 7;
        const uint64_t* rec = tile + i * kRecWords;
        if (rec[0] == seq) {
            const uint64_t a = rec[1 + 2 * piece], b = rec[2 + 2 * piece];
            u32x4 v;
            v[0] = (uint32_t)a; v[1] = (uint32_t)(a >> 32);
            v[2] = (uint32_t)b; v[3] = (uint32_t)(b >> 32);
            store16<true>(dst + q, v);
        }
    }
    if (t < kWave) {
        // Lanes past the workgroup's records vote 0 (their bits belong to the
        // other half of the word, which another workgroup writes).
        const uint64_t word = __ballot(t < G && tile[(t < G ? t : 0) * kRecWords] == seq);
        if (t == 0) {
            if constexpr (G == 64) bitmap[item0 / 64] = word;
            else reinterpret_cast<uint32_t*>(bitmap)[item0 / 32] = (uint32_t)word;  // little-endian half
        }
    }
}

hipError_t launch_allgather(const void* const* shards, int n, void* out, size_t groups,
                            uint64_t seq, void* bitmap, hipStream_t stream) {
    Ptrs<const u32x4*> p;
    for (int r = 0; r < kMaxRanks; ++r) p.p[r] = r < n ? static_cast<const u32x4*>(shards[r]) : nullptr;
    u32x4* o = static_cast<u32x4*>(out);
    uint64_t* b = static_cast<uint64_t*>(bitmap);
    // Records read plus payloads written.  From 768 MiB, three times the
    // last-level cache, the staging loads carry the non-temporal hint: at 8
    // ranks 126 vs 138 us with 48 MiB shards, 169 vs 184 with 64 MiB and 257
    // vs 277 with 96 MiB.  At 528 MiB (8 x 32 or 4 x 64 MiB) it cost 10%,
    // and at 8 x 2 MiB it made the call 45% slower.  The same calls take 32
    // records per workgroup.  At most 2^22 groups per shard, so the grid's x
    // stays below 2^23.
    const size_t moved = (size_t)n * groups * kGroup * (kRecBytes + 128);
    const bool stream_regime = moved >= ((size_t)768 << 20);
    uint32_t per_shard = (uint32_t)(stream_regime ? 2 * groups : groups);
    dim3 grid(per_shard, (unsigned)n);
    void* args[] = {&p, &o, &b, &seq, &per_shard};
    const void* k = stream_regime ? (const void*)&k_allgather<kPolicyNonTemporal, 32>
                                  : (const void*)&k_allgather<0, 64>;
    return hipLaunchKernel(k, grid, dim3(kGBlock), args, 0, stream);
}

}  // namespace pcdp
