// pc_staged.hpp -- LDS-staged loads for the bandwidth-regime folds.
//
// "Purlin: Separating Orchestration from the Datapath of Collectives",
// Section 3.3: a transfer is pipelined through a few shared-memory stages so
// that enough bytes are in flight to cover the memory latency (Equation (3)
// sizes the pipeline by the bandwidth-delay product; the pipeline is primed,
// run in steady state and drained).  On gfx950 a buffer load can write its
// 16 bytes per lane straight into LDS, so the stages fill without passing
// through registers.
//
// Shape.  One 256-lane workgroup per CU (the LDS request is kept above half
// of the CU's 160 KiB, so no second workgroup of the kernel fits).  Work is
// cut into tiles of 1024 16-byte chunks per rank; lane t of the workgroup
// owns chunks t, t + 256, t + 512, t + 768 of a tile, so wave w covers the
// four 1 KiB rows w*64 + 256*u of the tile (u = 0..3).  A workgroup takes its
// tiles in batches of 8 (32 rows per wave), and the tiles left over in
// batches of 4, 2 and 1, so no batch holds a tile that does not exist.
// Every wave runs its own pipeline over the rows of a batch: a stage holds
// one row of each of the N ranks (N KiB per wave); S stages are primed, then
// for each row: wait until its loads have landed, read it from LDS, fold it,
// and refill the stage with the row S places ahead.  The folded results of
// the batch stay in registers until the batch's read phase is over; the
// workgroup then passes a barrier and stores them, so HBM sees long runs of
// reads and short runs of writes.
//
// Waits are explicit.  The loads of a wave complete in issue order, so
// before reading row j the wave waits until at most (rows issued after j) * N
// loads are outstanding, and before refilling a stage it waits until its own
// reads of that stage have returned.  The compiler's own wait placement for
// load-to-LDS was found to let reads of a stage run ahead of the loads that
// fill it, so it is not relied on; each wait is an inline "s_waitcnt" that is
// also a compiler barrier for memory accesses, fenced by scheduling barriers.
// Every stage is its own LDS array, so the compiler can tell the stages apart
// and does not add waits of its own that would drain the pipeline.
#pragma once

#include "pc_device.hpp"

#include <type_traits>
#include <utility>

namespace pcdp {

typedef __attribute__((address_space(3))) void* lds_ptr_t;

constexpr int kStageBatchTiles = 8;                  // tiles per full batch
constexpr uint32_t kStageTileChunks = 1024;          // chunks per tile per rank
constexpr uint32_t kStageBlock = 256;                // lanes per workgroup
constexpr uint32_t kStageMinLdsBytes = 84u << 10;    // over half of the CU's LDS
constexpr int kStageMaxDepth = 8;
// Ranks from which the staged folds are used: with 2 ranks the staged
// reduce lost to the register kernel (29.4 vs 28.5 us at 8 ranks' worth of
// bytes), and below 4 ranks a workgroup's stages no longer fill over half of
// the CU's LDS.
constexpr int kStageMinRanks = 4;

// Stages per wave: about 24 KiB of a wave's loads in flight, at least 3
// stages, at most 8 (the number of stage arrays).
template <int N>
constexpr int stage_depth() {
    constexpr int want = (24 + N - 1) / N;
    return want < 3 ? 3 : want > kStageMaxDepth ? kStageMaxDepth : want;
}

template <int N>
constexpr uint32_t stage_lds_bytes() {
    return (uint32_t)stage_depth<N>() * 4u * N * 1024u;
}

// Dynamic LDS to request at launch so that the workgroup takes over half of
// the CU's LDS (one workgroup per CU).
template <int N>
constexpr uint32_t stage_pad_bytes() {
    return stage_lds_bytes<N>() >= kStageMinLdsBytes ? 0u : kStageMinLdsBytes - stage_lds_bytes<N>();
}

// Wait until at most kCount vector memory operations of this wave are
// outstanding.
template <int kCount>
__device__ __forceinline__ void wait_vm() {
    static_assert(kCount >= 0 && kCount < 64, "vmcnt range");
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(kCount) : "memory");
    __builtin_amdgcn_sched_barrier(0);
}

// Wait until this wave's LDS reads have returned.
__device__ __forceinline__ void wait_lds_reads() {
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
}

// Declares the stage arrays of a kernel (unused ones take no LDS).
#define PC_STAGE_ARRAYS(N)                   \
    __shared__ u32x4 pc_stage0[4 * (N) * 64]; \
    __shared__ u32x4 pc_stage1[4 * (N) * 64]; \
    __shared__ u32x4 pc_stage2[4 * (N) * 64]; \
    __shared__ u32x4 pc_stage3[4 * (N) * 64]; \
    __shared__ u32x4 pc_stage4[4 * (N) * 64]; \
    __shared__ u32x4 pc_stage5[4 * (N) * 64]; \
    __shared__ u32x4 pc_stage6[4 * (N) * 64]; \
    __shared__ u32x4 pc_stage7[4 * (N) * 64];
#define PC_STAGE_LIST pc_stage0, pc_stage1, pc_stage2, pc_stage3, pc_stage4, pc_stage5, pc_stage6, pc_stage7

// A tile of a batch: its first chunk in every rank buffer and its valid
// bytes per rank (less than a whole tile only for a ragged last tile).
struct StageTile {
    size_t first;
    uint32_t bytes;
};

// One batch of kTiles tiles, seen by one wave: folds the wave's 4 * kTiles
// rows.  kReady: also evaluates sentinel-free readiness per pack (no half of
// any rank's 16 bytes equals 0xFFFF), gathers the ballot of row j into lane
// j (words_lo / words_hi) and row j's lane bit into ready_bits.
template <int N, bool kReady, int kTiles>
struct StagedBatch {
    static constexpr int S = stage_depth<N>();
    static constexpr int kRows = 4 * kTiles;
    const Ptrs<const u32x4*>& src;
    const StageTile (&tile)[kTiles];
    u32x4* const stage[kStageMaxDepth];
    const uint32_t w, lane;
    u32x4 res[kRows];
    uint64_t ready_bits = 0;
    uint32_t words_lo = 0, words_hi = 0;

    template <int J>
    __device__ __forceinline__ void issue() {
        const StageTile t = tile[J / 4];
        u32x4* const st = stage[J % S];
#pragma unroll
        for (int r = 0; r < N; ++r) {
            const __amdgpu_buffer_rsrc_t rs = tile_rsrc(src.p[r] + t.first, t.bytes);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_ptr_t)(st + (w * N + r) * 64), 16,
                                                     ((J % 4) * 256 + w * 64 + lane) * 16u, 0, 0,
                                                     kPolicyNonTemporal);
        }
    }

    template <int J>
    __device__ __forceinline__ void prime() {
        if constexpr (J < S) issue<J>();
    }

    template <int J>
    __device__ __forceinline__ void step() {
        constexpr int kLast = J + S - 1 < kRows - 1 ? J + S - 1 : kRows - 1;
        wait_vm<(kLast - J) * N>();
        const u32x4* const st = stage[J % S];
        u32x4 v[N];
#pragma unroll
        for (int r = 0; r < N; ++r) v[r] = st[(w * N + r) * 64 + lane];
        if constexpr (kReady) {
            bool ready = true;
#pragma unroll
            for (int r = 0; r < N; ++r)
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    ready &= ((v[r][e] & 0xFFFFu) != 0xFFFFu) & ((v[r][e] >> 16) != 0xFFFFu);
            ready_bits |= (uint64_t)ready << J;
            const uint64_t word = __ballot(ready);
            words_lo = lane == (uint32_t)J ? (uint32_t)word : words_lo;
            words_hi = lane == (uint32_t)J ? (uint32_t)(word >> 32) : words_hi;
        }
        res[J] = fold_chunk<N>(v);
        if constexpr (J + S < kRows) {
            wait_lds_reads();  // the stage is refilled only after it has been read
            issue<J + S>();
        }
    }

    template <int... Js>
    __device__ __forceinline__ void run(std::integer_sequence<int, Js...>) {
        (prime<Js>(), ...);
        (step<Js>(), ...);
    }

    __device__ __forceinline__ void run() { run(std::make_integer_sequence<int, kRows>{}); }
};

// Runs body(std::integral_constant<int, T>{}, g0) over a workgroup's tiles
// g0, g0 + stride, ... < ntiles: full batches of 8, then the rest as
// batches of 4, 2 and 1.  The body is a generic lambda of the kernel, so it
// names the kernel's stage arrays directly (held behind a pointer table the
// compiler lost track of them and spilled).
// The same batch with the ranks on a diagonal: at step t, rank r loads row
// t - r, so at any moment the ranks' loads sit one row (4 KiB) apart instead
// of at the same offset of every rank buffer.  Rank buffers whose bases are
// congruent modulo 32 KiB put same-offset loads into the same DRAM banks on
// different pages.  The 8 x 64 MiB reduce took 92.4 - 93.5 us on such
// layouts (separate allocations, which agree modulo 2 MiB: 88.2 - 92.3 us,
// depending on where they landed) against 86.6 - 87.3 us with the rank
// buffers 4 to 16 KiB apart; on the diagonal the congruent layouts took
// 87.0 - 88.8 us.  bases_congruent below chooses it.  Row j is still folded
// in rank order 0..N-1: its accumulators take rank r at step j + r.  Each
// step reads one stage of N rows (one per rank) as before; a batch takes
// 4 * kTiles + N - 1 steps, the first and last N - 1 with fewer loads.
template <int N, int kTiles>
struct DiagonalBatch {
    static constexpr int S = stage_depth<N>();
    static constexpr int kRows = 4 * kTiles;
    static constexpr int kSteps = kRows + N - 1;
    const Ptrs<const u32x4*>& src;
    const StageTile (&tile)[kTiles];
    u32x4* const stage[kStageMaxDepth];
    const uint32_t w, lane;
    u32x4 res[kRows];
    float acc[kRows][8];

    // Ranks that load at step t: rows t - r within [0, kRows).
    static constexpr int first_rank(int t) { return t - (kRows - 1) > 0 ? t - (kRows - 1) : 0; }
    static constexpr int last_rank(int t) { return t < N - 1 ? t : N - 1; }
    static constexpr int loads_at(int t) { return t < 0 || t >= kSteps ? 0 : last_rank(t) - first_rank(t) + 1; }
    // Loads issued after step t's own when step t waits: those of steps
    // t + 1 .. t + S - 1.
    static constexpr int loads_after(int t) {
        int n = 0;
        for (int u = t + 1; u < t + S && u < kSteps; ++u) n += loads_at(u);
        return n;
    }

    template <int T, int R>
    __device__ __forceinline__ void issue_rank() {
        if constexpr (R >= first_rank(T) && R <= last_rank(T)) {
            constexpr int J = T - R;
            const StageTile t = tile[J / 4];
            const __amdgpu_buffer_rsrc_t rs = tile_rsrc(src.p[R] + t.first, t.bytes);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_ptr_t)(stage[T % S] + (w * N + R) * 64), 16,
                                                     ((J % 4) * 256 + w * 64 + lane) * 16u, 0, 0,
                                                     kPolicyNonTemporal);
        }
    }

    template <int T, int... Rs>
    __device__ __forceinline__ void issue(std::integer_sequence<int, Rs...>) {
        (issue_rank<T, Rs>(), ...);
    }

    template <int T>
    __device__ __forceinline__ void issue() {
        if constexpr (T < kSteps) issue<T>(std::make_integer_sequence<int, N>{});
    }

    template <int T, int R>
    __device__ __forceinline__ void fold_rank(const u32x4* st) {
        if constexpr (R >= first_rank(T) && R <= last_rank(T)) {
            constexpr int J = T - R;
            const u32x4 v = st[(w * N + R) * 64 + lane];
            if constexpr (R == 0) {
#pragma unroll
                for (int e = 0; e < 8; ++e) acc[J][e] = -0.0f;
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                acc[J][2 * e] = acc[J][2 * e] + widen_lo(v[e]);
                acc[J][2 * e + 1] = acc[J][2 * e + 1] + widen_hi(v[e]);
            }
            if constexpr (R == N - 1) {
                u32x4 o;
#pragma unroll
                for (int e = 0; e < 4; ++e) o[e] = narrow_pair(acc[J][2 * e], acc[J][2 * e + 1]);
                res[J] = o;
            }
        }
    }

    template <int T, int... Rs>
    __device__ __forceinline__ void fold(const u32x4* st, std::integer_sequence<int, Rs...>) {
        (fold_rank<T, Rs>(st), ...);
    }

    template <int T>
    __device__ __forceinline__ void prime() {
        if constexpr (T < S) issue<T>();
    }

    template <int T>
    __device__ __forceinline__ void step() {
        wait_vm<loads_after(T)>();
        fold<T>(stage[T % S], std::make_integer_sequence<int, N>{});
        if constexpr (T + S < kSteps) {
            wait_lds_reads();  // the stage is refilled only after it has been read
            issue<T + S>();
        }
    }

    template <int... Ts>
    __device__ __forceinline__ void run(std::integer_sequence<int, Ts...>) {
        (prime<Ts>(), ...);
        (step<Ts>(), ...);
    }

    __device__ __forceinline__ void run() { run(std::make_integer_sequence<int, kSteps>{}); }
};

// Which batch a launch takes: the diagonal when every rank buffer's base is
// congruent to rank 0's modulo kBankPeriod.  Measured on the 8 x 64 MiB
// reduce with the rank buffers 0, 32 KiB, 64 KiB, 128 KiB, 1 MiB or 2 MiB
// apart (and in separate allocations) the diagonal was faster or level;
// with the buffers 4 to 16 KiB apart the plain pipeline already ran at
// 86.6 - 87.3 us, and the diagonal would cancel a 4 KiB spacing.
constexpr uintptr_t kBankPeriod = 32u << 10;

__host__ inline bool bases_congruent(const void* const* p, int n) {
    for (int r = 1; r < n; ++r)
        if (((uintptr_t)p[r] - (uintptr_t)p[0]) % kBankPeriod != 0) return false;
    return true;
}

template <typename Body>
__device__ __forceinline__ void for_each_stage_batch(const Body& body, uint32_t ntiles) {
    const uint32_t stride = gridDim.x;
    uint32_t g0 = blockIdx.x;
    uint32_t left = (ntiles - blockIdx.x + stride - 1) / stride;  // blockIdx.x < ntiles
    for (; left >= 8; left -= 8, g0 += 8 * stride) body(std::integral_constant<int, 8>{}, g0);
    if (left & 4) {
        body(std::integral_constant<int, 4>{}, g0);
        g0 += 4 * stride;
    }
    if (left & 2) {
        body(std::integral_constant<int, 2>{}, g0);
        g0 += 2 * stride;
    }
    if (left & 1) body(std::integral_constant<int, 1>{}, g0);
}

// Byte offset of row j's chunk for this lane within its tile.
__device__ __forceinline__ uint32_t stage_row_offset(int j, uint32_t w, uint32_t lane) {
    return ((uint32_t)(j % 4) * 256u + w * 64u + lane) * 16u;
}

}  // namespace pcdp
