// pc_reduce.hip -- the rank-ordered N-way reduce and the twoshot split.
//
// Reduce: "Purlin: Separating Orchestration from the Datapath of
// Collectives", Section 3.3 (the Atom's reduce of n typed sources, Equation
// (2)); oneshot's local reduction in "SiFAR: Synchronization-Free All-Reduce
// for Low-Latency LLM Inference", Section 3.1, Figure 5.
// Twoshot: SiFAR Section 3.1, Figure 6 (reduce-scatter, then broadcast) and
// "flash-comm: Self-Synchronizing Collective Communication for LLM
// Decoding", Section 3.3 (one owner reduces each block once and distributes
// it) and Section 4.3 (sharded two-hop).
//
// Work mapping.  Each 16-byte chunk (8 bf16) of the output belongs to one
// lane; a 256-lane workgroup owns a tile of 256*U consecutive chunks, lane t
// taking chunks t, t+256, ... so every load and store instruction of a wave
// covers 1 KiB of consecutive bytes per rank.  All N*U loads of a lane are
// issued before its first fold, which keeps N*U*16 bytes per lane in flight:
// the gfx950 counterpart of sizing a copy pipeline to the bandwidth-delay
// product (Purlin, Section 3.3, Equation (3)).  Cache-resident payloads use
// one workgroup per tile (k_reduce).  Payloads far beyond the last-level
// cache use a persistent grid: with four or more ranks one workgroup per CU
// whose loads go straight to LDS stages (k_reduce_staged, pc_staged.hpp),
// otherwise two workgroups per CU whose loads land in registers
// (k_reduce_persistent); with one rank, and with two or three from 128 MiB
// per rank, short-lived workgroups of 8 KiB tiles instead (k_reduce).
// Three output modes cover the oneshot reduce, twoshot phase 1 and the
// single-launch twoshot; at the largest sizes the
// single-launch twoshot folds first and hands its tiles out afterwards, in
// the same launch (k_twoshot_persistent).  The two-launch twoshot's second
// kernel copies each owner slice out (k_copyout), at 7 and 8 ranks from
// 48 MiB per rank with one destination per workgroup (k_copyout_dest).
#include "pc_device.hpp"
#include "pc_launch.hpp"
#include "pc_staged.hpp"

namespace pcdp {

constexpr int kBlock = 256;

// Where a folded chunk goes.  kOne: dst.p[0] (oneshot reduce).  kOwner:
// dst.p[s], the owner of slice s (twoshot phase 1).  kAll: every dst.p[r]
// (single-launch twoshot: the owner folds its block once and distributes it).
enum class Out { kOne, kOwner, kAll };

// ---- slice reduce (oneshot when there is one slice) ----------------------------
// Grid: x = tile within a slice, y = slice.  Slice s covers chunks
// [s*nslice, (s+1)*nslice) of every input; where its folds go is set by kOut.
// A lane loads its U chunks of every rank through tile-sized buffer
// resources (a ragged tile needs no branch), folds, and stores with
// device-scope stores.  Per call in a graph at 8 ranks, against the kernel
// below: the oneshot 1.71 vs 1.79 us at 8 KiB per rank and 2.10 vs 2.28 at
// 1 MiB; the single-launch twoshot 2.27 vs 2.55 us at 256 KiB and 3.32 vs
// 4.14 at 1 MiB.  The twoshot forms take it from 128 KiB per rank; below
// that their small ragged slices favour the kernel below (single launch at
// 8 KiB per rank: 1.83 vs 2.00 us).  kLoadPolicy: default for cache-resident
// payloads; non-temporal in the bandwidth regime with one to three ranks.
template <int N, int U, int kLoadPolicy, Out kOut>
__global__ __launch_bounds__(kBlock) void k_reduce(Ptrs<const u32x4*> src, Ptrs<u32x4*> dst,
                                                     uint32_t nslice) {
    constexpr uint32_t kTile = kBlock * U;
    const uint32_t s = kOut == Out::kOne ? 0u : blockIdx.y;
    size_t first;
    uint32_t chunks;
    if constexpr (kOut == Out::kOne) {
        const uint32_t tile0 = blockIdx.x * kTile;  // below nslice < 2^32
        const uint32_t left = nslice - tile0;
        first = tile0;
        chunks = left < kTile ? left : kTile;
    } else {  // several slices: the 128-byte-aligned tiles of slice_tile()
        const SliceTile st = slice_tile(s, blockIdx.x, nslice, kTile);
        first = st.first;
        chunks = st.chunks;
    }
    const uint32_t t = threadIdx.x, bytes = chunks * 16u;
    u32x4 v[U][N];
#pragma unroll
    for (int r = 0; r < N; ++r) {
        const __amdgpu_buffer_rsrc_t rs = tile_rsrc(src.p[r] + first, bytes);
#pragma unroll
        for (int u = 0; u < U; ++u) v[u][r] = load16_rsrc<kLoadPolicy>(rs, (u * kBlock + t) * 16u);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const u32x4 o = fold_chunk<N>(v[u]);
        if constexpr (kOut == Out::kAll) {
#pragma unroll
            for (int r = 0; r < N; ++r) store16_tile(tile_rsrc(dst.p[r] + first, bytes), (u * kBlock + t) * 16u, o);
        } else {
            store16_tile(tile_rsrc(dst.p[kOut == Out::kOne ? 0 : s] + first, bytes), (u * kBlock + t) * 16u, o);
        }
    }
}

// The twoshot forms below 128 KiB per rank: the same mapping with 64-bit
// addresses and default-policy stores; a ragged tile takes a guarded
// chunk-by-chunk path, so lanes past it issue nothing.
template <int N, Out kOut>
__device__ __forceinline__ void put_chunk(const Ptrs<u32x4*>& dst, uint32_t s, size_t at, u32x4 v) {
    if constexpr (kOut == Out::kAll) {
#pragma unroll
        for (int r = 0; r < N; ++r) dst.p[r][at] = v;
    } else {
        dst.p[kOut == Out::kOwner ? s : 0][at] = v;
    }
}

template <int N, int U, Out kOut>
__global__ __launch_bounds__(kBlock) void k_reduce_small(Ptrs<const u32x4*> src, Ptrs<u32x4*> dst,
                                                           uint32_t nslice) {
    constexpr uint32_t kTile = kBlock * U;
    const uint32_t s = kOut == Out::kOne ? 0u : blockIdx.y;
    size_t first;
    uint32_t left;
    if constexpr (kOut == Out::kOne) {
        const uint32_t tile0 = blockIdx.x * kTile;
        first = tile0;
        left = nslice - tile0;
    } else {
        const SliceTile st = slice_tile(s, blockIdx.x, nslice, kTile);
        first = st.first;
        left = st.chunks;
    }
    const uint32_t t = threadIdx.x;
    const u32x4* in[N];
#pragma unroll
    for (int r = 0; r < N; ++r) in[r] = src.p[r] + first;
    if (left >= kTile) {
        u32x4 v[U][N];
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int r = 0; r < N; ++r) v[u][r] = in[r][u * kBlock + t];
#pragma unroll
        for (int u = 0; u < U; ++u) put_chunk<N, kOut>(dst, s, first + u * kBlock + t, fold_chunk<N>(v[u]));
    } else {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const uint32_t c = u * kBlock + t;
            if (c < left) {
                u32x4 v[N];
#pragma unroll
                for (int r = 0; r < N; ++r) v[r] = in[r][c];
                put_chunk<N, kOut>(dst, s, first + c, fold_chunk<N>(v));
            }
        }
    }
}

// ---- bandwidth regime: persistent slice reduce ------------------------------------
// For working sets far beyond the last-level cache.  The grid is sized by the
// host to whole rounds of at most two workgroups per CU, and workgroup w takes
// tiles w, w + grid, w + 2*grid, ...  Each tile is 16 KiB per rank, accessed
// through tile-sized buffer resources (a ragged last tile needs no branch).
// A workgroup takes its tiles in batches of up to kBatch: for each tile every
// lane issues all 4*N non-temporal loads and folds its 4 chunks, keeping the
// results in registers; after the batch the workgroup passes a barrier and
// issues all of the batch's stores together, as device-scope stores.  DRAM
// then sees long runs of reads and long runs of writes instead of a fine mix;
// for this 8:1 read/write stream that, the two-per-CU persistent grid and the
// store policy each measurably raise HBM efficiency (see the design notes).
// Grid tile g covers slice g / tiles_per_slice.  The fan-out mode stores each
// result N times; it batches one tile, which keeps it free of register spills.
template <int N, Out kOut>
constexpr int batch_tiles() { return kOut == Out::kAll ? 1 : 8; }

// Geometry of grid tile g: its slice, first chunk and valid bytes per rank.
struct TileAt {
    uint32_t s;
    size_t first;
    uint32_t bytes;
};

// Several slices: tiles on the 128-byte-aligned grid of slice_tile().
template <Out kOut>
__device__ __forceinline__ TileAt tile_at(uint32_t g, uint32_t nslice, uint32_t tiles_per_slice,
                                          uint32_t tile_chunks) {
    if constexpr (kOut == Out::kOne) {
        const uint32_t tile0 = g * tile_chunks;
        const uint32_t left = nslice - tile0;
        return {0u, (size_t)tile0, (left < tile_chunks ? left : tile_chunks) * 16u};
    } else {
        const uint32_t s = g / tiles_per_slice;
        const SliceTile st = slice_tile(s, g - s * tiles_per_slice, nslice, tile_chunks);
        return {s, st.first, st.chunks * 16u};
    }
}

// One batch: tiles g0, g0 + stride, ... (kBatch of them).  kAllValid: every
// tile of the batch exists, so the loads of consecutive tiles are free to
// overlap; otherwise each tile is guarded (a workgroup's last batch).
template <int N, Out kOut, int kBatch, bool kAllValid>
__device__ __forceinline__ void reduce_batch(const Ptrs<const u32x4*>& src, const Ptrs<u32x4*>& dst,
                                             uint32_t nslice, uint32_t tiles_per_slice,
                                             uint32_t ntiles, uint32_t g0, uint32_t stride) {
    constexpr int U = 4;
    constexpr uint32_t kTile = kBlock * U;
    const uint32_t t = threadIdx.x;
    u32x4 o[kBatch][U];
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
        const uint32_t g = g0 + j * stride;
        if (!kAllValid && g >= ntiles) continue;  // uniform for the workgroup
        const TileAt at = tile_at<kOut>(g, nslice, tiles_per_slice, kTile);
        u32x4 v[U][N];
#pragma unroll
        for (int r = 0; r < N; ++r) {
            const __amdgpu_buffer_rsrc_t rs = tile_rsrc(src.p[r] + at.first, at.bytes);
#pragma unroll
            for (int u = 0; u < U; ++u) v[u][r] = load16_tile(rs, (u * kBlock + t) * 16u);
        }
#pragma unroll
        for (int u = 0; u < U; ++u) o[j][u] = fold_chunk<N>(v[u]);
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
        const uint32_t g = g0 + j * stride;
        if (!kAllValid && g >= ntiles) continue;
        const TileAt at = tile_at<kOut>(g, nslice, tiles_per_slice, kTile);
        constexpr int kFan = kOut == Out::kAll ? N : 1;
#pragma unroll
        for (int f = 0; f < kFan; ++f) {
            const int d = kOut == Out::kAll ? f : (kOut == Out::kOwner ? (int)at.s : 0);
            const __amdgpu_buffer_rsrc_t ro = tile_rsrc(dst.p[d] + at.first, at.bytes);
#pragma unroll
            for (int u = 0; u < U; ++u) store16_tile(ro, (u * kBlock + t) * 16u, o[j][u]);
        }
    }
}

template <int N, Out kOut>
__global__ __launch_bounds__(kBlock) __attribute__((amdgpu_waves_per_eu(2)))
void k_reduce_persistent(Ptrs<const u32x4*> src, Ptrs<u32x4*> dst, uint32_t nslice,
                         uint32_t tiles_per_slice, uint32_t ntiles) {
    constexpr int kBatch = batch_tiles<N, kOut>();
    const uint32_t stride = gridDim.x;
    for (uint32_t g0 = blockIdx.x; g0 < ntiles; g0 += stride * kBatch) {
        if (g0 + (kBatch - 1) * stride < ntiles)
            reduce_batch<N, kOut, kBatch, true>(src, dst, nslice, tiles_per_slice, ntiles, g0, stride);
        else
            reduce_batch<N, kOut, kBatch, false>(src, dst, nslice, tiles_per_slice, ntiles, g0, stride);
    }
}

// ---- bandwidth regime: LDS-staged persistent slice reduce --------------------------
// The oneshot reduce and twoshot phase 1 beyond the caches: one workgroup per
// CU, every wave streaming its rows through LDS stages (pc_staged.hpp), the
// batch's results held in registers and stored after a barrier.  The grid
// is sized to whole rounds of one workgroup per CU, with equal tiles per
// workgroup (to within one); grid tile g is tile_at(g), so slices keep the
// 128-byte-aligned tiling.  Compared with k_reduce_persistent, whose loads
// land in registers, at 8 ranks x 64 MiB on two MI355X boxes, interleaved:
// 88.0 - 88.4 us against 90.9 - 91.6 us, and 90.1 - 90.7 against 91.7 - 92.0.
// kWhole: every tile is a whole 1024 chunks (the slice length is a multiple
// of the tile), so the tile size is a constant rather than a value per tile,
// and fewer scalar registers stay live across a batch (with a size per tile
// they spill to VGPR lanes).  At 8 ranks x 64 MiB, interleaved on one
// MI355X: 87.9 vs 89.5 us (91.7 vs 92.9 on a slower box).  kDiagonal: the
// ranks' loads run on a diagonal (DiagonalBatch in pc_staged.hpp), chosen
// by bases_congruent from the rank buffers' addresses.
template <int N, Out kOut, bool kWhole, bool kDiagonal>
__global__ __launch_bounds__(kStageBlock) __attribute__((amdgpu_waves_per_eu(1, 1)))
void k_reduce_staged(Ptrs<const u32x4*> src, Ptrs<u32x4*> dst, uint32_t nslice,
                     uint32_t tiles_per_slice, uint32_t ntiles) {
    static_assert(kOut != Out::kAll, "the fan-out keeps the register kernel");
    PC_STAGE_ARRAYS(N)
    const uint32_t lane = threadIdx.x & 63, w = threadIdx.x >> 6, stride = gridDim.x;
    for_each_stage_batch([&](auto tiles, uint32_t g0) {
        constexpr int kTiles = decltype(tiles)::value;
        StageTile tile[kTiles];
        uint32_t slice[kTiles];
#pragma unroll
        for (int j = 0; j < kTiles; ++j) {
            const TileAt at = tile_at<kOut>(g0 + j * stride, nslice, tiles_per_slice, kStageTileChunks);
            tile[j] = {at.first, kWhole ? kStageTileChunks * 16u : at.bytes};
            slice[j] = at.s;
        }
        std::conditional_t<kDiagonal, DiagonalBatch<N, kTiles>, StagedBatch<N, false, kTiles>> b{
            src, tile, {PC_STAGE_LIST}, w, lane};
        b.run();
        __syncthreads();
#pragma unroll
        for (int j = 0; j < 4 * kTiles; ++j) {
            const StageTile t = tile[j / 4];
            const __amdgpu_buffer_rsrc_t ro =
                tile_rsrc(dst.p[kOut == Out::kOne ? 0 : slice[j / 4]] + t.first, t.bytes);
            store16_tile(ro, stage_row_offset(j, w, lane), b.res[j]);
        }
    }, ntiles);
}

// ---- single-launch twoshot, bandwidth regime: fold, then hand out ---------------
// Each workgroup first folds its tiles as twoshot phase 1 does, into the
// owner's output only (N input streams, one output stream), and only then
// reads those tiles back and writes them to the N-1 other outputs (one input
// stream, N-1 output streams, non-temporal as in the copy-out at these
// sizes): the two-launch form's traffic in one launch.  No workgroup reads
// what another one wrote.  Every byte position belongs to one tile, and
// every access to it, in any buffer, is made by the workgroup that owns that
// tile; a lane reads back exactly the chunks it stored, after all of the
// workgroup's stores have completed, with device-scope loads that the L2
// serves (the stores wrote through to it).  So no flag, no fence between
// workgroups and no workspace is needed, and exact aliasing of inputs and
// outputs stays safe.
template <int N>
__global__ __launch_bounds__(kBlock) __attribute__((amdgpu_waves_per_eu(2)))
void k_twoshot_persistent(Ptrs<const u32x4*> src, Ptrs<u32x4*> dst, uint32_t nslice,
                          uint32_t tiles_per_slice, uint32_t ntiles) {
    constexpr int kBatch = batch_tiles<N, Out::kOwner>();
    constexpr int U = 4;
    constexpr uint32_t kTile = kBlock * U;
    const uint32_t stride = gridDim.x;
    for (uint32_t g0 = blockIdx.x; g0 < ntiles; g0 += stride * kBatch) {
        if (g0 + (kBatch - 1) * stride < ntiles)
            reduce_batch<N, Out::kOwner, kBatch, true>(src, dst, nslice, tiles_per_slice, ntiles, g0, stride);
        else
            reduce_batch<N, Out::kOwner, kBatch, false>(src, dst, nslice, tiles_per_slice, ntiles, g0, stride);
    }
    __builtin_amdgcn_s_waitcnt(0);  // this wave's stores have completed
    __syncthreads();
    const uint32_t t = threadIdx.x;
    for (uint32_t g = blockIdx.x; g < ntiles; g += stride) {
        const TileAt at = tile_at<Out::kOwner>(g, nslice, tiles_per_slice, kTile);
        const __amdgpu_buffer_rsrc_t rs = tile_rsrc(dst.p[at.s] + at.first, at.bytes);
        u32x4 v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) v[u] = load16_rsrc<kPolicyDeviceScope>(rs, (u * kBlock + t) * 16u);
#pragma unroll
        for (int r = 0; r < N; ++r) {
            const __amdgpu_buffer_rsrc_t rd = tile_rsrc(dst.p[r] + at.first, (uint32_t)r == at.s ? 0u : at.bytes);
#pragma unroll
            for (int u = 0; u < U; ++u) store16_rsrc<kPolicyNonTemporal>(rd, (u * kBlock + t) * 16u, v[u]);
            // One output's stores at a time per wave: 168.3 vs 174.8 us at
            // 8 ranks x 64 MiB (174 vs 196 on another MI355X), level at the
            // other sizes and rank counts measured.
            wait_vm<0>();
        }
    }
}

// ---- twoshot copy-out: the owner's slice goes to every other rank's output ----
// Grid: x = tile within a slice, y = slice s.  Reads outs[s] once per chunk
// and writes it to the N-1 other outputs.  Tile-sized buffer resources clamp
// the ragged last tile, and the owner's own range gets a zero-length
// resource, so a lane's N-1 stores issue back to back with no branch (a
// branch per destination made each store wait for the one before it).
// kStorePolicy: the copies' cache policy (default, or non-temporal once the
// outputs are far larger than the last-level cache).
template <int N, int U, int kStorePolicy>
__global__ __launch_bounds__(kBlock) void k_copyout(Ptrs<u32x4*> outs, uint32_t nslice) {
    constexpr uint32_t kTile = kBlock * U;
    const uint32_t s = blockIdx.y;
    const SliceTile st = slice_tile(s, blockIdx.x, nslice, kTile);
    const size_t first = st.first;
    const uint32_t bytes = st.chunks * 16u;
    const uint32_t t = threadIdx.x;
    const __amdgpu_buffer_rsrc_t rs = tile_rsrc(outs.p[s] + first, bytes);
    u32x4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = load16_rsrc<0>(rs, (u * kBlock + t) * 16u);
#pragma unroll
    for (int r = 0; r < N; ++r) {
        const __amdgpu_buffer_rsrc_t rd = tile_rsrc(outs.p[r] + first, (uint32_t)r == s ? 0u : bytes);
#pragma unroll
        for (int u = 0; u < U; ++u) store16_rsrc<kStorePolicy>(rd, (u * kBlock + t) * 16u, v[u]);
    }
}

// ---- twoshot copy-out, one destination per workgroup (bandwidth regime) --------
// Work item w copies one 4 KiB tile of one slice into one other output.  The
// N-1 items of a tile get ids with the same remainder mod 8, and workgroups
// are dispatched round-robin over the MI355X's 8 XCDs, so the N-1 copies of a
// tile run on one XCD and all but the first read of it hit that XCD's L2.
// HBM takes writes fastest from many short-lived workgroups that each write
// a few KiB; k_copyout keeps up to (N-1) x 8 KiB of stores in flight per
// workgroup.  At 8 ranks x 64 MiB, interleaved on one MI355X: 74.9 vs 85.8 us
// for the copy-out, 168.9 vs 180.2 us for the whole call (the same work items
// without the XCD grouping: 126.7 us).  From a grid cap of about 4M
// workgroups a workgroup takes every grid-th item, keeping its remainder.
constexpr uint32_t kXcds = 8;
constexpr uint32_t kCopyDestGridCap = 1u << 22;
constexpr int kCopyDestMinRanks = 7;

template <int N>
__global__ __launch_bounds__(kBlock) void k_copyout_dest(Ptrs<u32x4*> outs, uint32_t nslice,
                                                         uint32_t tiles_per_slice, uint32_t items) {
    const uint32_t ntiles = tiles_per_slice * N;
    const uint32_t t = threadIdx.x;
    for (uint32_t w = blockIdx.x; w < items; w += gridDim.x) {
        const uint32_t rest = w / kXcds;
        const uint32_t tile = rest / (N - 1) * kXcds + w % kXcds;
        if (tile >= ntiles) continue;  // the last group of 8 tiles may be partial
        const uint32_t di = rest % (N - 1);
        const uint32_t s = tile / tiles_per_slice;
        const uint32_t r = di < s ? di : di + 1;  // every output but the owner's
        const SliceTile st = slice_tile(s, tile - s * tiles_per_slice, nslice, kBlock);
        const uint32_t bytes = st.chunks * 16u;
        const u32x4 v = load16_rsrc<0>(tile_rsrc(outs.p[s] + st.first, bytes), t * 16u);
        store16_rsrc<kPolicyNonTemporal>(tile_rsrc(outs.p[r] + st.first, bytes), t * 16u, v);
    }
}

// ---- bandwidth regime with one to three ranks: short-lived workgroups --------------
// k_reduce with two chunks per lane (8 KiB tiles) and non-temporal loads:
// workgroups that fold one tile and end.  With few input streams the writes
// are a large share of the traffic, and HBM takes writes fastest from many
// short-lived workgroups (as for the Atom copy and k_copyout_dest).  At
// 128 MiB per rank, against the persistent kernel: 1 rank 37.6 vs 41.6 us,
// 2 ranks 55.9 vs 61.3, 3 ranks 77.9 vs 81.4; at 512 MiB 168 vs 216, 264 vs
// 310 and 355 vs 403.  At 32-64 MiB per rank two and three ranks are level
// or slower this way (2 ranks, 64 MiB: 29.3 vs 28.4 us), one rank is faster
// at every size (64 MiB: 17.8 vs 18.8).  From four ranks the staged kernel
// stays ahead (8 ranks, 256 MiB: 364 vs 387 us).

// ---- launch table ---------------------------------------------------------------
// Shapes by payload: small payloads (latency regime) take one chunk per lane
// so the most workgroups start at once; mid payloads take two; payloads with
// a working set of 64 MiB or more use the bandwidth-regime kernels above
// (staged from four ranks, short-lived or persistent below that).
enum class Regime { kSmall, kMid, kStream };

// Compute units of the current device, looked up once per device (256 if
// the query fails).
uint32_t device_cus() {
    static int cached[64] = {};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    int cus = __atomic_load_n(&cached[dev], __ATOMIC_RELAXED);
    if (cus <= 0) {
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
            cus <= 0)
            cus = 256;
        __atomic_store_n(&cached[dev], cus, __ATOMIC_RELAXED);
    }
    return (uint32_t)cus;
}

// `working_set` is the bytes one call reads plus the bytes it writes.  The
// bandwidth-regime kernels take over from 64 MiB: measured with inputs not in
// the caches (the common case, since peers have just written them) they are
// ahead from 8 MiB per rank at N = 8, and with warm caches within 2%.
static Regime pick_regime(size_t nchunks_per_rank, size_t working_set) {
    if (working_set >= ((size_t)64 << 20)) return Regime::kStream;
    if (nchunks_per_rank >= (size_t)kBlock * 2 * 512) return Regime::kMid;
    return Regime::kSmall;
}

// Bytes per rank from which the twoshot forms store with device scope
// (k_reduce rather than k_reduce_small, and the copy-out likewise).
constexpr size_t kScopeStoreRankBytes = (size_t)128 << 10;

template <int N, int U, int kLoadPolicy, Out kOut>
static hipError_t go_reduce(Ptrs<const u32x4*> src, Ptrs<u32x4*> dst, uint32_t nslice,
                            uint32_t slices, hipStream_t stream) {
    // At most 2^31 chunks per rank: below 2^23 tiles per slice.
    constexpr uint32_t kTile = kBlock * U;
    dim3 grid(slice_tiles(nslice, slices, kTile), slices);
    void* args[] = {&src, &dst, &nslice};
    const bool small = kOut != Out::kOne && (size_t)nslice * slices * 16 < kScopeStoreRankBytes;
    const void* k = small ? (const void*)&k_reduce_small<N, U, kOut>
                          : (const void*)&k_reduce<N, U, kLoadPolicy, kOut>;
    return hipLaunchKernel(k, grid, dim3(kBlock), args, 0, stream);
}

template <int N, Out kOut>
static hipError_t go_reduce_persistent(Ptrs<const u32x4*> src, Ptrs<u32x4*> dst, uint32_t nslice,
                                       uint32_t slices, hipStream_t stream) {
    constexpr uint32_t kTile = kBlock * 4;
    uint32_t tiles_per_slice = slice_tiles(nslice, slices, kTile);
    uint32_t ntiles = tiles_per_slice * slices;
    // Whole rounds of at most two workgroups per CU, then as few workgroups
    // as give that many rounds, so every workgroup does the same number of
    // tiles (to within one).
    const uint32_t slots = 2 * device_cus();
    const uint32_t rounds = (ntiles + slots - 1) / slots;
    const uint32_t grid = (ntiles + rounds - 1) / rounds;
    void* args[] = {&src, &dst, &nslice, &tiles_per_slice, &ntiles};
    return hipLaunchKernel((const void*)&k_reduce_persistent<N, kOut>, dim3(grid), dim3(kBlock),
                           args, 0, stream);
}

// The staged kernel serves four or more ranks.  A/B against the register
// kernel on one MI355X, warm / caches flushed, us: 8 ranks 4.7 / 10.1 vs
// 5.1-5.7 / 10.7-11.1 at 4 MiB per rank, 17.0 / 22.2 vs 18.4 / 22.5 at 12,
// 45.2 / 50.5 vs 45.3 / 50.9 at 32, 90.1-90.7 / 93.7-94.5 vs 91.7-92.0 /
// 96.8-96.9 at 64; 6 ranks 69.8-70.6 vs 71.8-72.2 and 4 ranks 49.7-51.4 vs
// 51.2-51.4 at 64.  With 2 ranks it lost (29.4 vs 28.5-28.9 warm, 35.7 vs
// 33.2-33.7 flushed at 64 MiB), so fewer ranks keep the register kernel.
// Whole rounds of one workgroup per CU, then as few workgroups as give that
// many rounds, so every workgroup does the same number of tiles (to within
// one).  The dynamic LDS request keeps a second workgroup off each CU.
template <int N, Out kOut>
static hipError_t go_reduce_staged(Ptrs<const u32x4*> src, Ptrs<u32x4*> dst, uint32_t nslice,
                                   uint32_t slices, hipStream_t stream) {
    uint32_t tiles_per_slice = slice_tiles(nslice, slices, kStageTileChunks);
    uint32_t ntiles = tiles_per_slice * slices;
    const uint32_t cus = device_cus();
    const uint32_t rounds = (ntiles + cus - 1) / cus;
    const uint32_t grid = (ntiles + rounds - 1) / rounds;
    void* args[] = {&src, &dst, &nslice, &tiles_per_slice, &ntiles};
    // Slices that are whole numbers of tiles start on the 128-byte grid, so
    // every tile of every slice is whole.
    const bool whole = nslice % kStageTileChunks == 0;
    const bool diagonal = bases_congruent((const void* const*)src.p, N);
    const void* k = whole ? (diagonal ? (const void*)&k_reduce_staged<N, kOut, true, true>
                                      : (const void*)&k_reduce_staged<N, kOut, true, false>)
                          : (diagonal ? (const void*)&k_reduce_staged<N, kOut, false, true>
                                      : (const void*)&k_reduce_staged<N, kOut, false, false>);
    return hipLaunchKernel(k, dim3(grid), dim3(kStageBlock), args, stage_pad_bytes<N>(), stream);
}

// Bytes per rank from which two or three ranks take the short-lived
// k_reduce (one rank takes it throughout the bandwidth regime).
constexpr size_t kShortMinRankBytes = (size_t)128 << 20;

template <int N, Out kOut>
static hipError_t go_reduce_regime(Regime rg, Ptrs<const u32x4*> src, Ptrs<u32x4*> dst,
                                   uint32_t nslice, uint32_t slices, hipStream_t stream) {
    switch (rg) {
        case Regime::kStream:
            if constexpr (kOut != Out::kAll && N < kStageMinRanks)
                if (N == 1 || (size_t)nslice * slices * 16 >= kShortMinRankBytes)
                    return go_reduce<N, 2, kPolicyNonTemporal, kOut>(src, dst, nslice, slices, stream);
            if constexpr (kOut == Out::kAll || N < kStageMinRanks)
                return go_reduce_persistent<N, kOut>(src, dst, nslice, slices, stream);
            else return go_reduce_staged<N, kOut>(src, dst, nslice, slices, stream);
        case Regime::kMid: return go_reduce<N, 2, 0, kOut>(src, dst, nslice, slices, stream);
        default: return go_reduce<N, 1, 0, kOut>(src, dst, nslice, slices, stream);
    }
}

template <Out kOut>
static hipError_t dispatch_reduce(int n, Regime rg, Ptrs<const u32x4*> src, Ptrs<u32x4*> dst,
                                  uint32_t nslice, uint32_t slices, hipStream_t stream) {
    switch (n) {
        case 1: return go_reduce_regime<1, kOut>(rg, src, dst, nslice, slices, stream);
        case 2: return go_reduce_regime<2, kOut>(rg, src, dst, nslice, slices, stream);
        case 3: return go_reduce_regime<3, kOut>(rg, src, dst, nslice, slices, stream);
        case 4: return go_reduce_regime<4, kOut>(rg, src, dst, nslice, slices, stream);
        case 5: return go_reduce_regime<5, kOut>(rg, src, dst, nslice, slices, stream);
        case 6: return go_reduce_regime<6, kOut>(rg, src, dst, nslice, slices, stream);
        case 7: return go_reduce_regime<7, kOut>(rg, src, dst, nslice, slices, stream);
        case 8: return go_reduce_regime<8, kOut>(rg, src, dst, nslice, slices, stream);
        default: return hipErrorInvalidValue;
    }
}

// From 48 MiB per rank, where the two policies are level at 8 ranks, the
// copies carry the non-temporal hint: 181 vs 192 us at 64 MiB per rank and
// 269 vs 310 us at 96 MiB.  Below it the default policy is faster (87 vs
// 92 us at 32 MiB), because the copies still find room in the caches.  At
// 7 and 8 ranks the copies then go one destination per workgroup
// (k_copyout_dest); with fewer ranks that kernel measured level (4 to 6
// ranks, within 1-3% either way at 64 and 96 MiB per rank) and is not used.
constexpr size_t kCopyoutStreamBytes = (size_t)48 << 20;

template <int N>
static hipError_t go_copyout_dest(Ptrs<u32x4*> outs, uint32_t nslice, hipStream_t stream) {
    uint32_t tiles_per_slice = slice_tiles(nslice, N, kBlock);
    const uint32_t groups = (tiles_per_slice * N + kXcds - 1) / kXcds;
    uint32_t items = groups * kXcds * (N - 1);
    constexpr uint32_t kCap = kCopyDestGridCap / (kXcds * (N - 1)) * (kXcds * (N - 1));
    const uint32_t grid = items < kCap ? items : kCap;  // a multiple of 8 either way
    void* args[] = {&outs, &nslice, &tiles_per_slice, &items};
    return hipLaunchKernel((const void*)&k_copyout_dest<N>, dim3(grid), dim3(kBlock), args, 0, stream);
}

template <int N>
static hipError_t go_copyout(Ptrs<u32x4*> outs, uint32_t nslice, uint32_t slices, bool wide,
                             bool nt, hipStream_t stream) {
    if constexpr (N >= kCopyDestMinRanks)
        if (nt) return go_copyout_dest<N>(outs, nslice, stream);
    void* args[] = {&outs, &nslice};
    if (wide) {
        dim3 grid(slice_tiles(nslice, slices, 2 * kBlock), slices);
        // Device-scope stores up to 8 MiB per rank (8 ranks, 4 MiB: 12.2 vs
        // 13.8 us per call in a graph), the default policy above (16 MiB: 45.4
        // vs 49.6 us with device scope), non-temporal from 48 MiB.
        const bool scoped = (size_t)nslice * slices * 16 < ((size_t)8 << 20);
        const void* k = nt       ? (const void*)&k_copyout<N, 2, kPolicyNonTemporal>
                        : scoped ? (const void*)&k_copyout<N, 2, kPolicyDeviceScope>
                                 : (const void*)&k_copyout<N, 2, 0>;
        return hipLaunchKernel(k, grid, dim3(kBlock), args, 0, stream);
    }
    // From 128 KiB per rank the cache-resident copy-out stores with device
    // scope, as the slice reduce before it (two-launch twoshot, 8 ranks, per
    // call in a graph: 3.83 vs 4.82 us at 256 KiB per rank, 5.55 vs 6.45 at
    // 1 MiB).
    dim3 grid(slice_tiles(nslice, slices, kBlock), slices);
    const bool scoped = (size_t)nslice * slices * 16 >= kScopeStoreRankBytes;
    return hipLaunchKernel(scoped ? (const void*)&k_copyout<N, 1, kPolicyDeviceScope> : (const void*)&k_copyout<N, 1, 0>,
                           grid, dim3(kBlock), args, 0, stream);
}

static void fill_src(Ptrs<const u32x4*>& p, const void* const* src, int n) {
    for (int r = 0; r < kMaxRanks; ++r) p.p[r] = r < n ? static_cast<const u32x4*>(src[r]) : nullptr;
}

hipError_t launch_reduce(const void* const* src, int n, void* out, size_t nchunks,
                         hipStream_t stream) {
    Ptrs<const u32x4*> s;
    Ptrs<u32x4*> d = {};
    fill_src(s, src, n);
    d.p[0] = static_cast<u32x4*>(out);
    const Regime rg = pick_regime(nchunks, nchunks * 16 * (size_t)(n + 1));
    return dispatch_reduce<Out::kOne>(n, rg, s, d, (uint32_t)nchunks, 1, stream);
}

hipError_t launch_twoshot(const void* const* src, int n, void* const* outs, size_t nchunks_slice,
                          hipStream_t stream) {
    Ptrs<const u32x4*> s;
    Ptrs<u32x4*> d = {};
    fill_src(s, src, n);
    for (int r = 0; r < n; ++r) d.p[r] = static_cast<u32x4*>(outs[r]);
    const size_t per_rank = nchunks_slice * (size_t)n;
    const Regime rg = pick_regime(per_rank, per_rank * 16 * (size_t)(n + 1));
    hipError_t e =
        dispatch_reduce<Out::kOwner>(n, rg, s, d, (uint32_t)nchunks_slice, (uint32_t)n, stream);
    if (e != hipSuccess || n == 1) return e;
    const bool wide = rg != Regime::kSmall;
    const bool nt = per_rank * 16 >= kCopyoutStreamBytes;
    switch (n) {
        case 2: return go_copyout<2>(d, (uint32_t)nchunks_slice, n, wide, nt, stream);
        case 3: return go_copyout<3>(d, (uint32_t)nchunks_slice, n, wide, nt, stream);
        case 4: return go_copyout<4>(d, (uint32_t)nchunks_slice, n, wide, nt, stream);
        case 5: return go_copyout<5>(d, (uint32_t)nchunks_slice, n, wide, nt, stream);
        case 6: return go_copyout<6>(d, (uint32_t)nchunks_slice, n, wide, nt, stream);
        case 7: return go_copyout<7>(d, (uint32_t)nchunks_slice, n, wide, nt, stream);
        case 8: return go_copyout<8>(d, (uint32_t)nchunks_slice, n, wide, nt, stream);
        default: return hipErrorInvalidValue;
    }
}

// The single-launch twoshot folds first and hands out after (the kernel
// above) from a working set, inputs plus outputs, of 640 MiB (two and a half
// times the last-level cache) with five or more ranks.  A/B on one MI355X, µs,
// the kernel above against the single fan-out pass: 8 ranks 229 vs 246-249
// at 64 MiB per rank, 168-170 vs 176 at 48; 7 ranks 215 vs 244 at 72 MiB;
// 6 ranks 163 vs 172-175 at 64 MiB; 5 ranks 171-173 vs 191-195 at 96 MiB.
// On another MI355X: 8 ranks 112-113 vs 119 at 40 MiB and 128-129 vs 141-142
// at 44, but 103 vs 99-100 at 36 (a 576 MiB working set).  The read-back
// adds 1/n of the traffic, so with fewer ranks the fan-out pass stays ahead
// (4 ranks: even at 128 MiB per rank, 104 vs 84-85 at 64).
constexpr size_t kSplitWorkingSet = (size_t)640 << 20;
constexpr int kSplitMinRanks = 5;

template <int N>
static hipError_t go_twoshot_split(Ptrs<const u32x4*> src, Ptrs<u32x4*> dst, uint32_t nslice,
                                   hipStream_t stream) {
    constexpr uint32_t kTile = kBlock * 4;
    uint32_t tiles_per_slice = slice_tiles(nslice, N, kTile);
    uint32_t ntiles = tiles_per_slice * N;
    const uint32_t slots = 2 * device_cus();
    const uint32_t rounds = (ntiles + slots - 1) / slots;
    const uint32_t grid = (ntiles + rounds - 1) / rounds;
    void* args[] = {&src, &dst, &nslice, &tiles_per_slice, &ntiles};
    return hipLaunchKernel((const void*)&k_twoshot_persistent<N>, dim3(grid), dim3(kBlock), args, 0,
                           stream);
}

hipError_t launch_twoshot_fused(const void* const* src, int n, void* const* outs,
                                size_t nchunks_slice, hipStream_t stream) {
    Ptrs<const u32x4*> s;
    Ptrs<u32x4*> d = {};
    fill_src(s, src, n);
    for (int r = 0; r < n; ++r) d.p[r] = static_cast<u32x4*>(outs[r]);
    // Working set: every input read once and every output written once.
    const size_t per_rank = nchunks_slice * (size_t)n;
    const Regime rg = pick_regime(per_rank, per_rank * 16 * 2 * (size_t)n);
    if (n >= kSplitMinRanks && per_rank * 16 * 2 * (size_t)n >= kSplitWorkingSet) {
        const uint32_t ns = (uint32_t)nchunks_slice;
        switch (n) {
            case 5: return go_twoshot_split<5>(s, d, ns, stream);
            case 6: return go_twoshot_split<6>(s, d, ns, stream);
            case 7: return go_twoshot_split<7>(s, d, ns, stream);
            case 8: return go_twoshot_split<8>(s, d, ns, stream);
            default: return hipErrorInvalidValue;
        }
    }
    return dispatch_reduce<Out::kAll>(n, rg, s, d, (uint32_t)nchunks_slice, (uint32_t)n, stream);
}

}  // namespace pcdp
