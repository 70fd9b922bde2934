// pc_device.hpp -- device-side building blocks of the gfx950 datapath kernels.
//
// Element arithmetic follows "Purlin: Separating Orchestration from the
// Datapath of Collectives", Section 3.3, Equation (2): every bf16 contribution
// is widened to fp32, contributions are added in a fixed rank order in fp32,
// and the finished sum is rounded back to bf16.  Rounding is to nearest,
// ties to even; every NaN becomes the canonical quiet NaN 0x7FC0, so a NaN
// result has exactly one bit pattern whichever operand's payload the adder
// would have kept.  Subnormals are kept: the library is compiled with
// -fno-gpu-flush-denormals-to-zero and without contraction.
//
// Memory is moved in 16-byte units (global_load_dwordx4 / global_store_dwordx4)
// so that a wave64 touches 1 KiB contiguous per instruction.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pcdp {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef int32_t i32x4 __attribute__((ext_vector_type(4)));

constexpr int kMaxRanks = 8;
constexpr int kWave = 64;

// Pointer bundles passed by value as kernel arguments (they live in SGPRs).
template <typename T>
struct Ptrs {
    T p[kMaxRanks];
};

// ---- loads and stores -------------------------------------------------------
// A 16-byte store through a 64-bit address; the streaming (non-temporal)
// variant keeps data that is written once from evicting data that is reused.
template <bool kStream>
__device__ __forceinline__ void store16(u32x4* p, u32x4 v) {
    if constexpr (kStream) __builtin_nontemporal_store(v, p);
    else *p = v;
}

// Buffer-resource access for the bandwidth regime.  A resource covers one
// tile, [base, base + bytes), with a scalar base address, so every lane
// addresses with a 32-bit offset.  The hardware range check makes a ragged
// last tile branch-free: loads past `bytes` return zero and stores past it
// are discarded (offsets and `bytes` are multiples of 16, so a 16-byte
// access is either wholly inside or wholly outside).
// Loads carry the non-temporal hint; stores use device-scope cache policy
// (sc1) without it, which GPU measurements showed is markedly better for HBM
// than non-temporal stores when writes are mixed into a large read stream.
constexpr int kRsrcWord3 = 0x00020000;    // raw (untyped) buffer access on gfx9
constexpr int kPolicyNonTemporal = 0x02;  // nt
constexpr int kPolicyDeviceScope = 0x10;  // sc1

__device__ __forceinline__ __amdgpu_buffer_rsrc_t tile_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                             kRsrcWord3);
}

// 16-byte buffer load / store at `byte_off` with cache policy kPolicy (0 =
// default).  A resource of zero bytes turns every store into a no-op, which
// lets a loop over destinations skip one of them without a branch.
template <int kPolicy>
__device__ __forceinline__ u32x4 load16_rsrc(__amdgpu_buffer_rsrc_t rs, uint32_t byte_off) {
    return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, byte_off, 0, kPolicy));
}

template <int kPolicy>
__device__ __forceinline__ void store16_rsrc(__amdgpu_buffer_rsrc_t rs, uint32_t byte_off, u32x4 v) {
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(i32x4, v), rs, byte_off, 0, kPolicy);
}

__device__ __forceinline__ u32x4 load16_tile(__amdgpu_buffer_rsrc_t rs, uint32_t byte_off) {
    return load16_rsrc<kPolicyNonTemporal>(rs, byte_off);
}

__device__ __forceinline__ void store16_tile(__amdgpu_buffer_rsrc_t rs, uint32_t byte_off, u32x4 v) {
    store16_rsrc<kPolicyDeviceScope>(rs, byte_off, v);
}

// ---- tiles of a slice ---------------------------------------------------------
// Slice s of `nslice` chunks starts at chunk s*nslice.  Its tiles of up to
// `tile` chunks lie on a grid aligned to 8 chunks (128 bytes, one cache line)
// of the buffer: tile j covers [base + j*tile, base + (j+1)*tile) clipped to
// the slice, where base is the slice start rounded down to 8 chunks, so only
// a slice's first tile can start off a line.  Tiles cut from an unaligned
// slice start would put every wave access across cache lines.
struct SliceTile {
    size_t first;     // first chunk
    uint32_t chunks;  // 0 .. tile
};

__host__ __device__ inline SliceTile slice_tile(uint32_t s, uint32_t j, size_t nslice, uint32_t tile) {
    const size_t start = (size_t)s * nslice, end = start + nslice;
    size_t lo = (start & ~(size_t)7) + (size_t)j * tile;
    size_t hi = lo + tile;
    lo = lo < start ? start : lo;
    lo = lo > end ? end : lo;
    hi = hi > end ? end : hi;
    return {lo, (uint32_t)(hi - lo)};
}

// Tiles per slice: the most that any of `slices` slices needs.
__host__ __device__ inline uint32_t slice_tiles(size_t nslice, uint32_t slices, uint32_t tile) {
    size_t most = 0;
    for (uint32_t s = 0; s < slices; ++s) {
        const size_t n = (nslice + ((size_t)s * nslice) % 8 + tile - 1) / tile;
        most = n > most ? n : most;
    }
    return (uint32_t)most;
}

// ---- bf16 <-> fp32 ----------------------------------------------------------
// A 32-bit word holds two bf16: element 2i in bits 0..15, element 2i+1 in
// bits 16..31.  Widening is exact: the bf16 bits become the upper fp32 half.
__device__ __forceinline__ float widen_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float widen_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// fp32 -> bf16 rounded to nearest even, left in the upper 16 bits of the
// returned word (the lower 16 bits are junk).  Adding 0x7FFF plus the kept
// value's lowest bit rounds ties to even; a carry into the exponent is the
// right answer and carries out of the largest finite value give +-Inf.
__device__ __forceinline__ uint32_t round_bf16_hi(float f) {
    const uint32_t u = __float_as_uint(f);
    const uint32_t r = u + 0x7FFFu + ((u >> 16) & 1u);
    return ((u & 0x7FFFFFFFu) > 0x7F800000u) ? 0x7FC00000u : r;
}

// Two fp32 sums -> one word of two bf16 (lo -> bits 0..15, hi -> 16..31).
__device__ __forceinline__ uint32_t narrow_pair(float lo, float hi) {
    return (round_bf16_hi(hi) & 0xFFFF0000u) | (round_bf16_hi(lo) >> 16);
}

// ---- the rank-ordered fold of one 16-byte chunk -------------------------------
// v[r] holds 8 bf16 of rank r's chunk; the result holds the 8 sums.  Each of
// the 8 lanes-within-the-chunk has its own accumulator that starts at -0.0f
// and takes ranks 0, 1, ..., N-1 in that order; no term is ever combined with
// another before it reaches the accumulator.
template <int N>
__device__ __forceinline__ u32x4 fold_chunk(const u32x4 (&v)[N]) {
    float lo[4], hi[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        lo[e] = -0.0f;
        hi[e] = -0.0f;
    }
#pragma unroll
    for (int r = 0; r < N; ++r) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            lo[e] = lo[e] + widen_lo(v[r][e]);
            hi[e] = hi[e] + widen_hi(v[r][e]);
        }
    }
    u32x4 o;
#pragma unroll
    for (int e = 0; e < 4; ++e) o[e] = narrow_pair(lo[e], hi[e]);
    return o;
}

}  // namespace pcdp
