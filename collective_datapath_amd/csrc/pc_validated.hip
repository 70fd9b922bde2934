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
// Tile b (elems_per_flag elements, one workgroup) is validated by flag word b
// of every rank.  The retry loop is bounded by max_attempts so every kernel
// ends; attempts[b] receives the attempt that validated (1-based) or 0.
#include "pc_device.hpp"
#include "pc_launch.hpp"

namespace pcdp {

constexpr int kVBlock = 256;

// One attempt's reads.  The first attempt reads payload and flags the
// default way, so they may come from the caches; a stale cached flag holds
// an earlier call's value, which only makes the check fail.  A retry must
// not be served stale data, so it reads both device-coherently.  Policy and
// scope are template parameters, so each attempt is one straight block of
// loads.
template <int N, int U, int kPolicy>
__device__ __forceinline__ void load_payload(u32x4 (&v)[U][N], const Ptrs<const u32x4*>& src,
                                             size_t first, uint32_t t) {
    constexpr uint32_t kTile = kVBlock * U;
#pragma unroll
    for (int r = 0; r < N; ++r) {
        const __amdgpu_buffer_rsrc_t rs = tile_rsrc(src.p[r] + first, kTile * 16u);
#pragma unroll
        for (int u = 0; u < U; ++u) v[u][r] = load16_rsrc<kPolicy>(rs, (u * kVBlock + t) * 16u);
    }
}

// The validation fold: the uint32 sum (mod 2^32) of every rank's flag b.
template <int N, int kScope>
__device__ __forceinline__ uint32_t fold_flags(const Ptrs<const uint32_t*>& flags, uint32_t b) {
    uint32_t folded = 0;
#pragma unroll
    for (int r = 0; r < N; ++r) folded += __hip_atomic_load(flags.p[r] + b, __ATOMIC_RELAXED, kScope);
    return folded;
}

// U = elems_per_flag / 2048: each lane folds U chunks of the tile.
template <int N, int U>
__global__ __launch_bounds__(kVBlock) void k_reduce_validated(Ptrs<const u32x4*> src,
                                                               Ptrs<const uint32_t*> flags,
                                                               u32x4* out, uint32_t flag,
                                                               uint32_t max_attempts,
                                                               uint32_t* attempts) {
    __shared__ uint32_t verdict;
    const uint32_t b = blockIdx.x, t = threadIdx.x;
    const size_t first = (size_t)b * (kVBlock * U);
    const uint32_t expect = (uint32_t)N * flag;
    uint32_t accepted = 0;
    for (uint32_t a = 1; a <= max_attempts; ++a) {
        u32x4 v[U][N];
        if (a == 1) load_payload<N, U, 0>(v, src, first, t);
        else load_payload<N, U, kPolicyDeviceScope>(v, src, first, t);
        if (t == 0) {
            const uint32_t folded = a == 1 ? fold_flags<N, __HIP_MEMORY_SCOPE_WORKGROUP>(flags, b)
                                           : fold_flags<N, __HIP_MEMORY_SCOPE_AGENT>(flags, b);
            verdict = folded == expect;
        }
        __syncthreads();
        const bool ok = verdict != 0;  // one decision for the whole workgroup
        if (ok) {
#pragma unroll
            for (int u = 0; u < U; ++u) out[first + u * kVBlock + t] = fold_chunk<N>(v[u]);
            accepted = a;
            break;
        }
        __syncthreads();  // every wave has read this attempt's verdict
    }
    if (t == 0) attempts[b] = accepted;
}

template <int N, int U>
static hipError_t go_validated(Ptrs<const u32x4*> s, Ptrs<const uint32_t*> f, u32x4* out,
                               uint32_t flag, uint32_t max_attempts, uint32_t* attempts,
                               size_t tiles, hipStream_t stream) {
    void* args[] = {&s, &f, &out, &flag, &max_attempts, &attempts};
    return hipLaunchKernel((const void*)&k_reduce_validated<N, U>, dim3((unsigned)tiles),
                           dim3(kVBlock), args, 0, stream);
}

template <int N>
static hipError_t go_validated_u(int u, Ptrs<const u32x4*> s, Ptrs<const uint32_t*> f, u32x4* out,
                                 uint32_t flag, uint32_t max_attempts, uint32_t* attempts,
                                 size_t tiles, hipStream_t stream) {
    switch (u) {
        case 1: return go_validated<N, 1>(s, f, out, flag, max_attempts, attempts, tiles, stream);
        case 2: return go_validated<N, 2>(s, f, out, flag, max_attempts, attempts, tiles, stream);
        case 3: return go_validated<N, 3>(s, f, out, flag, max_attempts, attempts, tiles, stream);
        case 4: return go_validated<N, 4>(s, f, out, flag, max_attempts, attempts, tiles, stream);
        default: return hipErrorInvalidValue;
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
