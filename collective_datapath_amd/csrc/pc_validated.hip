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
// Tile b (elems_per_flag elements, one workgroup of elems_per_flag / 8
// lanes) is validated by flag word b of every rank.  The retry loop is
// bounded by max_attempts so every kernel ends; attempts[b] receives the
// attempt that validated (1-based) or 0.
#include "pc_device.hpp"
#include "pc_launch.hpp"

namespace pcdp {

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
