// pc_api.hip -- the C ABI declared in include/pc.h: argument validation, the
// fold-order permutation, and dispatch to the kernel launchers.
//
// Admission follows the spirit of "flash-comm: Self-Synchronizing Collective
// Communication for LLM Decoding", Section 4.1: a call is checked before
// anything is launched (group size, 16-byte address and length alignment,
// size ceiling), and a rejected call has no side effect.  Empty payloads are
// legal no-ops so that every rank can issue the same call sequence
// (Section 4.2).  Nothing here allocates; the only state is the per-device
// address of the static workspace of pc_twoshot_linked_static.
#include "../../include/pc.h"
#include "pc_launch.hpp"

#include <hip/hip_runtime.h>

namespace {

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Half-open byte ranges [a, a+na) and [b, b+nb) intersect.
inline bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
    const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
    return x < y + nb && y < x + na;
}

inline bool valid_n(int n) { return n >= 1 && n <= PC_MAX_RANKS; }

bool is_permutation(const int32_t* order, int n) {
    bool seen[PC_MAX_RANKS] = {};
    for (int j = 0; j < n; ++j) {
        const int32_t r = order[j];
        if (r < 0 || r >= n || seen[r]) return false;
        seen[r] = true;
    }
    return true;
}

// Every pointer non-null (PC_EINVAL) and 16-byte aligned (PC_EALIGN).
template <typename T>
pc_status check_ptrs(const T* const* ptrs, int n) {
    for (int r = 0; r < n; ++r)
        if (!ptrs[r]) return PC_EINVAL;
    for (int r = 0; r < n; ++r)
        if (!aligned16(ptrs[r])) return PC_EALIGN;
    return PC_OK;
}

inline pc_status from_hip(hipError_t e) { return e == hipSuccess ? PC_OK : PC_EHIP; }

inline bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

inline bool aligned8(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 7u) == 0; }

}  // namespace

extern "C" {

pc_status pc_reduce(const uint16_t* const* inputs, int n, uint16_t* out, size_t k,
                    const int32_t* order, void* stream) {
    if (!valid_n(n) || !inputs) return PC_EINVAL;
    if (order && !is_permutation(order, n)) return PC_EINVAL;
    if (k > PC_MAX_ELEMS) return PC_EINVAL;
    if (k % 8) return PC_EALIGN;
    if (k == 0) return PC_OK;
    if (pc_status st = check_ptrs(inputs, n)) return st;
    if (!out) return PC_EINVAL;
    if (!aligned16(out)) return PC_EALIGN;
    const size_t bytes = k * sizeof(uint16_t);
    for (int r = 0; r < n; ++r)
        if (inputs[r] != out && overlaps(inputs[r], bytes, out, bytes)) return PC_EINVAL;
    const void* src[PC_MAX_RANKS];
    for (int j = 0; j < n; ++j) src[j] = inputs[order ? order[j] : j];
    return from_hip(pcdp::launch_reduce(src, n, out, k / 8, static_cast<hipStream_t>(stream)));
}

pc_status pc_copy(void* dst, const void* src, size_t bytes, void* stream) {
    if (bytes > 2 * PC_MAX_ELEMS) return PC_EINVAL;
    if (bytes % 16) return PC_EALIGN;
    if (bytes == 0) return PC_OK;
    if (!dst || !src) return PC_EINVAL;
    if (!aligned16(dst) || !aligned16(src)) return PC_EALIGN;
    if (dst == src) return PC_OK;  // copying a range onto itself changes nothing
    if (overlaps(dst, bytes, src, bytes)) return PC_EINVAL;
    return from_hip(pcdp::launch_copy(src, dst, bytes / 16, static_cast<hipStream_t>(stream)));
}

pc_status pc_pack_ll(const uint16_t* src, uint64_t* dst, size_t k, uint32_t seq, void* stream) {
    if (seq == 0 || k > PC_MAX_ELEMS) return PC_EINVAL;
    if (k % 8) return PC_EALIGN;
    if (k == 0) return PC_OK;
    if (!src || !dst) return PC_EINVAL;
    if (!aligned16(src) || !aligned16(dst)) return PC_EALIGN;
    if (overlaps(src, k * sizeof(uint16_t), dst, (k / 2) * sizeof(uint64_t))) return PC_EINVAL;
    return from_hip(pcdp::launch_pack_ll(src, dst, k / 8, seq, static_cast<hipStream_t>(stream)));
}

pc_status pc_consume_ll(const uint64_t* const* lines, int n, uint16_t* out, size_t k,
                        uint32_t seq, uint64_t* ready_bitmap, void* stream) {
    if (!valid_n(n) || !lines || seq == 0 || k > PC_MAX_ELEMS) return PC_EINVAL;
    if (k % 128) return PC_EALIGN;
    if (k == 0) return PC_OK;
    if (pc_status st = check_ptrs(lines, n)) return st;
    if (!out || !ready_bitmap) return PC_EINVAL;
    if (!aligned16(out) || !aligned16(ready_bitmap)) return PC_EALIGN;
    const size_t nlines = k / 2;
    const size_t line_bytes = nlines * sizeof(uint64_t);
    const size_t out_bytes = k * sizeof(uint16_t);
    const size_t bm_bytes = (nlines / 64) * sizeof(uint64_t);
    if (overlaps(out, out_bytes, ready_bitmap, bm_bytes)) return PC_EINVAL;
    for (int r = 0; r < n; ++r)
        if (overlaps(lines[r], line_bytes, out, out_bytes) ||
            overlaps(lines[r], line_bytes, ready_bitmap, bm_bytes))
            return PC_EINVAL;
    const void* src[PC_MAX_RANKS];
    for (int r = 0; r < n; ++r) src[r] = lines[r];
    return from_hip(pcdp::launch_consume_ll(src, n, out, nlines, seq, ready_bitmap,
                                            static_cast<hipStream_t>(stream)));
}

// Shared admission of the two twoshot entry points.  On PC_OK with k > 0 the
// pointers are copied to src/dst; *empty is set for the k == 0 no-op.
static pc_status check_twoshot(const uint16_t* const* inputs, int n, uint16_t* const* outs,
                               size_t k, const void** src, void** dst, bool* empty) {
    *empty = false;
    if (!valid_n(n) || !inputs || !outs || k > PC_MAX_ELEMS) return PC_EINVAL;
    if (k % (8 * (size_t)n)) return PC_EALIGN;
    if (k == 0) {
        *empty = true;
        return PC_OK;
    }
    if (pc_status st = check_ptrs(inputs, n)) return st;
    if (pc_status st = check_ptrs(outs, n)) return st;
    const size_t bytes = k * sizeof(uint16_t);
    for (int a = 0; a < n; ++a) {
        for (int b = a + 1; b < n; ++b)
            if (overlaps(outs[a], bytes, outs[b], bytes)) return PC_EINVAL;
        for (int r = 0; r < n; ++r)
            if (inputs[r] != outs[a] && overlaps(inputs[r], bytes, outs[a], bytes)) return PC_EINVAL;
    }
    for (int r = 0; r < n; ++r) {
        src[r] = inputs[r];
        dst[r] = outs[r];
    }
    return PC_OK;
}

pc_status pc_twoshot(const uint16_t* const* inputs, int n, uint16_t* const* outs, size_t k,
                     void* stream) {
    const void* src[PC_MAX_RANKS];
    void* dst[PC_MAX_RANKS];
    bool empty;
    if (pc_status st = check_twoshot(inputs, n, outs, k, src, dst, &empty)) return st;
    if (empty) return PC_OK;
    return from_hip(pcdp::launch_twoshot(src, n, dst, k / 8 / (size_t)n,
                                         static_cast<hipStream_t>(stream)));
}

pc_status pc_twoshot_fused(const uint16_t* const* inputs, int n, uint16_t* const* outs, size_t k,
                           void* stream) {
    const void* src[PC_MAX_RANKS];
    void* dst[PC_MAX_RANKS];
    bool empty;
    if (pc_status st = check_twoshot(inputs, n, outs, k, src, dst, &empty)) return st;
    if (empty) return PC_OK;
    return from_hip(pcdp::launch_twoshot_fused(src, n, dst, k / 8 / (size_t)n,
                                               static_cast<hipStream_t>(stream)));
}

static_assert(PC_LINKED_GROUPS == pcdp::kLinkGroups, "fixed grid of the linked twoshot");
static_assert(PC_LINKED_STATUS_WORD == pcdp::kLinkGroups, "status word follows the counters");
static_assert(PC_LINKED_POLL_LIMIT_WORD == pcdp::kLinkGroups + 1, "poll limit follows the status word");

size_t pc_twoshot_linked_workspace_bytes(int n, size_t k) {
    if (!valid_n(n) || k > PC_MAX_ELEMS || k % (8 * (size_t)n)) return 0;
    const size_t tiles = k ? pcdp::linked_tiles(n, k / 8 / (size_t)n) : 0;
    return sizeof(uint64_t) * (pcdp::kLinkGroups + pcdp::kLinkHeaderWords + tiles);
}

pc_status pc_twoshot_linked(const uint16_t* const* inputs, int n, uint16_t* const* outs, size_t k,
                            uint64_t* workspace, size_t workspace_bytes, void* stream) {
    const void* src[PC_MAX_RANKS];
    void* dst[PC_MAX_RANKS];
    bool empty;
    if (pc_status st = check_twoshot(inputs, n, outs, k, src, dst, &empty)) return st;
    if (empty) return PC_OK;
    if (!workspace) return PC_EINVAL;
    if (!aligned16(workspace)) return PC_EALIGN;
    const size_t need = pc_twoshot_linked_workspace_bytes(n, k);
    if (workspace_bytes < need) return PC_EINVAL;
    const size_t bytes = k * sizeof(uint16_t);
    for (int r = 0; r < n; ++r)
        if (overlaps(workspace, need, inputs[r], bytes) || overlaps(workspace, need, outs[r], bytes))
            return PC_EINVAL;
    const hipError_t e = pcdp::launch_twoshot_linked(src, n, dst, k / 8 / (size_t)n, workspace, nullptr,
                                                     static_cast<hipStream_t>(stream));
    return e == hipErrorCooperativeLaunchTooLarge ? PC_EUNSUPPORTED : from_hip(e);
}

static_assert(PC_LINKED_STATIC_SCRATCH_BYTES == pcdp::kStaticScratchBytes, "static scratch size");

pc_status pc_twoshot_linked_static(const uint16_t* const* inputs, int n, uint16_t* const* outs, size_t k,
                                   uint64_t* gave_up, void* stream) {
    const void* src[PC_MAX_RANKS];
    void* dst[PC_MAX_RANKS];
    bool empty;
    if (pc_status st = check_twoshot(inputs, n, outs, k, src, dst, &empty)) return st;
    if (empty) return PC_OK;
    if (pc_twoshot_linked_workspace_bytes(n, k) > PC_LINKED_STATIC_SCRATCH_BYTES) return PC_EINVAL;
    if (gave_up) {
        if (!aligned8(gave_up)) return PC_EALIGN;
        const size_t bytes = k * sizeof(uint16_t);
        for (int r = 0; r < n; ++r)
            if (overlaps(gave_up, 8, inputs[r], bytes) || overlaps(gave_up, 8, outs[r], bytes)) return PC_EINVAL;
    }
    void* ws = nullptr;
    if (from_hip(pcdp::static_workspace(&ws))) return PC_EHIP;
    const hipError_t e = pcdp::launch_twoshot_linked(src, n, dst, k / 8 / (size_t)n, ws, gave_up,
                                                     static_cast<hipStream_t>(stream));
    return e == hipErrorCooperativeLaunchTooLarge ? PC_EUNSUPPORTED : from_hip(e);
}

pc_status pc_allgather_copy(const uint8_t* const* shards, int n, uint16_t* out,
                            size_t shard_bytes, uint64_t seq, uint64_t* ready_bitmap,
                            void* stream) {
    if (!valid_n(n) || !shards || seq == 0 || shard_bytes > 2 * PC_MAX_ELEMS) return PC_EINVAL;
    if (shard_bytes % 8192) return PC_EALIGN;
    if (shard_bytes == 0) return PC_OK;
    if (pc_status st = check_ptrs(shards, n)) return st;
    if (!out || !ready_bitmap) return PC_EINVAL;
    if (!aligned16(out) || !aligned16(ready_bitmap)) return PC_EALIGN;
    const size_t blocks = shard_bytes / PC_BLOCK_PAYLOAD_BYTES;
    const size_t rec_bytes = blocks * PC_BLOCK_RECORD_BYTES;
    const size_t out_bytes = (size_t)n * shard_bytes;
    const size_t bm_bytes = (size_t)n * blocks / 64 * sizeof(uint64_t);
    if (overlaps(out, out_bytes, ready_bitmap, bm_bytes)) return PC_EINVAL;
    for (int r = 0; r < n; ++r)
        if (overlaps(shards[r], rec_bytes, out, out_bytes) ||
            overlaps(shards[r], rec_bytes, ready_bitmap, bm_bytes))
            return PC_EINVAL;
    const void* src[PC_MAX_RANKS];
    for (int r = 0; r < n; ++r) src[r] = shards[r];
    return from_hip(pcdp::launch_allgather(src, n, out, blocks / 64, seq, ready_bitmap,
                                           static_cast<hipStream_t>(stream)));
}

pc_status pc_reduce_validated(const uint16_t* const* inputs, const uint32_t* const* flags, int n,
                              uint16_t* out, size_t k, size_t elems_per_flag, uint32_t flag,
                              uint32_t max_attempts, uint32_t* attempts, void* stream) {
    if (!valid_n(n) || !inputs || !flags || k > PC_MAX_ELEMS) return PC_EINVAL;
    if (max_attempts < 1 || max_attempts > PC_MAX_ATTEMPTS) return PC_EINVAL;
    if (elems_per_flag == 0 || elems_per_flag % 2048 || elems_per_flag > 4 * 2048) return PC_EINVAL;
    if (k % elems_per_flag) return PC_EALIGN;
    if (k == 0) return PC_OK;
    if (pc_status st = check_ptrs(inputs, n)) return st;
    for (int r = 0; r < n; ++r)
        if (!flags[r]) return PC_EINVAL;
    for (int r = 0; r < n; ++r)
        if (!aligned4(flags[r])) return PC_EALIGN;
    if (!out || !attempts) return PC_EINVAL;
    if (!aligned16(out) || !aligned4(attempts)) return PC_EALIGN;
    const size_t bytes = k * sizeof(uint16_t);
    const size_t tiles = k / elems_per_flag;
    const size_t tbytes = tiles * sizeof(uint32_t);
    if (overlaps(out, bytes, attempts, tbytes)) return PC_EINVAL;
    for (int r = 0; r < n; ++r) {
        if (inputs[r] != out && overlaps(inputs[r], bytes, out, bytes)) return PC_EINVAL;
        if (overlaps(inputs[r], bytes, attempts, tbytes) || overlaps(flags[r], tbytes, attempts, tbytes) ||
            overlaps(flags[r], tbytes, out, bytes))
            return PC_EINVAL;
    }
    const void* src[PC_MAX_RANKS];
    const void* fl[PC_MAX_RANKS];
    for (int r = 0; r < n; ++r) {
        src[r] = inputs[r];
        fl[r] = flags[r];
    }
    return from_hip(pcdp::launch_reduce_validated(src, fl, n, out, k, elems_per_flag, flag,
                                                  max_attempts, attempts,
                                                  static_cast<hipStream_t>(stream)));
}

pc_status pc_publish_sentinel(const uint16_t* src, uint16_t* slot, size_t k, void* stream) {
    if (k > PC_MAX_ELEMS) return PC_EINVAL;
    if (k % 8) return PC_EALIGN;
    if (k == 0) return PC_OK;
    if (!src || !slot) return PC_EINVAL;
    if (!aligned16(src) || !aligned16(slot)) return PC_EALIGN;
    const size_t bytes = k * sizeof(uint16_t);
    if (src != slot && overlaps(src, bytes, slot, bytes)) return PC_EINVAL;
    return from_hip(pcdp::launch_publish_sentinel(src, slot, k / 8, static_cast<hipStream_t>(stream)));
}

pc_status pc_consume_sentinel(uint16_t* const* slots, int n, uint16_t* out, size_t k,
                              uint64_t* ready_bitmap, void* stream) {
    if (!valid_n(n) || !slots || k > PC_MAX_ELEMS) return PC_EINVAL;
    if (k % 512) return PC_EALIGN;
    if (k == 0) return PC_OK;
    if (pc_status st = check_ptrs(slots, n)) return st;
    if (!out || !ready_bitmap) return PC_EINVAL;
    if (!aligned16(out) || !aligned16(ready_bitmap)) return PC_EALIGN;
    const size_t bytes = k * sizeof(uint16_t);
    const size_t bm_bytes = (k / 512) * sizeof(uint64_t);
    if (overlaps(out, bytes, ready_bitmap, bm_bytes)) return PC_EINVAL;
    for (int a = 0; a < n; ++a) {
        if (overlaps(slots[a], bytes, out, bytes) || overlaps(slots[a], bytes, ready_bitmap, bm_bytes))
            return PC_EINVAL;
        for (int b = a + 1; b < n; ++b)
            if (overlaps(slots[a], bytes, slots[b], bytes)) return PC_EINVAL;
    }
    void* sp[PC_MAX_RANKS];
    for (int r = 0; r < n; ++r) sp[r] = slots[r];
    return from_hip(pcdp::launch_consume_sentinel(sp, n, out, k / 8, ready_bitmap,
                                                  static_cast<hipStream_t>(stream)));
}

const char* pc_strerror(pc_status status) {
    switch (status) {
        case PC_OK: return "success";
        case PC_EINVAL: return "invalid argument";
        case PC_EALIGN: return "misaligned pointer or size";
        case PC_EUNSUPPORTED: return "unsupported";
        case PC_EHIP: return "HIP launch failed";
        default: return "unknown status";
    }
}

int pc_abi_version(void) { return PC_ABI_VERSION; }

}  // extern "C"
