/*
 * pc.h -- C ABI of the MI355X collective datapath library (libpcdp.so).
 *
 * The library implements one GPU's share of the all-reduce / all-gather
 * datapath: the Atom's byte-range copy, an N-way elementwise reduction of N rank-staged bf16 buffers in a
 * fixed rank order, sequence-number ("LL") line packing and consume-side
 * readiness validation, sentinel readiness, a speculative reduce validated by
 * folded flags, the twoshot split (slice reduce, then copy-out; also in one
 * launch, with or without flags between the phases), and an all-gather copy
 * whose blocks carry sequence-number headers.  The N peers' staged buffers
 * are N distinct device regions.
 *
 * Conventions shared by every call:
 *  - All functions are extern "C", return pc_status and never throw.
 *  - bf16 values are passed as their 16-bit patterns (uint16_t).
 *  - Pointer arrays (`inputs`, `lines`, `outs`, `shards`) and `order` are HOST
 *    arrays, read only during the call.  The pointers inside them and every
 *    other data pointer are DEVICE pointers on the current HIP device, each
 *    16-byte aligned.  The caller allocates and frees all memory; the library
 *    allocates nothing and keeps no state between calls, apart from
 *    pc_twoshot_linked_static's static workspace (pc_twoshot_linked keeps its
 *    call counters in a workspace the caller owns).
 *  - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *    Work is enqueued asynchronously; outputs are valid once the stream has
 *    reached the call.  No call synchronizes the device.
 *  - Arguments are validated before anything is enqueued; on any error
 *    nothing is launched and outputs are untouched.  A size of zero is a
 *    legal no-op (PC_OK); its device pointers are then not examined.
 *  - Calls that overlap in time on the same output buffers race; calls on
 *    different streams touching disjoint buffers are independent.
 *  - Performance, not correctness: large calls reach full HBM bandwidth when
 *    every device buffer starts on a 128-byte boundary (a cache line).  A
 *    buffer that is only 16-byte aligned makes each wave access touch one
 *    more line, written in parts by different workgroups; at 8 ranks x
 *    64 MiB that made the twoshot calls about a quarter slower.
 *
 * Arithmetic (every reduction here):
 *  Each output element is y = narrow(((-0.0f + w(x_{o0})) + w(x_{o1})) + ... +
 *  w(x_{o(n-1)})) where w() widens bf16 to fp32 exactly, each addition is an
 *  IEEE binary32 addition rounded to nearest-even with subnormals kept, and
 *  narrow() rounds fp32 to bf16 to nearest-even, overflow giving +-Inf and any
 *  NaN giving the canonical quiet NaN 0x7FC0.  o0..o(n-1) is ascending rank
 *  order unless `order` says otherwise.  The result is bit-exact: one correct
 *  bit pattern per element.
 *  ("Purlin: Separating Orchestration from the Datapath of Collectives",
 *  Section 3.3, Equation (2); "flash-comm: Self-Synchronizing Collective
 *  Communication for LLM Decoding", Section 3.3.)
 */
#ifndef PC_H
#define PC_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#if defined(__GNUC__)
#define PC_API __attribute__((visibility("default")))
#else
#define PC_API
#endif

typedef int pc_status;

enum {
    PC_OK = 0,
    PC_EINVAL = -1,       /* bad argument: n out of range, NULL pointer,     */
                          /* order not a permutation, seq == 0, overlapping  */
                          /* buffers, size above the maximum                 */
    PC_EALIGN = -2,       /* a device pointer or a size is misaligned        */
    PC_EUNSUPPORTED = -3, /* the device cannot run the call (pc_twoshot_linked: */
                          /* its fixed grid does not fit on the GPU at once)  */
    PC_EHIP = -4          /* the HIP runtime refused the launch              */
};

#define PC_ABI_VERSION 8
#define PC_MAX_RANKS 8
#define PC_LL_LINE_BYTES 8          /* u32 data (element 2j low, 2j+1 high) | u32 seq   */
#define PC_BLOCK_PAYLOAD_BYTES 128
#define PC_BLOCK_RECORD_BYTES 136   /* u64 seq header, then 128 payload bytes           */
#define PC_MAX_ELEMS ((size_t)1 << 34) /* largest k accepted per rank (32 GiB of bf16) */

/*
 * pc_reduce -- N-way rank-ordered reduction (oneshot's local reduce).
 * Source: Purlin, Section 3.3 (Listing 3's reduce over n equally sized typed
 * sources into one destination; Equation (2) for the arithmetic); SiFAR:
 * Synchronization-Free All-Reduce for Low-Latency LLM Inference, Section 3.1
 * (oneshot: every GPU reduces all N buffers elementwise).
 *   inputs : host array of n device pointers, each to k bf16 values.  Inputs
 *            may alias each other.
 *   n      : 1..PC_MAX_RANKS.
 *   out    : device pointer to k bf16 values.  It may be exactly one of the
 *            inputs (in place); any other overlap with an input is PC_EINVAL.
 *   k      : elements per rank; multiple of 8, at most PC_MAX_ELEMS.
 *   order  : host array, a permutation of 0..n-1 giving the fold order, or
 *            NULL for 0,1,..,n-1.
 * Errors: PC_EINVAL, PC_EALIGN (pointer not 16-byte aligned, k % 8 != 0),
 *         PC_EHIP.
 */
PC_API pc_status pc_reduce(const uint16_t* const* inputs, int n, uint16_t* out, size_t k,
                    const int32_t* order, void* stream);

/*
 * pc_copy -- the Atom's copy: `bytes` bytes from src to dst, unchanged.
 * Source: Purlin, Section 3.3 (the Atom's two primitives are a copy of one
 * contiguous range and a typed reduce; the copy's per-element step is a
 * store).  The copy-outs of pc_twoshot and pc_allgather_copy are this
 * primitive with a fan-out or a readiness test added.
 *   dst, src : device, 16-byte aligned; disjoint, or exactly equal (then
 *              nothing is launched).
 *   bytes    : multiple of 16, at most 2*PC_MAX_ELEMS.
 * Every bit pattern is copied as is (NaN payloads included).
 * Errors: PC_EINVAL (NULL pointer, partial overlap, bytes above the maximum),
 * PC_EALIGN, PC_EHIP.
 */
PC_API pc_status pc_copy(void* dst, const void* src, size_t bytes, void* stream);

/*
 * pc_pack_ll -- stage k bf16 values as k/2 sequence-stamped 8-byte lines.
 * Source: flash-comm, Section 3.1 (sequence-number readiness: data and the
 * call's sequence number share one transfer unit) and Section 4.3 (16-byte
 * packets of 8 payload bytes and two copies of the sequence number, i.e. two
 * such lines); Purlin, Section 3.2 (latency path: payload packed with a flag).
 *   src  : device, k bf16 values.
 *   dst  : device, k/2 uint64 lines; line j = (src[2j] | src[2j+1] << 16)
 *          | (uint64)seq << 32 (little-endian: data bytes 0..3, seq 4..7).
 *          Must not overlap src.
 *   k    : multiple of 8, at most PC_MAX_ELEMS.
 *   seq  : the current call's sequence number, nonzero (zero-filled memory
 *          must never read as ready).
 * Errors: PC_EINVAL, PC_EALIGN, PC_EHIP.
 */
PC_API pc_status pc_pack_ll(const uint16_t* src, uint64_t* dst, size_t k, uint32_t seq, void* stream);

/*
 * pc_consume_ll -- validate N ranks' LL lines and fold the ready ones.
 * Source: flash-comm, Section 4.3 (one-hop: poll the source slots, reduce only
 * once every source has arrived, fold by source rank in rank order),
 * Section 3.1 (accept a unit only when its sequence number matches the
 * current call), Section 3.3 (rank order 0..N-1).
 *   lines  : host array of n device pointers, each to k/2 uint64 lines.
 *   out    : device, k bf16.  For every line j that is ready on all n ranks,
 *            out[2j], out[2j+1] = the rank-ordered fold of the lines' two
 *            halves.  Output of a line that is not ready is left untouched.
 *   k      : multiple of 128 (whole bitmap words), at most PC_MAX_ELEMS.
 *   seq    : nonzero; a line is current iff its high 32 bits equal seq.
 *   ready_bitmap : device, k/128 uint64 words; bit (j & 63) of word (j >> 6)
 *            is 1 iff line j was ready.  Every word is written.
 *   out, ready_bitmap and the lines must not overlap one another.
 * Errors: PC_EINVAL, PC_EALIGN (pointer alignment, k % 128 != 0), PC_EHIP.
 */
PC_API pc_status pc_consume_ll(const uint64_t* const* lines, int n, uint16_t* out, size_t k,
                        uint32_t seq, uint64_t* ready_bitmap, void* stream);

/*
 * pc_twoshot -- reduce-scatter by slice owner, then copy-out to every rank.
 * Source: SiFAR, Section 3.1 and Figure 6 (twoshot: each GPU reduces one
 * portion, then broadcasts it to all peers); flash-comm, Section 3.3 (each
 * output block has one owner that reduces it once and distributes it) and
 * Section 4.3 (sharded two-hop); Purlin, Section 3.1 (AllReduce as a
 * ReduceScatter followed by an AllGather, Figure 4).
 *   inputs : host array of n device pointers, k bf16 each.
 *   outs   : host array of n device pointers, k bf16 each, pairwise
 *            disjoint.  Slice s = [s*k/n, (s+1)*k/n) is folded in rank order
 *            0..n-1 into outs[s] (its owner), then copied from outs[s] into
 *            every other outs[r].  Every outs[r] equals pc_reduce's result
 *            bit for bit.  outs[r] may be exactly an input buffer (in place);
 *            other overlaps with inputs are PC_EINVAL.
 *   k      : multiple of 8*n, at most PC_MAX_ELEMS.
 * Two kernels are enqueued on `stream`, the copy-out after the slice reduce.
 * Errors: PC_EINVAL, PC_EALIGN, PC_EHIP.
 */
PC_API pc_status pc_twoshot(const uint16_t* const* inputs, int n, uint16_t* const* outs, size_t k,
                     void* stream);

/*
 * pc_twoshot_fused -- twoshot in one launch: each owner block is folded once
 * and distributed at once.
 * Source: flash-comm, Section 4.3 (sharded two-hop: the two phases are linked
 * per block, so an owner hands out a finished block while others are still in
 * progress) and Section 3.3 (a block is computed once by its owner and
 * distributed); Purlin, Section 3.1 (AllReduce composed from ReduceScatter
 * and AllGather) and Listing 1 (compose: the second step consumes the
 * first's intermediate in place, in one kernel).
 * Same arguments, layouts, aliasing rules and errors as pc_twoshot, and the
 * same result bit for bit: slice s = [s*k/n, (s+1)*k/n) is folded in rank
 * order 0..n-1 exactly once, and the workgroup that folds a block writes it
 * to every outs[r].  One kernel is enqueued.  Below a working set (inputs
 * plus outputs) of 640 MiB, or with fewer than five ranks, each folded
 * block goes to every output at once; from there the workgroup first writes
 * all of its blocks to their owners' outputs and then reads them back from
 * there to write the other outputs.
 */
PC_API pc_status pc_twoshot_fused(const uint16_t* const* inputs, int n, uint16_t* const* outs,
                                  size_t k, void* stream);

/*
 * pc_twoshot_linked -- twoshot in one launch, its two phases linked tile by
 * tile through epoch-stamped readiness flags, the epoch kept on the device.
 * Source: flash-comm, Section 4.3 (sharded two-hop: readiness checks join the
 * slice reduction and the result distribution per block) and Section 4.2
 * (state derived from a call counter kept on the device, so a captured graph
 * can be replayed; one fixed grid per family; every rank issues the same
 * call sequence); Purlin, Section 4.2 (a persistent per-block epoch advanced
 * after each call is the value that signals readiness).
 * Same inputs, outs, k, aliasing rules and result as pc_twoshot, bit for bit.
 * The tiles of slice s are folded into outs[s] by one set of workgroups; each
 * tile's flag is then set to the call's epoch, and other workgroups wait for
 * that flag and copy the tile from outs[s] into every other outs[r].
 *   workspace : device, 16-byte aligned, at least
 *               pc_twoshot_linked_workspace_bytes(n, k) bytes, owned by the
 *               caller.  It must be zero-filled before its first use and then
 *               left to the library: it carries one 64-bit call counter per
 *               workgroup of a fixed grid of PC_LINKED_GROUPS workgroups, so
 *               successive calls (and graph replays) need no host-side epoch
 *               and no clearing.  Epochs are 64-bit and never wrap.  A
 *               workspace serves any n and k it is large enough for.  Two
 *               calls that may run at the same time (other streams) need
 *               separate workspaces; it must not overlap any input or output.
 *   workspace[PC_LINKED_STATUS_WORD] (uint64) : the number of tiles, summed
 *               over all calls, whose wait for a flag was abandoned after a
 *               bounded number of polls; the copies of those tiles into the
 *               non-owner outputs are then skipped (those bytes of outs[r],
 *               r != s, are left as they were), while every owner output
 *               outs[s] is complete.  It stays 0 while the grid is resident,
 *               which is checked before launch.
 *   workspace[PC_LINKED_POLL_LIMIT_WORD] (uint64) : polls per wait before it
 *               is abandoned; 0 (the zero-filled default) or anything above
 *               2^20 means 2^20.  The caller may set it between calls (a
 *               diagnostic knob: tests use it to reach the give-up path fast).
 * Errors: PC_EINVAL (also: NULL workspace, workspace_bytes too small,
 * workspace overlapping a buffer), PC_EALIGN, PC_EUNSUPPORTED (the device
 * cannot hold PC_LINKED_GROUPS of these workgroups at once), PC_EHIP.
 */
#define PC_LINKED_GROUPS 256
#define PC_LINKED_STATUS_WORD 256     /* index in uint64 words */
#define PC_LINKED_POLL_LIMIT_WORD 257 /* index in uint64 words */

/* Workspace bytes pc_twoshot_linked needs for (n, k); 0 if n or k would be
 * rejected by it.  For k == 0 it is the fixed part of the workspace. */
PC_API size_t pc_twoshot_linked_workspace_bytes(int n, size_t k);

PC_API pc_status pc_twoshot_linked(const uint16_t* const* inputs, int n, uint16_t* const* outs,
                                   size_t k, uint64_t* workspace, size_t workspace_bytes,
                                   void* stream);

/*
 * pc_twoshot_linked_static -- pc_twoshot_linked for callers that cannot
 * allocate (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc): the same computation, result and status counting,
 * with the workspace held by the library in static device memory instead of
 * passed in.  The call allocates nothing (no hipMalloc, hipFree or
 * allocating library routine); the caller passes only inputs and outputs.
 *   inputs, n, outs, k : as pc_twoshot_linked.  The workspace that
 *            pc_twoshot_linked_workspace_bytes(n, k) would give must fit in
 *            PC_LINKED_STATIC_SCRATCH_BYTES (1 MiB: about 2 GiB per rank at 8
 *            ranks); larger calls are rejected with PC_EINVAL and nothing
 *            is launched.
 *   gave_up : device, 8-byte aligned, or NULL.  The number of tiles whose
 *            wait was abandoned is added to *gave_up (NULL: to a word of the
 *            static workspace that the caller cannot read).  It must not
 *            overlap an input or output.
 * The static workspace is zero when the library is loaded, lives until the
 * process ends (one per GPU the library runs on) and keeps the call
 * counters between calls, as a caller-owned workspace does.  Every call on
 * one GPU shares it: calls that may overlap in time on one GPU (other
 * streams) race and must not be issued.
 * Errors: PC_EINVAL (also: the size limit above, gave_up overlapping a
 * buffer), PC_EALIGN, PC_EUNSUPPORTED, PC_EHIP.
 */
#define PC_LINKED_STATIC_SCRATCH_BYTES ((size_t)1 << 20)
PC_API pc_status pc_twoshot_linked_static(const uint16_t* const* inputs, int n, uint16_t* const* outs,
                                          size_t k, uint64_t* gave_up, void* stream);

/*
 * pc_allgather_copy -- gather N shards of sequence-stamped blocks.
 * Source: flash-comm, Section 4.3 (all-gather: every source publishes one
 * shard, receivers wait on the same readiness layer and place each shard in
 * the output) and Appendix A, Table 8 discussion (128-byte writes arrive
 * whole); Purlin, Section 3.1 (AllGather output is rank-ordered).
 *   shards : host array of n device pointers.  Shard r holds B =
 *            shard_bytes/128 records of 136 bytes: a uint64 sequence header,
 *            then 128 payload bytes.
 *   out    : device, n*shard_bytes bytes (n*shard_bytes/2 bf16).  Record b
 *            of shard r whose header equals seq is copied to bytes
 *            [(r*B + b)*128, +128); a record that does not match leaves those
 *            bytes untouched.
 *   shard_bytes : payload bytes per shard; multiple of 8192 (64 blocks, one
 *            bitmap word), at most 2*PC_MAX_ELEMS.
 *   seq    : nonzero; compared with the whole 64-bit header.
 *   ready_bitmap : device, n*B/64 uint64 words; bit i (LSB-first) is 1 iff
 *            block i = r*B + b was copied.  Every word is written.
 *   out, ready_bitmap and the shards must not overlap one another.
 * Errors: PC_EINVAL, PC_EALIGN, PC_EHIP.
 */
PC_API pc_status pc_allgather_copy(const uint8_t* const* shards, int n, uint16_t* out,
                            size_t shard_bytes, uint64_t seq, uint64_t* ready_bitmap,
                            void* stream);

/*
 * pc_reduce_validated -- speculative reduce checked by a folded flag.
 * Source: SiFAR, Section 4 (paragraphs on eliminating flag exchange, on the
 * verification logic with Figure 14, and on speculative reduction): each
 * rank writes the call's flag into its validation buffer before the
 * reduction; the consumer reduces the flags (integer sum) next to the
 * payload and accepts iff the sum equals n * flag, rerunning otherwise.
 *   inputs  : host array of n device pointers, k bf16 each (may alias).
 *   flags   : host array of n device pointers, k/elems_per_flag uint32 each,
 *             4-byte aligned; word b of rank r validates tile b.
 *   out     : device, k bf16.  Tile b = elements [b*t, (b+1)*t), t =
 *             elems_per_flag.  A tile whose folded flag (sum mod 2^32 over
 *             ranks) equals n*flag (mod 2^32) is folded in rank order 0..n-1
 *             into out; a tile that never validates leaves out untouched.
 *             out may be exactly one input; other overlaps are PC_EINVAL.
 *   elems_per_flag : 2048, 4096, 6144 or 8192; k must be a multiple of it.
 *   flag    : the current call's flag (callers advance it every call and
 *             alternate two validation buffers, as the pages do).
 *   max_attempts : 1..PC_MAX_ATTEMPTS.  A tile that fails the check is
 *             re-read (flags and payload, past the caches) up to this many
 *             times in total; the bound makes every call finish.
 *   attempts: device, k/elems_per_flag uint32: the attempt that validated
 *             tile b (1-based), or 0.  Every word is written.
 * Flags and payload are read in the same attempt without ordering; as on
 * the pages, the check is sound when ranks progress monotonically.
 * Errors: PC_EINVAL, PC_EALIGN, PC_EHIP.
 */
#define PC_MAX_ATTEMPTS 65536u
PC_API pc_status pc_reduce_validated(const uint16_t* const* inputs, const uint32_t* const* flags,
                                     int n, uint16_t* out, size_t k, size_t elems_per_flag,
                                     uint32_t flag, uint32_t max_attempts, uint32_t* attempts,
                                     void* stream);

/*
 * pc_publish_sentinel -- producer side of sentinel readiness.
 * Source: flash-comm, Section 3.1 (sentinel readiness: storage is prefilled
 * with a reserved pattern that a producer overwrites; a real value equal to
 * the pattern is published as a canonical quiet NaN so it never looks
 * unarrived).
 *   src  : device, k bf16 values.
 *   slot : device, k bf16; receives src with every 0xFFFF (PC_SENTINEL)
 *          replaced by 0x7FC0.  May be exactly src (in place); any other
 *          overlap is PC_EINVAL.  Written in 16-byte packs, one store each.
 *   k    : multiple of 8, at most PC_MAX_ELEMS.
 * Errors: PC_EINVAL, PC_EALIGN, PC_EHIP.
 */
#define PC_SENTINEL 0xFFFFu
#define PC_SENTINEL_PACK_ELEMS 8
PC_API pc_status pc_publish_sentinel(const uint16_t* src, uint16_t* slot, size_t k, void* stream);

/*
 * pc_consume_sentinel -- consumer side: validate, fold and re-arm.
 * Source: flash-comm, Section 3.1 (a pack that no longer holds the sentinel
 * has arrived; the consumer restores the sentinel after capturing it) and
 * Section 4.3 (one-hop: slots by source rank, fold only once every source has
 * arrived, folded in rank order); Purlin, Section 3.3, Equation (2) (the fold).
 *   slots : host array of n device pointers, k bf16 each, pairwise disjoint;
 *           the receive storage of the n sources.  READ AND WRITTEN: every
 *           pack that is consumed is re-armed (set back to 0xFFFF).
 *   out   : device, k bf16.  Pack p (elements 8p..8p+7) is ready iff no
 *           element of pack p holds 0xFFFF in any slot; then out[8p..8p+7] =
 *           the rank-ordered fold, else out and the slots are left untouched.
 *           No result element is ever 0xFFFF (NaN results are 0x7FC0).
 *   k     : multiple of 512 (whole bitmap words), at most PC_MAX_ELEMS.
 *   ready_bitmap : device, k/512 uint64 words; bit (p & 63) of word (p >> 6)
 *           is 1 iff pack p was ready.  Every word is written.
 *   out, ready_bitmap and the slots must not overlap one another.
 * Errors: PC_EINVAL, PC_EALIGN (pointer alignment, k % 512 != 0), PC_EHIP.
 */
PC_API pc_status pc_consume_sentinel(uint16_t* const* slots, int n, uint16_t* out, size_t k,
                                     uint64_t* ready_bitmap, void* stream);

/* Static text for a status code (never NULL). */
PC_API const char* pc_strerror(pc_status status);

/* PC_ABI_VERSION of the loaded library. */
PC_API int pc_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* PC_H */
