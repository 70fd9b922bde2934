/*
 * pc_oracle.c -- plain, slow, obviously correct CPU oracle for the datapath.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the library's product path may link,
 * load or call this file; only the tests, the smoke check and the benchmark's
 * CPU-baseline leg do.  It shares no source, header or table with the HIP
 * path: every definition below is written out again from the pages.
 *
 * Sources (page title, then the passage):
 *  - "Purlin: Separating Orchestration from the Datapath of Collectives",
 *    Section 3.3 (The Atom's Unified Pipeline), paragraph "Deterministic
 *    reduction within the pipeline", Equation (2): one accumulator per output
 *    element, contributions added rank by rank in ascending order, the sum
 *    beginning at zero;
 *    each input widened from its type to FP32, accumulated in FP32, and the sum
 *    converted back to the element type only after it is complete.
 *  - "flash-comm: Self-Synchronizing Collective Communication for LLM
 *    Decoding", Section 3.3 (fixed rank order 0..N-1, or one owner per output
 *    block), Section 3.1 (sequence-number readiness: a transfer unit is
 *    accepted only when its sequence number equals the current call's),
 *    Section 4.3 (one-hop fold after all sources are ready; sharded two-hop;
 *    all-gather as the distribution half).
 *  - "SiFAR: Synchronization-Free All-Reduce for Low-Latency LLM Inference",
 *    Section 3.1 and Figure 6 (twoshot = reduce-scatter of disjoint slices,
 *    then broadcast of every reduced slice to every rank).
 *
 * Readings where the pages are silent (each one is listed with its reason in
 * the design notes):
 *  - the accumulator starts at -0.0f, the exact additive identity of binary32
 *    under round-to-nearest-even, so a one-rank fold returns its input;
 *  - fp32 -> bf16 rounds to nearest, ties to even; every NaN becomes the
 *    canonical quiet NaN 0x7FC0 (which NaN payload survives an addition of two
 *    NaNs is not fixed by IEEE 754, so only a canonical pattern is unique);
 *  - subnormals are kept (no flush-to-zero, no denormals-are-zero);
 *  - an LL line is 8 bytes: bits 0..31 hold elements 2j (low half) and 2j+1
 *    (high half), bits 32..63 hold the sequence number;
 *  - a block record is 136 bytes: a u64 sequence header, then 128 payload
 *    bytes;
 *  - the ready bitmap is LSB-first u64 words: item i is bit (i & 63) of word
 *    (i >> 6);
 *  - output of a line or block that is not ready is left untouched;
 *  - the sentinel of sentinel readiness is the bf16 pattern 0xFFFF (a NaN),
 *    the readiness unit is a pack of 8 bf16 (16 bytes), and a published value
 *    equal to the sentinel is replaced by the canonical quiet NaN 0x7FC0.
 *
 * Floating point here is IEEE binary32 on x86-64 SSE2 (FLT_EVAL_METHOD 0),
 * built without -ffast-math and without contraction; orc_fpenv_ok() checks
 * at run time that MXCSR has FTZ and DAZ clear in every thread that folds.
 */
#include <float.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <xmmintrin.h>

#if !defined(FLT_EVAL_METHOD) || FLT_EVAL_METHOD != 0
#error "the oracle needs float arithmetic evaluated in binary32 (FLT_EVAL_METHOD == 0)"
#endif

#define ORC_MXCSR_FTZ (1u << 15)
#define ORC_MXCSR_DAZ (1u << 6)

static int mxcsr_ieee(void) {
    unsigned int csr = _mm_getcsr();
    return (csr & (ORC_MXCSR_FTZ | ORC_MXCSR_DAZ)) == 0;
}

/* 1 when this thread's float environment matches IEEE binary32 with
 * gradual underflow; 0 otherwise. */
int orc_fpenv_ok(void) { return mxcsr_ieee(); }

/* ---- element conversions (Purlin Section 3.3, Equation (2)) ------------- */

/* bf16 -> fp32: the bf16 bits are the upper half of the fp32 bits (exact). */
float orc_widen(uint16_t h) {
    uint32_t u = ((uint32_t)h) << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

/* fp32 -> bf16, round to nearest, ties to even; NaN -> 0x7FC0. */
uint16_t orc_narrow(float f) {
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    uint32_t mag = u & 0x7FFFFFFFu;
    if (mag > 0x7F800000u) return (uint16_t)0x7FC0u; /* any NaN */
    uint32_t keep = u >> 16;            /* truncated bf16 */
    uint32_t rest = u & 0xFFFFu;        /* discarded low half */
    /* Round up when the discarded half is above one half ulp, or exactly
     * one half and the kept value is odd.  Carrying into the exponent is the
     * correct result, and carrying out of the largest finite gives +-Inf. */
    if (rest > 0x8000u || (rest == 0x8000u && (keep & 1u))) keep += 1u;
    return (uint16_t)keep;
}

void orc_narrow_array(const float* in, uint16_t* out, size_t count) {
    for (size_t i = 0; i < count; ++i) out[i] = orc_narrow(in[i]);
}

void orc_widen_array(const uint16_t* in, float* out, size_t count) {
    for (size_t i = 0; i < count; ++i) out[i] = orc_widen(in[i]);
}

/* ---- the rank-ordered fold (Purlin Eq. (2); flash-comm Section 3.3) ------ */

/* Sum of contribution i over ranks order[0], order[1], ..., order[n-1],
 * in that order, in binary32. */
static float fold_element(const uint16_t* const* x, int n, const int32_t* order, size_t i) {
    float acc = -0.0f;
    for (int j = 0; j < n; ++j) {
        int r = order ? order[j] : j;
        acc = acc + orc_widen(x[r][i]);
    }
    return acc;
}

static int check_order(int n, const int32_t* order) {
    if (!order) return 1;
    int seen[64] = {0};
    if (n > 64) return 0;
    for (int j = 0; j < n; ++j) {
        if (order[j] < 0 || order[j] >= n || seen[order[j]]) return 0;
        seen[order[j]] = 1;
    }
    return 1;
}

typedef struct {
    const uint16_t* const* x;
    int n;
    const int32_t* order;
    uint16_t* out;
    size_t begin, end;
    int env_ok;
} reduce_job;

static void* reduce_range(void* arg) {
    reduce_job* job = (reduce_job*)arg;
    job->env_ok = mxcsr_ieee();
    for (size_t i = job->begin; i < job->end; ++i)
        job->out[i] = orc_narrow(fold_element(job->x, job->n, job->order, i));
    return NULL;
}

/* out[i] = narrow(fold over ranks of widen(inputs[r][i])), for i < k.
 * `threads` > 1 splits the element range only; every element's fold is the
 * same sequence of additions whatever the split.  Returns 0 on success,
 * -1 on bad arguments, -2 when the float environment is not IEEE. */
int orc_reduce(const uint16_t* const* inputs, int n, uint16_t* out, size_t k,
               const int32_t* order, int threads) {
    if (n < 1 || !inputs || (k && !out) || !check_order(n, order)) return -1;
    if (threads < 1) threads = 1;
    if (threads > 256) threads = 256;
    if ((size_t)threads > k) threads = k ? (int)k : 1;
    reduce_job jobs[256];
    pthread_t tids[256];
    size_t per = k / (size_t)threads, extra = k % (size_t)threads, at = 0;
    for (int t = 0; t < threads; ++t) {
        size_t len = per + ((size_t)t < extra ? 1 : 0);
        jobs[t] = (reduce_job){inputs, n, order, out, at, at + len, 0};
        at += len;
    }
    if (threads == 1) {
        reduce_range(&jobs[0]);
        return jobs[0].env_ok ? 0 : -2;
    }
    int started = 0;
    for (; started < threads; ++started)
        if (pthread_create(&tids[started], NULL, reduce_range, &jobs[started]) != 0) break;
    for (int t = started; t < threads; ++t) reduce_range(&jobs[t]);
    for (int t = 0; t < started; ++t) pthread_join(tids[t], NULL);
    for (int t = 0; t < threads; ++t)
        if (!jobs[t].env_ok) return -2;
    return 0;
}

/* ---- LL lines (flash-comm Sections 3.1 and 4.3; Purlin Section 3.2) ----- */

/* dst[j] holds elements 2j and 2j+1 in its low 32 bits and seq in its high
 * 32 bits.  k must be even. */
int orc_pack_ll(const uint16_t* src, uint64_t* dst, size_t k, uint32_t seq) {
    if (k % 2) return -1;
    for (size_t j = 0; j < k / 2; ++j) {
        uint64_t data = (uint64_t)src[2 * j] | ((uint64_t)src[2 * j + 1] << 16);
        dst[j] = data | ((uint64_t)seq << 32);
    }
    return 0;
}

/* For each line j: ready iff every rank's line j carries `seq`.  A ready
 * line's two elements are folded over ranks 0..n-1 and stored; a line that
 * is not ready leaves out[2j], out[2j+1] as they were.  Bit j of the bitmap
 * is set to `ready`; every bitmap word covering the k/2 lines is written.
 * k must be a multiple of 128 (whole bitmap words). */
int orc_consume_ll(const uint64_t* const* lines, int n, uint16_t* out, size_t k,
                   uint32_t seq, uint64_t* bitmap) {
    if (n < 1 || k % 128) return -1;
    if (!mxcsr_ieee()) return -2;
    size_t nlines = k / 2;
    for (size_t w = 0; w < nlines / 64; ++w) bitmap[w] = 0;
    for (size_t j = 0; j < nlines; ++j) {
        int ready = 1;
        for (int r = 0; r < n; ++r)
            if ((uint32_t)(lines[r][j] >> 32) != seq) ready = 0;
        if (!ready) continue;
        bitmap[j / 64] |= (uint64_t)1 << (j % 64);
        for (int h = 0; h < 2; ++h) {
            float acc = -0.0f;
            for (int r = 0; r < n; ++r) {
                uint16_t e = (uint16_t)((lines[r][j] >> (16 * h)) & 0xFFFFu);
                acc = acc + orc_widen(e);
            }
            out[2 * j + h] = orc_narrow(acc);
        }
    }
    return 0;
}

/* ---- twoshot (SiFAR Section 3.1, Figure 6; flash-comm Section 4.3) ------ */

/* Slice s = [s*k/n, (s+1)*k/n) is reduced once by its owner s, in rank order
 * 0..n-1, and that one result is copied into every rank's output. */
int orc_twoshot(const uint16_t* const* inputs, int n, uint16_t* const* outs, size_t k) {
    if (n < 1 || k % (size_t)n) return -1;
    size_t slice = k / (size_t)n;
    const uint16_t* part[64];
    if (n > 64) return -1;
    for (int s = 0; s < n; ++s) {
        for (int r = 0; r < n; ++r) part[r] = inputs[r] + (size_t)s * slice;
        uint16_t* owner = outs[s] + (size_t)s * slice;
        int rc = orc_reduce(part, n, owner, slice, NULL, 1);
        if (rc) return rc;
        for (int r = 0; r < n; ++r)
            if (r != s) memcpy(outs[r] + (size_t)s * slice, owner, slice * sizeof(uint16_t));
    }
    return 0;
}

/* ---- all-gather copy with block readiness (flash-comm Section 4.3) ------ */

/* shards[r] is an array of 136-byte records [u64 seq][128 payload bytes];
 * a shard carries shard_bytes of payload, i.e. B = shard_bytes/128 records.
 * Record b of shard r is accepted iff its header equals seq; its payload
 * then goes to out + (r*B + b)*128 and bit r*B + b is set.  A rejected
 * block leaves its output bytes untouched and its bit clear.
 * shard_bytes must be a multiple of 8192 (whole bitmap words per shard). */
int orc_allgather_copy(const uint8_t* const* shards, int n, uint8_t* out, size_t shard_bytes,
                       uint64_t seq, uint64_t* bitmap) {
    if (n < 1 || shard_bytes % 8192) return -1;
    size_t blocks = shard_bytes / 128;
    for (size_t w = 0; w < (size_t)n * blocks / 64; ++w) bitmap[w] = 0;
    for (int r = 0; r < n; ++r) {
        for (size_t b = 0; b < blocks; ++b) {
            const uint8_t* rec = shards[r] + 136 * b;
            uint64_t header;
            memcpy(&header, rec, sizeof header);
            if (header != seq) continue;
            size_t item = (size_t)r * blocks + b;
            memcpy(out + item * 128, rec + 8, 128);
            bitmap[item / 64] |= (uint64_t)1 << (item % 64);
        }
    }
    return 0;
}

/* ---- sentinel readiness (flash-comm Section 3.1, Section 4.3) ----------- */

#define ORC_SENTINEL 0xFFFFu
#define ORC_CANON_NAN 0x7FC0u

/* Producer: dst[i] = src[i], except that a value equal to the sentinel is
 * published as the canonical quiet NaN, so real data never looks unarrived. */
int orc_publish_sentinel(const uint16_t* src, uint16_t* dst, size_t k) {
    for (size_t i = 0; i < k; ++i)
        dst[i] = src[i] == ORC_SENTINEL ? (uint16_t)ORC_CANON_NAN : src[i];
    return 0;
}

/* Consumer: pack p (elements 8p..8p+7) is ready iff no element of pack p in
 * any rank's slot is the sentinel.  A ready pack is folded over ranks
 * 0..n-1 into out and its slots are re-armed (every element set back to the
 * sentinel); a pack that is not ready leaves out and the slots untouched.
 * Bit p of the bitmap (LSB-first u64 words) is set to `ready`; every word is
 * written.  k must be a multiple of 512 (whole bitmap words). */
int orc_consume_sentinel(uint16_t* const* slots, int n, uint16_t* out, size_t k, uint64_t* bitmap) {
    if (n < 1 || k % 512) return -1;
    if (!mxcsr_ieee()) return -2;
    size_t packs = k / 8;
    for (size_t w = 0; w < packs / 64; ++w) bitmap[w] = 0;
    for (size_t p = 0; p < packs; ++p) {
        int ready = 1;
        for (int r = 0; r < n; ++r)
            for (size_t e = 8 * p; e < 8 * p + 8; ++e)
                if (slots[r][e] == ORC_SENTINEL) ready = 0;
        if (!ready) continue;
        bitmap[p / 64] |= (uint64_t)1 << (p % 64);
        for (size_t e = 8 * p; e < 8 * p + 8; ++e) {
            float acc = -0.0f;
            for (int r = 0; r < n; ++r) acc = acc + orc_widen(slots[r][e]);
            out[e] = orc_narrow(acc);
        }
        for (int r = 0; r < n; ++r)
            for (size_t e = 8 * p; e < 8 * p + 8; ++e) slots[r][e] = (uint16_t)ORC_SENTINEL;
    }
    return 0;
}

/* ---- speculative reduce with a folded validation flag -------------------- */
/* "SiFAR: Synchronization-Free All-Reduce for Low-Latency LLM Inference",
 * Section 4 (the paragraphs on eliminating flag exchange, on the verification
 * logic with Figure 14, and on speculative reduction): every rank writes the call's flag into
 * its validation buffer; the validation buffers are reduced (an integer sum
 * over ranks) next to the payload, and the result is accepted iff the folded
 * flag equals n * flag.  Tile b covers elements [b*t, (b+1)*t) with t =
 * elems_per_flag and is validated by flag word b of every rank.  With the
 * inputs fixed, the first attempt decides: ok[b] = 1 and the tile is folded
 * into out when the check passes, else ok[b] = 0 and out is untouched.  The
 * sum and the product wrap modulo 2^32. */
int orc_reduce_validated(const uint16_t* const* inputs, const uint32_t* const* flags, int n,
                         uint16_t* out, size_t k, size_t elems_per_flag, uint32_t flag,
                         uint32_t* ok) {
    if (n < 1 || elems_per_flag == 0 || k % elems_per_flag) return -1;
    if (!mxcsr_ieee()) return -2;
    size_t tiles = k / elems_per_flag;
    for (size_t b = 0; b < tiles; ++b) {
        uint32_t folded = 0;
        for (int r = 0; r < n; ++r) folded += flags[r][b];
        ok[b] = folded == (uint32_t)n * flag;
        if (!ok[b]) continue;
        for (size_t i = b * elems_per_flag; i < (b + 1) * elems_per_flag; ++i)
            out[i] = orc_narrow(fold_element(inputs, n, NULL, i));
    }
    return 0;
}
