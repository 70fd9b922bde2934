/*
 * pc_abi_check.c -- drives libpcdp.so through include/pc.h from plain C, with
 * no Python and no torch in the process: device memory comes from the HIP
 * runtime API, streams are the null stream.
 *
 * Expected values are closed forms, not outputs of the library:
 *  - a copy returns its source bytes (Purlin, Section 3.3);
 *  - a fold of exactly representable values (rank r holds (r+1)/8) has an
 *    exact sum (Purlin, Section 3.3, Equation (2));
 *  - the cancellation triple (2^25, 1, -2^25) gives +0 in order (0,1,2) and
 *    1.0 in order (0,2,1), because 2^25 + 1 rounds back to 2^25 in binary32;
 *  - LL pack then consume at one rank returns every bf16 pattern unchanged,
 *    NaNs as the canonical 0x7FC0, with every ready bit set; a consume with
 *    another sequence number accepts nothing and writes nothing (flash-comm,
 *    Sections 3.1 and 4.3);
 *  - every twoshot form leaves the exact sum in every output;
 *  - an all-gather of all-current records is the concatenation of their
 *    payloads (flash-comm, Section 4.3);
 *  - malformed calls return their status codes and launch nothing.
 *
 * Exit status: 0 = every check passed, 1 = a check failed, 77 = no GPU.
 */
#include "pc.h"

#include <hip/hip_runtime_api.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#define HIP_OK(x)                                                                   \
    do {                                                                            \
        hipError_t e_ = (x);                                                        \
        if (e_ != hipSuccess) {                                                     \
            fprintf(stderr, "%s:%d: %s\n", __FILE__, __LINE__, hipGetErrorString(e_)); \
            exit(1);                                                                \
        }                                                                           \
    } while (0)

#define EXPECT(cond, what)                                                          \
    do {                                                                            \
        if (!(cond)) {                                                              \
            fprintf(stderr, "FAILED: %s (%s:%d)\n", what, __FILE__, __LINE__);      \
            exit(1);                                                                \
        }                                                                           \
    } while (0)

static void* dev_alloc(size_t bytes) {
    void* p = NULL;
    HIP_OK(hipMalloc(&p, bytes));
    return p;
}

static void* host_alloc(size_t bytes) {
    void* p = malloc(bytes ? bytes : 1);
    EXPECT(p != NULL, "host allocation");
    return p;
}

static void fill16(uint16_t* h, size_t n, uint16_t v) {
    for (size_t i = 0; i < n; ++i) h[i] = v;
}

static int all16(const uint16_t* h, size_t n, uint16_t v) {
    for (size_t i = 0; i < n; ++i)
        if (h[i] != v) return 0;
    return 1;
}

/* bf16 patterns of (r+1)/8 for r = 0..7: 0.125, 0.25, ..., 1.0 */
static const uint16_t kEighths[8] = {0x3E00, 0x3E80, 0x3EC0, 0x3F00, 0x3F20, 0x3F40, 0x3F60, 0x3F80};

/* Rank r holds (r+1)/8 everywhere: the sum over n ranks is n(n+1)/16, exact. */
static void check_reduce_exact_sums(void) {
    /* A multiple of 8*4 (twoshot at n = 4): slices of 256*3 + 5 chunks, so
     * whole tiles and a ragged tail in every slice. */
    const size_t k = 8 * 4 * (256 * 3 + 5);
    uint16_t* h = host_alloc(k * 2);
    const uint16_t* in[PC_MAX_RANKS];
    uint16_t* d_in[PC_MAX_RANKS];
    for (int r = 0; r < 8; ++r) {
        d_in[r] = dev_alloc(k * 2);
        fill16(h, k, kEighths[r]);
        HIP_OK(hipMemcpy(d_in[r], h, k * 2, hipMemcpyHostToDevice));
        in[r] = d_in[r];
    }
    uint16_t* d_out = dev_alloc(k * 2);
    /* n = 8: 4.5 (0x4090); n = 4: 1.25 (0x3FA0); n = 1: 0.125 */
    const int ns[3] = {8, 4, 1};
    const uint16_t want[3] = {0x4090, 0x3FA0, 0x3E00};
    for (int i = 0; i < 3; ++i) {
        EXPECT(pc_reduce(in, ns[i], d_out, k, NULL, NULL) == PC_OK, "pc_reduce status");
        HIP_OK(hipDeviceSynchronize());
        HIP_OK(hipMemcpy(h, d_out, k * 2, hipMemcpyDeviceToHost));
        EXPECT(all16(h, k, want[i]), "pc_reduce exact sum of eighths");
    }
    const int32_t reversed[8] = {7, 6, 5, 4, 3, 2, 1, 0};
    EXPECT(pc_reduce(in, 8, d_out, k, reversed, NULL) == PC_OK, "pc_reduce with order");
    HIP_OK(hipDeviceSynchronize());
    HIP_OK(hipMemcpy(h, d_out, k * 2, hipMemcpyDeviceToHost));
    EXPECT(all16(h, k, 0x4090), "pc_reduce reversed order, exact sum");

    /* Every twoshot form: the exact sum in every output, n = 4. */
    uint16_t* outs[PC_MAX_RANKS];
    for (int r = 0; r < 4; ++r) outs[r] = dev_alloc(k * 2);
    const size_t ws_bytes = pc_twoshot_linked_workspace_bytes(4, k);
    EXPECT(ws_bytes > 0, "linked workspace size");
    uint64_t* ws = dev_alloc(ws_bytes);
    HIP_OK(hipMemset(ws, 0, ws_bytes));
    for (int form = 0; form < 3; ++form) {
        for (int r = 0; r < 4; ++r) HIP_OK(hipMemset(outs[r], 0xFF, k * 2));
        pc_status st = form == 0   ? pc_twoshot(in, 4, outs, k, NULL)
                       : form == 1 ? pc_twoshot_fused(in, 4, outs, k, NULL)
                                   : pc_twoshot_linked(in, 4, outs, k, ws, ws_bytes, NULL);
        EXPECT(st == PC_OK, "twoshot status");
        HIP_OK(hipDeviceSynchronize());
        for (int r = 0; r < 4; ++r) {
            HIP_OK(hipMemcpy(h, outs[r], k * 2, hipMemcpyDeviceToHost));
            EXPECT(all16(h, k, 0x3FA0), "twoshot exact sum in every output");
        }
    }
    uint64_t status = 1;
    HIP_OK(hipMemcpy(&status, ws + PC_LINKED_STATUS_WORD, 8, hipMemcpyDeviceToHost));
    EXPECT(status == 0, "linked twoshot abandoned no wait");

    for (int r = 0; r < 4; ++r) HIP_OK(hipFree(outs[r]));
    HIP_OK(hipFree(ws));
    for (int r = 0; r < 8; ++r) HIP_OK(hipFree(d_in[r]));
    HIP_OK(hipFree(d_out));
    free(h);
}

/* The order argument is honoured: no reassociation across ranks. */
static void check_cancellation(void) {
    const size_t k = 64;
    const uint16_t vals[3] = {0x4C00 /* 2^25 */, 0x3F80 /* 1 */, 0xCC00 /* -2^25 */};
    uint16_t* h = host_alloc(k * 2);
    uint16_t* d[3];
    const uint16_t* in[3];
    for (int r = 0; r < 3; ++r) {
        d[r] = dev_alloc(k * 2);
        fill16(h, k, vals[r]);
        HIP_OK(hipMemcpy(d[r], h, k * 2, hipMemcpyHostToDevice));
        in[r] = d[r];
    }
    uint16_t* out = dev_alloc(k * 2);
    const int32_t o012[3] = {0, 1, 2}, o021[3] = {0, 2, 1};
    EXPECT(pc_reduce(in, 3, out, k, o012, NULL) == PC_OK, "cancellation status");
    HIP_OK(hipDeviceSynchronize());
    HIP_OK(hipMemcpy(h, out, k * 2, hipMemcpyDeviceToHost));
    EXPECT(all16(h, k, 0x0000), "(2^25 + 1) - 2^25 = +0");
    EXPECT(pc_reduce(in, 3, out, k, o021, NULL) == PC_OK, "cancellation status");
    HIP_OK(hipDeviceSynchronize());
    HIP_OK(hipMemcpy(h, out, k * 2, hipMemcpyDeviceToHost));
    EXPECT(all16(h, k, 0x3F80), "(2^25 - 2^25) + 1 = 1");
    for (int r = 0; r < 3; ++r) HIP_OK(hipFree(d[r]));
    HIP_OK(hipFree(out));
    free(h);
}

/* LL at one rank: pack then consume is the identity on every bf16 pattern. */
static void check_ll_identity(void) {
    const size_t k = 65536;
    uint16_t* h = host_alloc(k * 2);
    uint64_t* bm = host_alloc(k / 128 * 8);
    for (size_t i = 0; i < k; ++i) h[i] = (uint16_t)i;
    uint16_t* src = dev_alloc(k * 2);
    uint64_t* lines = dev_alloc(k / 2 * 8);
    uint16_t* out = dev_alloc(k * 2);
    uint64_t* d_bm = dev_alloc(k / 128 * 8);
    HIP_OK(hipMemcpy(src, h, k * 2, hipMemcpyHostToDevice));
    EXPECT(pc_pack_ll(src, lines, k, 7, NULL) == PC_OK, "pc_pack_ll status");
    const uint64_t* ln[1] = {lines};
    EXPECT(pc_consume_ll(ln, 1, out, k, 7, d_bm, NULL) == PC_OK, "pc_consume_ll status");
    HIP_OK(hipDeviceSynchronize());
    HIP_OK(hipMemcpy(h, out, k * 2, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(bm, d_bm, k / 128 * 8, hipMemcpyDeviceToHost));
    for (size_t i = 0; i < k; ++i) {
        const int nan = (i & 0x7F80u) == 0x7F80u && (i & 0x7Fu) != 0;
        EXPECT(h[i] == (nan ? 0x7FC0 : (uint16_t)i), "LL identity per pattern");
    }
    for (size_t w = 0; w < k / 128; ++w) EXPECT(bm[w] == ~(uint64_t)0, "LL all lines ready");
    /* Another sequence number: nothing ready, output untouched. */
    fill16(h, k, 0x1234);
    HIP_OK(hipMemcpy(out, h, k * 2, hipMemcpyHostToDevice));
    EXPECT(pc_consume_ll(ln, 1, out, k, 8, d_bm, NULL) == PC_OK, "pc_consume_ll status");
    HIP_OK(hipDeviceSynchronize());
    HIP_OK(hipMemcpy(h, out, k * 2, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(bm, d_bm, k / 128 * 8, hipMemcpyDeviceToHost));
    EXPECT(all16(h, k, 0x1234), "LL wrong seq leaves the output");
    for (size_t w = 0; w < k / 128; ++w) EXPECT(bm[w] == 0, "LL wrong seq: no ready bit");
    HIP_OK(hipFree(src));
    HIP_OK(hipFree(lines));
    HIP_OK(hipFree(out));
    HIP_OK(hipFree(d_bm));
    free(h);
    free(bm);
}

/* All-gather with every record current: the concatenation of the payloads. */
static void check_allgather_concat(void) {
    const int n = 3;
    const size_t shard_bytes = 8192 * 2, blocks = shard_bytes / PC_BLOCK_PAYLOAD_BYTES;
    const size_t rec_bytes = blocks * PC_BLOCK_RECORD_BYTES;
    uint8_t* h = host_alloc(rec_bytes);
    uint8_t* want = host_alloc(n * shard_bytes);
    uint8_t* got = host_alloc(n * shard_bytes);
    uint8_t* d_sh[3];
    const uint8_t* sh[3];
    const uint64_t seq = 0x100000009ull; /* compared as a full u64 */
    for (int r = 0; r < n; ++r) {
        for (size_t b = 0; b < blocks; ++b) {
            uint8_t* rec = h + b * PC_BLOCK_RECORD_BYTES;
            memcpy(rec, &seq, 8);
            for (size_t j = 0; j < PC_BLOCK_PAYLOAD_BYTES; ++j) {
                rec[8 + j] = (uint8_t)(r * 131 + b * 7 + j);
                want[(r * blocks + b) * PC_BLOCK_PAYLOAD_BYTES + j] = rec[8 + j];
            }
        }
        d_sh[r] = dev_alloc(rec_bytes);
        HIP_OK(hipMemcpy(d_sh[r], h, rec_bytes, hipMemcpyHostToDevice));
        sh[r] = d_sh[r];
    }
    uint16_t* out = dev_alloc(n * shard_bytes);
    uint64_t* d_bm = dev_alloc(n * blocks / 64 * 8);
    uint64_t bm[3 * 128 / 64];
    EXPECT(pc_allgather_copy(sh, n, out, shard_bytes, seq, d_bm, NULL) == PC_OK, "all-gather status");
    HIP_OK(hipDeviceSynchronize());
    HIP_OK(hipMemcpy(got, out, n * shard_bytes, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(bm, d_bm, sizeof bm, hipMemcpyDeviceToHost));
    EXPECT(memcmp(got, want, n * shard_bytes) == 0, "all-gather concatenation");
    for (size_t w = 0; w < n * blocks / 64; ++w) EXPECT(bm[w] == ~(uint64_t)0, "all-gather all ready");
    for (int r = 0; r < n; ++r) HIP_OK(hipFree(d_sh[r]));
    HIP_OK(hipFree(out));
    HIP_OK(hipFree(d_bm));
    free(h);
    free(want);
    free(got);
}

/* The Atom copy moves every byte pattern unchanged (NaN payloads too). */
static void check_copy(void) {
    const size_t bytes = 16 * (256 * 4 + 9);
    uint8_t* h = host_alloc(bytes);
    uint8_t* back = host_alloc(bytes);
    for (size_t i = 0; i < bytes; ++i) h[i] = (uint8_t)(i * 37 + (i >> 8));
    uint8_t* src = dev_alloc(bytes);
    uint8_t* dst = dev_alloc(bytes);
    HIP_OK(hipMemcpy(src, h, bytes, hipMemcpyHostToDevice));
    HIP_OK(hipMemset(dst, 0, bytes));
    EXPECT(pc_copy(dst, src, bytes, NULL) == PC_OK, "pc_copy status");
    HIP_OK(hipDeviceSynchronize());
    HIP_OK(hipMemcpy(back, dst, bytes, hipMemcpyDeviceToHost));
    EXPECT(memcmp(back, h, bytes) == 0, "pc_copy bytes unchanged");
    EXPECT(pc_copy(dst, dst + 16, 64, NULL) == PC_EINVAL, "pc_copy partial overlap");
    HIP_OK(hipFree(src));
    HIP_OK(hipFree(dst));
    free(h);
    free(back);
}

/* Rejected calls return their status codes; empty calls are no-ops. */
static void check_statuses(void) {
    uint16_t* a = dev_alloc(4096);
    uint16_t* out = dev_alloc(4096);
    const uint16_t* in[2] = {a, a};
    EXPECT(pc_reduce(in, 0, out, 8, NULL, NULL) == PC_EINVAL, "n = 0");
    EXPECT(pc_reduce(in, 9, out, 8, NULL, NULL) == PC_EINVAL, "n = 9");
    EXPECT(pc_reduce(in, 2, out, 12, NULL, NULL) == PC_EALIGN, "k not a multiple of 8");
    EXPECT(pc_reduce(in, 2, out + 1, 8, NULL, NULL) == PC_EALIGN, "misaligned output");
    EXPECT(pc_reduce(in, 2, a + 8, 64, NULL, NULL) == PC_EINVAL, "partial overlap");
    EXPECT(pc_reduce(in, 2, out, 0, NULL, NULL) == PC_OK, "empty reduce");
    EXPECT(pc_pack_ll(a, (uint64_t*)out, 8, 0, NULL) == PC_EINVAL, "seq = 0");
    EXPECT(pc_strerror(PC_EALIGN) != NULL && pc_strerror(12345) != NULL, "strerror");
    HIP_OK(hipFree(a));
    HIP_OK(hipFree(out));
}

int main(void) {
    int ndev = 0;
    if (hipGetDeviceCount(&ndev) != hipSuccess || ndev < 1) {
        printf("pc_abi_check: no GPU\n");
        return 77;
    }
    EXPECT(pc_abi_version() == PC_ABI_VERSION, "ABI version");
    check_statuses();
    check_copy();
    check_reduce_exact_sums();
    check_cancellation();
    check_ll_identity();
    check_allgather_concat();
    printf("pc_abi_check: OK\n");
    return 0;
}
