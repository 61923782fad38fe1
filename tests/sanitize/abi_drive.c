/* Drives the C ABI's host-side validation and size queries under the address
 * and undefined-behaviour sanitizers (the library's host code built with
 * them; device code is untouched).  Every call here fails validation or is a
 * host-only query, so nothing reaches a GPU.  The layer pointer tables of the
 * stream entry points are exact-size heap arrays, so a validation loop that
 * read one entry past `layers` would abort the run.  Built and run by
 * tests/test_abi_sanitizers.py; exits nonzero on any unexpected status. */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include "bq8.h"

static int fails = 0;
#define EXPECT(call, want)                                                                        \
    do {                                                                                          \
        const long got_ = (long)(call);                                                           \
        if (got_ != (long)(want)) {                                                               \
            fprintf(stderr, "FAIL line %d: %s -> %ld, want %ld\n", __LINE__, #call, got_,         \
                    (long)(want));                                                                \
            ++fails;                                                                              \
        }                                                                                         \
    } while (0)

int main(void)
{
    void *A = (void *)(uintptr_t)0x10000; /* aligned, never dereferenced */
    char *B = (char *)A;

    EXPECT(bq8_abi_version(), 1);
    for (int s = 0; s < 6; ++s)
        EXPECT(bq8_status_string((bq8_status)s)[0] != '\0', 1);

    /* quantize and the GGUF-layout products */
    EXPECT(q8_1_quantize(NULL, 1, 32, A, NULL), BQ8_ERR_NULL);
    EXPECT(q8_1_quantize(A, 0, 32, A, NULL), BQ8_ERR_SHAPE);
    EXPECT(q8_1_quantize((float *)(B + 2), 1, 32, A, NULL), BQ8_ERR_ALIGN);
    EXPECT(q4_0_mmvq_m6(NULL, 8, 64, A, A, NULL), BQ8_ERR_NULL);
    EXPECT(q4_0_mmvq_m6(A, 8, 48, A, A, NULL), BQ8_ERR_SHAPE);
    EXPECT(q4_0_mmvq_m17(B + 4, 8, 64, A, A, NULL), BQ8_ERR_ALIGN);
    EXPECT(q4_0_mmvq_m6(A, 8, 64, B + 4, A, NULL), BQ8_ERR_ALIGN); /* xq 4 mod 16 */
    EXPECT(q4_0_mmvq(A, 8, 64, A, 18, A, NULL), BQ8_ERR_SHAPE);

    /* packed layout */
    EXPECT(q4_0_pack_bytes(17408, 5120), 50135040);
    EXPECT(q4_0_pack_bytes(17408, 5000), -1);
    EXPECT(q4_0_pack(A, 16, 512, A, q4_0_pack_bytes(16, 512) - 1, NULL), BQ8_ERR_SIZE);
    EXPECT(q4_0_mmvq_packed(A, 16, 500, A, 6, A, NULL), BQ8_ERR_SHAPE);
    EXPECT(q4_0_mmvq_packed(A, 16, 512, B + 8, 6, A, NULL), BQ8_ERR_ALIGN); /* xq 8 mod 16 */
    EXPECT(q4_0_gate_up_silu_q8_1_packed(A, A, 64, 512, B + 4, 6, NULL, NULL, NULL, A, NULL),
           BQ8_ERR_ALIGN);
    EXPECT(q4_0_mmvq_packed_ws(A, 16, 512, A, 6, A, NULL, 1 << 20, NULL), BQ8_ERR_NULL);
    EXPECT(q4_0_mmvq_packed_ws(A, 16, 500, A, 6, A, A, 1 << 20, NULL), BQ8_ERR_SHAPE);
    EXPECT(q4_0_mmvq_packed_ws(A, 16, 512, A, 6, A, (char *)A + 128, 1 << 20, NULL),
           BQ8_ERR_ALIGN);
    EXPECT(q4_0_mmvq_packed_splits(5120, 17408), 4);
    EXPECT(q4_0_mmvq_packed_splits_rows(5120, 17408, 6), 4);
    EXPECT(q4_0_mmvq_packed_splits_rows(5120, 17408, 18), -1);
    EXPECT(q4_0_mmvq_packed_splits_rows(16, 256, 12), -1);
    EXPECT(q4_0_mmvq_packed_split(A, 16, 512, A, 6, 9, A, NULL), BQ8_ERR_SHAPE);
    EXPECT(q4_0_gate_up_silu_q8_1_packed(A, A, 48, 512, A, 6, NULL, NULL, NULL, A, NULL),
           BQ8_ERR_SHAPE); /* N % 32 != 0 */
    EXPECT(q4_0_gate_up_silu_q8_1_packed_ws(A, A, 64, 512, A, 6, NULL, NULL, NULL, A, NULL,
                                            1 << 24, NULL),
           BQ8_ERR_NULL);
    EXPECT(q4_0_gate_up_silu_q8_1_packed_ws(A, A, 48, 512, A, 6, NULL, NULL, NULL, A, A, 1 << 24,
                                            NULL),
           BQ8_ERR_SHAPE);
    EXPECT(q4_0_gate_up_silu_q8_1_packed_ws(A, A, 64, 512, A, 6, NULL, NULL, NULL, A,
                                            (char *)A + 128, 1 << 24, NULL),
           BQ8_ERR_ALIGN);

    /* Q6_K packs and the head */
    EXPECT(q6k_pack_bytes(248320, 5120), 1360793600);
    EXPECT(q6k_compact_bytes(248320, 5120), 1042944000);
    EXPECT(q6k_pack_expand(A, 248320, 5120, A, 1360793599, NULL), BQ8_ERR_SIZE);
    const int64_t sb = q6k_lmhead_top1_scratch_bytes(248320, 5120, 5);
    EXPECT(sb > 0 && sb < (1 << 20), 1);
    EXPECT(q6k_lmhead_top1_scratch_bytes(31040, 5120, 5) > 0, 1);
    EXPECT(q6k_lmhead_top1(A, 248320, 5120, A, 6, 1, 5, A, A, sb - 1, NULL), BQ8_ERR_SIZE);
    EXPECT(q6k_lmhead_top1(A, 248320, 5120, A, 6, 2, 5, A, A, sb, NULL), BQ8_ERR_SHAPE);
    EXPECT(q6k_lmhead_top1_compact(A, 248320, 5000, A, 6, 1, 5, A, A, sb, NULL), BQ8_ERR_SHAPE);
    EXPECT(q6k_lmhead_candidate_max(A, 248320, 5120, A, 6, 1, 5, NULL, 1, A, A, A, A, sb, NULL),
           BQ8_ERR_NULL); /* candidates asked for, no id array */
    EXPECT(q6k_lmhead_top1_noalloc(A, 248320, 5120, A, 6, 1, 5, NULL, NULL), BQ8_ERR_NULL);
    EXPECT(q6k_lmhead_top1_noalloc(A, 248320, 5120, A, 6, 2, 5, A, NULL), BQ8_ERR_SHAPE);
    EXPECT(q6k_lmhead_top1_noalloc(A, 248320, 24576, A, 9, 1, 8, A, NULL), BQ8_ERR_SIZE);

    /* glue and the summed RMS step */
    EXPECT(silu_mul_q8_1(A, A, 6, 48, NULL, A, NULL), BQ8_ERR_SHAPE);
    EXPECT(rms_norm_q8_1(A, 6, 5120, 0.0f, NULL, A, NULL), BQ8_ERR_SHAPE);
    EXPECT(rms_norm_q8_1_sum(A, 9, 6, 5120, 1e-6f, A, NULL, A, NULL), BQ8_ERR_SHAPE);

    /* the stream: exact-size layer tables, the last entry bad */
    int64_t off[5];
    EXPECT(q4_0_ffn_stream_layout(6, 5120, 17408, off), BQ8_OK);
    const int64_t layers = 3;
    const void **g = malloc(sizeof(void *) * layers), **u = malloc(sizeof(void *) * layers),
               **d = malloc(sizeof(void *) * layers);
    for (int64_t l = 0; l < layers; ++l)
        g[l] = u[l] = d[l] = B + 0x100 * l;
    d[layers - 1] = B + 8;
    EXPECT(q4_0_ffn_stream(g, u, d, layers, 6, 5120, 17408, A, 1e-6f, A, A, off[4], NULL),
           BQ8_ERR_ALIGN);
    EXPECT(q4_0_ffn_stream_packed(g, u, d, layers, 6, 5120, 17408, A, 1e-6f, A, A, off[4], NULL),
           BQ8_ERR_ALIGN);
    d[layers - 1] = NULL;
    EXPECT(q4_0_ffn_stream(g, u, d, layers, 6, 5120, 17408, A, 1e-6f, A, A, off[4], NULL),
           BQ8_ERR_NULL);
    d[layers - 1] = B;
    EXPECT(q4_0_ffn_stream(g, u, d, layers, 6, 5120, 17408, A, 1e-6f, A, A, off[4] - 1, NULL),
           BQ8_ERR_SIZE);
    free(g), free(u), free(d);

    /* the read probe */
    EXPECT(bq8_hbm_read_probe(A, 1032, 4, 4, A, NULL), BQ8_ERR_SHAPE);
    EXPECT(bq8_hbm_read_probe(A, 1024, 4, 3, A, NULL), BQ8_ERR_SHAPE);

    if (fails)
        return 1;
    printf("ok\n");
    return 0;
}
