/* Drives every entry point of the oracle on small, ragged shapes with
 * exact-size heap buffers, so that an address sanitizer build catches any
 * read or write past a buffer's end, and an undefined-behaviour build any
 * bad shift, overflow or misaligned access.  Also checks the round trips the
 * oracle's pins rely on.  Built and run by tests/test_oracle_sanitizers.py;
 * exits nonzero on any failed check. */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

float orc_f16_to_f32(uint16_t h);
uint16_t orc_f32_to_f16(float x);
void orc_f32_to_f16_array(const float *x, uint16_t *h, int64_t n);
void orc_f16_to_f32_array(const uint16_t *h, float *x, int64_t n);
void orc_q8_1_quantize(const float *x, int64_t M, int64_t K, uint8_t *out);
void orc_q8_1_fields(const uint8_t *xq, int64_t nblocks, uint16_t *d, uint16_t *s, int8_t *q);
void orc_q4_0_decode(const uint8_t *w, int64_t N, int64_t K, uint16_t *d, uint8_t *q);
void orc_q4_0_encode(const uint16_t *d, const uint8_t *q, int64_t N, int64_t K, uint8_t *w);
void orc_q4_0_q8_1_gemv(const uint8_t *w, int64_t N, int64_t K, const uint8_t *xq, int64_t M,
                        double *y, double *bound);
int64_t orc_q4_0_pack_bytes(int64_t N, int64_t K);
void orc_q4_0_pack(const uint8_t *w, int64_t N, int64_t K, uint8_t *wp);
void orc_q4_0_unpack(const uint8_t *wp, int64_t N, int64_t K, uint8_t *w);
void orc_q4_0p_q8_1_gemv(const uint8_t *wp, int64_t N, int64_t K, const uint8_t *xq, int64_t M,
                         double *y, double *bound);
void orc_q6k_decode(const uint8_t *raw, int64_t N, int64_t K, int8_t *q, int8_t *sc,
                    uint16_t *d);
void orc_q6k_encode(const int8_t *q, const int8_t *sc, const uint16_t *d, int64_t N, int64_t K,
                    uint8_t *raw);
int64_t orc_q6k_pack_bytes(int64_t N, int64_t K);
void orc_q6k_pack_expand(const uint8_t *raw, int64_t N, int64_t K, uint8_t *pack);
void orc_q6k_pack_logits(const uint8_t *pack, int64_t N, int64_t K, const uint8_t *xq,
                         int64_t rows, double *logits, double *bound);
int64_t orc_q6k_compact_bytes(int64_t N, int64_t K);
void orc_q6k_pack_compact(const uint8_t *raw, int64_t N, int64_t K, uint8_t *pack);
void orc_q6k_compact_unpack(const uint8_t *pack, int64_t N, int64_t K, uint8_t *raw);
void orc_top1(const double *logits, int64_t rows, int64_t N, int32_t *ids);
void orc_q6k_lmhead_top1(const uint8_t *pack, int64_t N, int64_t K, const float *x, int64_t M,
                         int64_t row0, int64_t rows, uint8_t *xq_out, double *logits,
                         double *bound, int32_t *ids);
void orc_silu_mul(const float *g, const float *u, int64_t n, double *h);
void orc_rms_norm(const float *y, int64_t M, int64_t K, double eps, double *out);

static uint64_t rng = 0x9E3779B97F4A7C15ull;
static uint32_t next32(void)
{
    rng ^= rng << 13;
    rng ^= rng >> 7;
    rng ^= rng << 17;
    return (uint32_t)(rng >> 11);
}
static float normal_ish(void) /* sum of uniforms, about N(0, 1) */
{
    float s = 0.0f;
    for (int i = 0; i < 12; ++i)
        s += (float)(next32() & 0xFFFFFF) / 16777216.0f;
    return s - 6.0f;
}
static void *xmalloc(size_t n) { return malloc(n ? n : 1); }
static int fails = 0;
#define CHECK(c, what)                                                                            \
    do {                                                                                          \
        if (!(c)) {                                                                               \
            fprintf(stderr, "FAIL %s (line %d)\n", what, __LINE__);                               \
            ++fails;                                                                              \
        }                                                                                         \
    } while (0)

/* random Q4_0 rows with fp16 scales in [1e-3, 2e-2) */
static uint8_t *q4_0_weights(int64_t N, int64_t K)
{
    const int64_t nb = K / 32;
    uint8_t *w = xmalloc((size_t)(N * nb * 18));
    for (int64_t i = 0; i < N * nb; ++i) {
        const uint16_t d = orc_f32_to_f16(1e-3f + 0.019f * (float)(next32() & 0xFFFF) / 65536.0f);
        w[i * 18] = (uint8_t)d;
        w[i * 18 + 1] = (uint8_t)(d >> 8);
        for (int j = 0; j < 16; ++j)
            w[i * 18 + 2 + j] = (uint8_t)next32();
    }
    return w;
}

static void q4_0_case(int64_t N, int64_t K, int64_t M)
{
    const int64_t nb = K / 32;
    float *x = xmalloc((size_t)(M * K) * sizeof(float));
    for (int64_t i = 0; i < M * K; ++i)
        x[i] = normal_ish();
    uint8_t *xq = xmalloc((size_t)(M * nb * 36));
    orc_q8_1_quantize(x, M, K, xq);
    uint16_t *d = xmalloc((size_t)(M * nb) * 2), *s = xmalloc((size_t)(M * nb) * 2);
    int8_t *q = xmalloc((size_t)(M * nb * 32));
    orc_q8_1_fields(xq, M * nb, d, s, q);

    uint8_t *w = q4_0_weights(N, K);
    uint16_t *wd = xmalloc((size_t)(N * nb) * 2);
    uint8_t *wq = xmalloc((size_t)(N * K));
    orc_q4_0_decode(w, N, K, wd, wq);
    uint8_t *w2 = xmalloc((size_t)(N * nb * 18));
    orc_q4_0_encode(wd, wq, N, K, w2);
    CHECK(memcmp(w, w2, (size_t)(N * nb * 18)) == 0, "q4_0 encode(decode(w)) == w");

    double *y = xmalloc((size_t)(M * N) * sizeof(double));
    double *b = xmalloc((size_t)(M * N) * sizeof(double));
    orc_q4_0_q8_1_gemv(w, N, K, xq, M, y, b);
    if (K % 512 == 0) {
        const int64_t pb = orc_q4_0_pack_bytes(N, K);
        CHECK(pb == N * nb * 18, "q4_0 pack size");
        uint8_t *wp = xmalloc((size_t)pb), *w3 = xmalloc((size_t)pb);
        orc_q4_0_pack(w, N, K, wp);
        orc_q4_0_unpack(wp, N, K, w3);
        CHECK(memcmp(w, w3, (size_t)pb) == 0, "q4_0 unpack(pack(w)) == w");
        double *yp = xmalloc((size_t)(M * N) * sizeof(double));
        double *bp = xmalloc((size_t)(M * N) * sizeof(double));
        orc_q4_0p_q8_1_gemv(wp, N, K, xq, M, yp, bp);
        CHECK(memcmp(y, yp, (size_t)(M * N) * sizeof(double)) == 0, "packed gemv == gemv");
        free(wp), free(w3), free(yp), free(bp);
    }
    free(x), free(xq), free(d), free(s), free(q), free(w), free(wd), free(wq), free(w2), free(y),
        free(b);
}

static void q6k_case(int64_t N, int64_t K, int64_t M, int64_t row0, int64_t rows)
{
    const int64_t ns = K / 256;
    uint8_t *raw = xmalloc((size_t)(N * ns * 210));
    for (int64_t i = 0; i < N * ns; ++i) {
        uint8_t *blk = raw + i * 210;
        for (int j = 0; j < 192; ++j)
            blk[j] = (uint8_t)next32();
        for (int j = 0; j < 16; ++j)
            blk[192 + j] = (uint8_t)(int8_t)((int)(next32() % 128) - 64);
        const uint16_t d = orc_f32_to_f16(1e-4f + 9e-4f * (float)(next32() & 0xFFFF) / 65536.0f);
        blk[208] = (uint8_t)d;
        blk[209] = (uint8_t)(d >> 8);
    }
    int8_t *q = xmalloc((size_t)(N * K)), *sc = xmalloc((size_t)(N * K / 16));
    uint16_t *d = xmalloc((size_t)(N * ns) * 2);
    orc_q6k_decode(raw, N, K, q, sc, d);
    uint8_t *raw2 = xmalloc((size_t)(N * ns * 210));
    orc_q6k_encode(q, sc, d, N, K, raw2);
    CHECK(memcmp(raw, raw2, (size_t)(N * ns * 210)) == 0, "q6k encode(decode(raw)) == raw");

    const int64_t pb = orc_q6k_pack_bytes(N, K);
    uint8_t *pack = xmalloc((size_t)pb);
    orc_q6k_pack_expand(raw, N, K, pack);
    const int64_t cb = orc_q6k_compact_bytes(N, K);
    CHECK(cb == N * ns * 210, "compact size");
    uint8_t *cpk = xmalloc((size_t)cb), *raw3 = xmalloc((size_t)cb);
    orc_q6k_pack_compact(raw, N, K, cpk);
    orc_q6k_compact_unpack(cpk, N, K, raw3);
    CHECK(memcmp(raw, raw3, (size_t)cb) == 0, "compact unpack(pack(raw)) == raw");

    float *x = xmalloc((size_t)(M * K) * sizeof(float));
    for (int64_t i = 0; i < M * K; ++i)
        x[i] = normal_ish();
    uint8_t *xq = xmalloc((size_t)(rows * (K / 32) * 36));
    double *lg = xmalloc((size_t)(rows * N) * sizeof(double));
    double *bd = xmalloc((size_t)(rows * N) * sizeof(double));
    int32_t *ids = xmalloc((size_t)rows * sizeof(int32_t));
    orc_q6k_lmhead_top1(pack, N, K, x, M, row0, rows, xq, lg, bd, ids);
    double *lg2 = xmalloc((size_t)(rows * N) * sizeof(double));
    double *bd2 = xmalloc((size_t)(rows * N) * sizeof(double));
    orc_q6k_pack_logits(pack, N, K, xq, rows, lg2, bd2);
    CHECK(memcmp(lg, lg2, (size_t)(rows * N) * sizeof(double)) == 0, "head logits agree");
    int32_t *ids2 = xmalloc((size_t)rows * sizeof(int32_t));
    orc_top1(lg, rows, N, ids2);
    for (int64_t r = 0; r < rows; ++r)
        CHECK(ids[r] == ids2[r] && ids[r] >= 0 && ids[r] < N, "top-1 ids agree and in range");
    free(raw), free(q), free(sc), free(d), free(raw2), free(pack), free(cpk), free(raw3), free(x),
        free(xq), free(lg), free(bd), free(ids), free(lg2), free(bd2), free(ids2);
}

int main(void)
{
    /* fp16 codec: every pattern, and the array forms at an odd length */
    for (uint32_t h = 0; h < 65536; ++h) {
        const float f = orc_f16_to_f32((uint16_t)h);
        if (f == f)
            CHECK(orc_f16_to_f32(orc_f32_to_f16(f)) == f || (h & 0x7FFF) == 0, "fp16 round trip");
    }
    float fa[7];
    uint16_t ha[7];
    for (int i = 0; i < 7; ++i)
        fa[i] = normal_ish();
    orc_f32_to_f16_array(fa, ha, 7);
    orc_f16_to_f32_array(ha, fa, 7);

    q4_0_case(1, 32, 1);
    q4_0_case(37, 1024, 3);
    q4_0_case(33, 512, 17);
    q4_0_case(16, 96, 6);
    q6k_case(1, 256, 1, 0, 1);
    q6k_case(130, 512, 6, 1, 5);
    q6k_case(64, 768, 8, 0, 8);

    float g[45], u[45];
    double h[45], rn[45];
    for (int i = 0; i < 45; ++i)
        g[i] = normal_ish(), u[i] = normal_ish();
    orc_silu_mul(g, u, 45, h);
    orc_rms_norm(g, 3, 15, 1e-6, rn);
    if (fails)
        return 1;
    printf("ok\n");
    return 0;
}
