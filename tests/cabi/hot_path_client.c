/* A plain C client of the C ABI (no Python, no torch): device memory from the
 * HIP runtime, a stream of its own, and every step of the hot path through
 * libbq8.so, checked against the CPU oracle (libbq8_oracle.so, test
 * infrastructure) on the same inputs.
 *
 *   Q8_1 quantize of x [6][5120]                 bytes equal the oracle's
 *   Q4_0 products, M = 6, [4103 x 5120]           GGUF layout and packed,
 *                                                 |gpu - oracle| <= 1e-5*bound + 1e-6
 *   Q6_K head, rows 1..5 of x, [3001 x 5120]      expanded, compact and
 *                                                 allocation-free calls: ids
 *                                                 equal the oracle's up to a
 *                                                 near tie within the bound
 *
 * Inputs come from one counter-based generator (splitmix64) below; it holds
 * none of the method's arithmetic.  Built and run by
 * tests/test_gpu_c_client.py; prints one line per check and exits nonzero on
 * the first failure. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "bq8.h"

/* the oracle's entry points (it ships no header) */
void orc_q8_1_quantize(const float *x, int64_t M, int64_t K, uint8_t *out);
void orc_q4_0_q8_1_gemv(const uint8_t *w, int64_t N, int64_t K, const uint8_t *xq, int64_t M,
                        double *y, double *bound);
void orc_q6k_pack_expand(const uint8_t *raw, int64_t N, int64_t K, uint8_t *pack);
void orc_q6k_lmhead_top1(const uint8_t *pack, int64_t N, int64_t K, const float *x, int64_t M,
                         int64_t row0, int64_t rows, uint8_t *xq_out, double *logits,
                         double *bound, int32_t *ids);

#define CHECK_HIP(call)                                                                           \
    do {                                                                                          \
        hipError_t e_ = (call);                                                                   \
        if (e_ != hipSuccess) {                                                                   \
            fprintf(stderr, "HIP error %s at line %d: %s\n", hipGetErrorString(e_), __LINE__,    \
                    #call);                                                                       \
            exit(2);                                                                              \
        }                                                                                         \
    } while (0)
#define CHECK_BQ8(call)                                                                           \
    do {                                                                                          \
        bq8_status s_ = (call);                                                                   \
        if (s_ != BQ8_OK) {                                                                       \
            fprintf(stderr, "bq8 error %s at line %d: %s\n", bq8_status_string(s_), __LINE__,    \
                    #call);                                                                       \
            exit(3);                                                                              \
        }                                                                                         \
    } while (0)

static uint64_t splitmix64(uint64_t *state)
{
    uint64_t z = (*state += 0x9E3779B97F4A7C15ull);
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

/* uniform in [-2, 2), a multiple of 2^-22 */
static float gen_unit(uint64_t *state)
{
    return (float)((int64_t)(splitmix64(state) >> 40) - (1 << 23)) * (1.0f / (1 << 22));
}

/* Q4_0 blocks: random nibbles, fp16 scale bits in [0x1400, 0x17FF] (about 1e-3) */
static void gen_q4_0(uint64_t seed, int64_t N, int64_t K, uint8_t *w)
{
    uint64_t st = seed;
    for (int64_t i = 0; i < N * (K / 32); ++i) {
        uint8_t *b = w + i * 18;
        const uint64_t r = splitmix64(&st);
        const uint16_t d = (uint16_t)(0x1400 + (r & 0x3FF));
        b[0] = (uint8_t)(d & 0xFF);
        b[1] = (uint8_t)(d >> 8);
        for (int j = 0; j < 16; j += 8) {
            uint64_t q = splitmix64(&st);
            memcpy(b + 2 + j, &q, 8);
        }
    }
}

/* raw Q6_K superblocks: random ql, qh and subscales, fp16 d bits in
 * [0x1000, 0x13FF] (about 5e-4) */
static void gen_q6k(uint64_t seed, int64_t N, int64_t K, uint8_t *raw)
{
    uint64_t st = seed;
    for (int64_t i = 0; i < N * (K / 256); ++i) {
        uint8_t *b = raw + i * 210;
        for (int j = 0; j < 208; j += 8) {
            uint64_t q = splitmix64(&st);
            memcpy(b + j, &q, 8);
        }
        const uint16_t d = (uint16_t)(0x1000 + (splitmix64(&st) & 0x3FF));
        b[208] = (uint8_t)(d & 0xFF);
        b[209] = (uint8_t)(d >> 8);
    }
}

static void *dmalloc(size_t bytes)
{
    void *p = NULL;
    CHECK_HIP(hipMalloc(&p, bytes));
    return p;
}

static int check_close(const char *what, const float *gpu, const double *ref, const double *bound,
                       int64_t n)
{
    double worst = 0.0;
    for (int64_t i = 0; i < n; ++i) {
        const double tol = 1e-5 * bound[i] + 1e-6;
        const double err = fabs((double)gpu[i] - ref[i]);
        if (!(err <= tol)) {
            fprintf(stderr, "%s: element %ld gpu %.9g oracle %.9g tol %.3g\n", what, (long)i,
                    (double)gpu[i], ref[i], tol);
            return 1;
        }
        if (err / tol > worst)
            worst = err / tol;
    }
    printf("ok %-40s %ld values, worst error %.3f of the bound\n", what, (long)n, worst);
    return 0;
}

/* ids equal, or a near tie: the oracle's logit of its own id exceeds that of
 * the GPU's id by no more than one logit's float bound */
static int check_ids(const char *what, const int32_t *gpu, const int32_t *ref,
                     const double *logits, const double *bound, int64_t rows, int64_t N)
{
    int near = 0;
    for (int64_t r = 0; r < rows; ++r) {
        const int32_t g = gpu[r], o = ref[r];
        if (g == o)
            continue;
        if (g < 0 || g >= N) {
            fprintf(stderr, "%s: row %ld id %d out of range\n", what, (long)r, g);
            return 1;
        }
        const double gap = logits[r * N + o] - logits[r * N + g];
        const double bo = bound[r * N + o], bg = bound[r * N + g];
        const double tol = 1e-5 * (bo > bg ? bo : bg) + 1e-6;
        if (!(gap <= tol)) {
            fprintf(stderr, "%s: row %ld gpu %d oracle %d gap %.9g > %.3g\n", what, (long)r, g, o,
                    gap, tol);
            return 1;
        }
        ++near;
    }
    printf("ok %-40s %ld rows, %d near-tie differences accepted\n", what, (long)rows, near);
    return 0;
}

int main(void)
{
    int ndev = 0;
    CHECK_HIP(hipGetDeviceCount(&ndev));
    if (ndev < 1) {
        fprintf(stderr, "no GPU\n");
        return 4;
    }
    CHECK_HIP(hipSetDevice(0));
    hipStream_t stream;
    CHECK_HIP(hipStreamCreate(&stream));
    printf("bq8 ABI version %d\n", (int)bq8_abi_version());

    /* ---- Q8_1 quantize of x [6][5120] */
    const int64_t M = 6, K = 5120, nb = K / 32;
    const size_t xbytes = (size_t)(M * K) * sizeof(float), xqbytes = (size_t)(M * nb * 36);
    float *x = (float *)malloc(xbytes);
    uint64_t st = 20251;
    for (int64_t i = 0; i < M * K; ++i)
        x[i] = gen_unit(&st);
    float *xd = (float *)dmalloc(xbytes);
    uint8_t *xqd = (uint8_t *)dmalloc(xqbytes);
    CHECK_HIP(hipMemcpy(xd, x, xbytes, hipMemcpyHostToDevice));
    CHECK_BQ8(q8_1_quantize(xd, M, K, xqd, stream));
    CHECK_HIP(hipStreamSynchronize(stream));
    uint8_t *xq = (uint8_t *)malloc(xqbytes), *xq_ref = (uint8_t *)malloc(xqbytes);
    CHECK_HIP(hipMemcpy(xq, xqd, xqbytes, hipMemcpyDeviceToHost));
    orc_q8_1_quantize(x, M, K, xq_ref);
    if (memcmp(xq, xq_ref, xqbytes) != 0) {
        fprintf(stderr, "q8_1_quantize: bytes differ from the oracle's\n");
        return 1;
    }
    printf("ok %-40s %zu bytes equal\n", "q8_1_quantize [6][5120]", xqbytes);

    /* ---- Q4_0 products at M = 6 on a ragged row count */
    const int64_t N = 4103;
    const size_t wbytes = (size_t)(N * nb * 18), ybytes = (size_t)(M * N) * sizeof(float);
    uint8_t *w = (uint8_t *)malloc(wbytes);
    gen_q4_0(7, N, K, w);
    uint8_t *wd = (uint8_t *)dmalloc(wbytes);
    CHECK_HIP(hipMemcpy(wd, w, wbytes, hipMemcpyHostToDevice));
    const int64_t wpbytes = q4_0_pack_bytes(N, K);
    if (wpbytes != (int64_t)wbytes) {
        fprintf(stderr, "q4_0_pack_bytes %ld, want %zu\n", (long)wpbytes, wbytes);
        return 1;
    }
    uint8_t *wpd = (uint8_t *)dmalloc((size_t)wpbytes);
    float *yd = (float *)dmalloc(ybytes);
    double *yref = (double *)malloc((size_t)(M * N) * sizeof(double));
    double *ybound = (double *)malloc((size_t)(M * N) * sizeof(double));
    float *y = (float *)malloc(ybytes);
    orc_q4_0_q8_1_gemv(w, N, K, xq_ref, M, yref, ybound);

    CHECK_BQ8(q4_0_mmvq_m6(wd, N, K, xqd, yd, stream));
    CHECK_HIP(hipStreamSynchronize(stream));
    CHECK_HIP(hipMemcpy(y, yd, ybytes, hipMemcpyDeviceToHost));
    if (check_close("q4_0_mmvq_m6 [4103 x 5120]", y, yref, ybound, M * N))
        return 1;
    CHECK_BQ8(q4_0_pack(wd, N, K, wpd, wpbytes, stream));
    CHECK_HIP(hipMemsetAsync(yd, 0xFF, ybytes, stream));
    CHECK_BQ8(q4_0_mmvq_packed(wpd, N, K, xqd, M, yd, stream));
    CHECK_HIP(hipStreamSynchronize(stream));
    CHECK_HIP(hipMemcpy(y, yd, ybytes, hipMemcpyDeviceToHost));
    if (check_close("q4_0_mmvq_packed M=6 [4103 x 5120]", y, yref, ybound, M * N))
        return 1;

    /* ---- Q6_K head: rows 1..5 of x through [3001 x 5120] */
    const int64_t V = 3001, row0 = 1, rows = 5;
    const size_t rawbytes = (size_t)(V * (K / 256) * 210);
    uint8_t *raw = (uint8_t *)malloc(rawbytes);
    gen_q6k(11, V, K, raw);
    const int64_t pbytes = q6k_pack_bytes(V, K), cbytes = q6k_compact_bytes(V, K);
    uint8_t *pack = (uint8_t *)malloc((size_t)pbytes);
    orc_q6k_pack_expand(raw, V, K, pack);
    uint8_t *hxq = (uint8_t *)malloc((size_t)(rows * nb * 36));
    double *logits = (double *)malloc((size_t)(rows * V) * sizeof(double));
    double *lbound = (double *)malloc((size_t)(rows * V) * sizeof(double));
    int32_t ids_ref[8] = {0}, ids[8] = {0};
    orc_q6k_lmhead_top1(pack, V, K, x, M, row0, rows, hxq, logits, lbound, ids_ref);

    uint8_t *rawd = (uint8_t *)dmalloc(rawbytes);
    uint8_t *packd = (uint8_t *)dmalloc((size_t)pbytes);
    uint8_t *cpackd = (uint8_t *)dmalloc((size_t)cbytes);
    const int64_t sbytes = q6k_lmhead_top1_scratch_bytes(V, K, rows);
    void *scratch = dmalloc((size_t)sbytes);
    int32_t *idsd = (int32_t *)dmalloc(8 * sizeof(int32_t));
    CHECK_HIP(hipMemcpy(rawd, raw, rawbytes, hipMemcpyHostToDevice));
    CHECK_BQ8(q6k_pack_expand(rawd, V, K, packd, pbytes, stream));
    CHECK_BQ8(q6k_pack_compact(rawd, V, K, cpackd, cbytes, stream));
    CHECK_HIP(hipStreamSynchronize(stream));
    {
        uint8_t *pgpu = (uint8_t *)malloc((size_t)pbytes);
        CHECK_HIP(hipMemcpy(pgpu, packd, (size_t)pbytes, hipMemcpyDeviceToHost));
        if (memcmp(pgpu, pack, (size_t)pbytes) != 0) {
            fprintf(stderr, "q6k_pack_expand: bytes differ from the oracle's\n");
            return 1;
        }
        free(pgpu);
        printf("ok %-40s %ld bytes equal\n", "q6k_pack_expand [3001 x 5120]", (long)pbytes);
    }

    int32_t first[8] = {0};
    for (int kind = 0; kind < 3; ++kind) {
        static const char *names[3] = {"q6k_lmhead_top1 (expanded)",
                                       "q6k_lmhead_top1_compact",
                                       "q6k_lmhead_top1_noalloc"};
        CHECK_HIP(hipMemsetAsync(idsd, 0xFF, 8 * sizeof(int32_t), stream));
        if (kind == 0)
            CHECK_BQ8(q6k_lmhead_top1(packd, V, K, xd, M, row0, rows, idsd, scratch, sbytes,
                                      stream));
        else if (kind == 1)
            CHECK_BQ8(q6k_lmhead_top1_compact(cpackd, V, K, xd, M, row0, rows, idsd, scratch,
                                              sbytes, stream));
        else
            CHECK_BQ8(q6k_lmhead_top1_noalloc(packd, V, K, xd, M, row0, rows, idsd, stream));
        CHECK_HIP(hipStreamSynchronize(stream));
        CHECK_HIP(hipMemcpy(ids, idsd, (size_t)rows * sizeof(int32_t), hipMemcpyDeviceToHost));
        if (check_ids(names[kind], ids, ids_ref, logits, lbound, rows, V))
            return 1;
        if (kind == 0)
            memcpy(first, ids, sizeof(ids));
        else if (memcmp(first, ids, (size_t)rows * sizeof(int32_t)) != 0) {
            fprintf(stderr, "%s: ids differ from the expanded pack's\n", names[kind]);
            return 1;
        }
    }

    /* a rejected call touches nothing and names its error */
    const bq8_status bad = q4_0_mmvq_packed(wpd, N, K + 1, xqd, M, yd, stream);
    if (bad != BQ8_ERR_SHAPE) {
        fprintf(stderr, "K = 5121 on the packed product: status %d, want BQ8_ERR_SHAPE\n", (int)bad);
        return 1;
    }
    printf("ok %-40s %s\n", "invalid shape rejected", bq8_status_string(bad));

    CHECK_HIP(hipStreamSynchronize(stream));
    CHECK_HIP(hipStreamDestroy(stream));
    CHECK_HIP(hipFree(xd));
    CHECK_HIP(hipFree(xqd));
    CHECK_HIP(hipFree(wd));
    CHECK_HIP(hipFree(wpd));
    CHECK_HIP(hipFree(yd));
    CHECK_HIP(hipFree(rawd));
    CHECK_HIP(hipFree(packd));
    CHECK_HIP(hipFree(cpackd));
    CHECK_HIP(hipFree(scratch));
    CHECK_HIP(hipFree(idsd));
    free(x);
    free(xq);
    free(xq_ref);
    free(w);
    free(yref);
    free(ybound);
    free(y);
    free(raw);
    free(pack);
    free(hxq);
    free(logits);
    free(lbound);
    printf("all checks passed\n");
    return 0;
}
