/*
 * bq8_oracle.c -- plain, slow, scalar CPU oracle for the block-quantized
 * GEMV hot path (Q8_1 activations, Q4_0 and Q6_K weights, greedy top-1).
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  The GPU library never
 * links, includes or calls anything here, and this file includes nothing
 * from the GPU library: the two share no code.
 *
 * Sources (web pages of the b70-optimization-lab and neural.download sites):
 *   [CLOSURE] "Qwen3.6 27B Q4_0 DFlash/SYCL closure",
 *             sections "What materially worked", "Why the objectives were
 *             missed" (Q4_0 MMVQ at verifier width, rows 1..17).
 *   [TOP1]    "Q6_K M=6 fused DFlash top-1 production record",
 *             sections "Outcome", "Why this was slow", "Exactness and safety
 *             contracts", "Memory and startup".
 *   [Q8CACHE] "Qwen3.6 27B B70 follow-up: Q8 activation cache, FP8 artifacts,
 *             MTP blocker", section "Q8_1 activation cache prototype".
 * The pages name the formats (Q4_0 weights, exact Q8_1 activations, Q6_K
 * expanded to int8 quants + int8 subscales + fp16 superblock scales) but not
 * their bit layouts; the layouts below are the public GGUF block formats,
 * which the pages' .gguf model files use.  Every such reading is marked
 * READING.
 *
 * Precision: every dot product is the plain definition -- dequantize each
 * element, multiply, accumulate -- in IEEE binary64.  With fp16 scales, int8
 * subscales and small integer quants every element product and every 32-wide
 * block sum is exact in binary64, so results differ from the exact real value
 * only by the final summation over blocks.  The Q8_1 quantizer decides
 * integers (the quants) from floating point, so it works in binary32, the
 * precision a GPU kernel uses, and both sides decide them identically.
 *
 * Build: gcc -O2 -ffp-contract=off -fno-fast-math -fopenmp -shared -fPIC.
 * OpenMP splits only over output rows; each row is summed in a fixed order,
 * so results do not depend on the thread count.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define QK 32          /* elements per Q4_0 / Q8_1 block */
#define QK_K 256       /* elements per Q6_K superblock   */
#define Q4_0_BYTES 18  /* fp16 d + 16 bytes of nibbles  */
#define Q8_1_BYTES 36  /* fp16 d + fp16 s + 32 int8      */
#define Q6_K_BYTES 210 /* ql[128] qh[64] scales[16] d    */

/* ------------------------------------------------------------------------ */
/* IEEE 754 binary16 <-> binary32, written from the format definition:       */
/* 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits; exponent 0 is    */
/* zero/subnormal (fraction * 2^-24), exponent 31 is inf/NaN.                */
/* ------------------------------------------------------------------------ */

float orc_f16_to_f32(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 31;
    int f = h & 1023;
    double v;
    if (e == 0)
        v = ldexp((double)f, -24);
    else if (e == 31)
        v = f ? NAN : INFINITY;
    else
        v = ldexp((double)(1024 + f), e - 25);
    return (float)(sign ? -v : v);
}

/* Round a non-negative double that holds an exactly representable
 * quotient to the nearest integer, ties to even. */
static double round_half_even(double v)
{
    double r = floor(v);
    double diff = v - r;
    if (diff > 0.5)
        return r + 1.0;
    if (diff < 0.5)
        return r;
    return fmod(r, 2.0) == 0.0 ? r : r + 1.0;
}

/* Round-to-nearest-even conversion binary32 -> binary16. */
uint16_t orc_f32_to_f16(float x)
{
    uint16_t sign = signbit(x) ? 0x8000u : 0u;
    if (isnan(x))
        return (uint16_t)(sign | 0x7E00u);
    double a = fabs((double)x);
    /* 65504 is the largest finite binary16; the half-way point to the next
     * (unrepresentable) step 65536 is 65520, and a tie rounds to the even
     * neighbour 65536, i.e. to infinity. */
    if (a >= 65520.0)
        return (uint16_t)(sign | 0x7C00u);
    if (a < ldexp(1.0, -14)) {
        /* subnormal range: quantum 2^-24; a result of 1024 quanta is the
         * smallest normal number, whose bit pattern is the same integer. */
        double q = round_half_even(ldexp(a, 24));
        return (uint16_t)(sign | (uint16_t)q);
    }
    int e2;
    frexp(a, &e2);            /* a = m * 2^e2 with m in [0.5, 1) */
    int e = e2 - 1;           /* a in [2^e, 2^(e+1)) */
    double m = round_half_even(ldexp(a, 10 - e)); /* in [1024, 2048] */
    if (m == 2048.0) {
        m = 1024.0;
        e += 1;
    }
    if (e + 15 >= 31)
        return (uint16_t)(sign | 0x7C00u);
    return (uint16_t)(sign | (uint16_t)((e + 15) << 10) | (uint16_t)(m - 1024.0));
}

void orc_f32_to_f16_array(const float *x, uint16_t *h, int64_t n)
{
    for (int64_t i = 0; i < n; ++i)
        h[i] = orc_f32_to_f16(x[i]);
}

void orc_f16_to_f32_array(const uint16_t *h, float *x, int64_t n)
{
    for (int64_t i = 0; i < n; ++i)
        x[i] = orc_f16_to_f32(h[i]);
}

static uint16_t rd16(const uint8_t *p) { return (uint16_t)(p[0] | (p[1] << 8)); }
static void wr16(uint8_t *p, uint16_t v)
{
    p[0] = (uint8_t)(v & 0xFF);
    p[1] = (uint8_t)(v >> 8);
}

/* ------------------------------------------------------------------------ */
/* Q8_1 activation quantization ([Q8CACHE] "Q8_1 activation cache            */
/* prototype": the exact Q8_1 activation reused by sibling Q4_0 matmuls;     */
/* [TOP1] "Why this was slow": the fused head quantizes the useful rows).    */
/*                                                                           */
/* READING (block layout, GGUF Q8_1): 36 bytes = d (fp16), s (fp16),         */
/* q[32] (int8), blocks row-major by (row, block).                           */
/* READING (arithmetic, binary32 throughout):                                */
/*   amax = max |x_j| over the 32 values;                                    */
/*   d    = amax / 127, one correctly rounded binary32 division;             */
/*   q_j  = x_j / d (binary32 division by the binary32 d), rounded to the     */
/*          nearest integer with halves away from zero;                      */
/*   stored d = fp16(d);  stored s = fp16(d * (float)sum_j q_j);              */
/*   d == 0 (amax zero, or so small that amax/127 underflows) gives all      */
/*   q = 0 and s = 0; q is clamped to [-127, 127], which changes nothing     */
/*   unless amax is subnormal and the rounded d lost precision.              */
/* ------------------------------------------------------------------------ */

static int round_half_away(float t)
{
    double a = floor(fabs((double)t) + 0.5); /* exact in binary64 */
    return (int)(t < 0.0f ? -a : a);
}

void orc_q8_1_quantize(const float *x, int64_t M, int64_t K, uint8_t *out)
{
    const int64_t nb = K / QK;
    for (int64_t m = 0; m < M; ++m) {
        for (int64_t b = 0; b < nb; ++b) {
            const float *xb = x + m * K + b * QK;
            uint8_t *blk = out + (m * nb + b) * Q8_1_BYTES;
            float amax = 0.0f;
            for (int j = 0; j < QK; ++j) {
                float a = fabsf(xb[j]);
                if (a > amax)
                    amax = a;
            }
            float d = amax / 127.0f;
            int sum = 0;
            for (int j = 0; j < QK; ++j) {
                int q = (d == 0.0f) ? 0 : round_half_away(xb[j] / d);
                if (q > 127)
                    q = 127;
                if (q < -127)
                    q = -127;
                blk[4 + j] = (uint8_t)(int8_t)q;
                sum += q;
            }
            float s = d * (float)sum;
            wr16(blk + 0, orc_f32_to_f16(d));
            wr16(blk + 2, orc_f32_to_f16(s));
        }
    }
}

/* Split Q8_1 blocks into their fields (test helper). */
void orc_q8_1_fields(const uint8_t *xq, int64_t nblocks, uint16_t *d, uint16_t *s, int8_t *q)
{
    for (int64_t i = 0; i < nblocks; ++i) {
        const uint8_t *blk = xq + i * Q8_1_BYTES;
        d[i] = rd16(blk);
        s[i] = rd16(blk + 2);
        for (int j = 0; j < QK; ++j)
            q[i * QK + j] = (int8_t)blk[4 + j];
    }
}

/* ------------------------------------------------------------------------ */
/* Q4_0 weights ([CLOSURE] "What materially worked": Q4_0 MMVQ; model file   */
/* Qwen3.6-27B-Q4_0.gguf).                                                   */
/* READING (GGUF Q4_0): 18 bytes = d (fp16) + qs[16]; element j (0..15) is   */
/* the low nibble of qs[j], element j+16 the high nibble; value d*(q - 8).   */
/* Blocks are row-major: row n of the [N][K] weight holds K/32 blocks.       */
/* ------------------------------------------------------------------------ */

void orc_q4_0_decode(const uint8_t *w, int64_t N, int64_t K, uint16_t *d, uint8_t *q)
{
    const int64_t nblk = N * (K / QK);
    for (int64_t i = 0; i < nblk; ++i) {
        const uint8_t *blk = w + i * Q4_0_BYTES;
        d[i] = rd16(blk);
        for (int j = 0; j < 16; ++j) {
            q[i * QK + j] = blk[2 + j] & 0x0F;
            q[i * QK + j + 16] = blk[2 + j] >> 4;
        }
    }
}

void orc_q4_0_encode(const uint16_t *d, const uint8_t *q, int64_t N, int64_t K, uint8_t *w)
{
    const int64_t nblk = N * (K / QK);
    for (int64_t i = 0; i < nblk; ++i) {
        uint8_t *blk = w + i * Q4_0_BYTES;
        wr16(blk, d[i]);
        for (int j = 0; j < 16; ++j)
            blk[2 + j] = (uint8_t)((q[i * QK + j] & 0x0F) | ((q[i * QK + j + 16] & 0x0F) << 4));
    }
}

/* y[m][n] = sum_k W[n][k] * X[m][k] with W and X the dequantized stored
 * values, in binary64.  bound[m][n] = sum over 32-blocks b of |t_b|, where
 * t_b is the block's exact contribution; it scales the parity tolerance.
 * w: Q4_0 [N][K/32]; xq: Q8_1 [M][K/32]; y, bound: [M][N]. */
void orc_q4_0_q8_1_gemv(const uint8_t *w, int64_t N, int64_t K, const uint8_t *xq, int64_t M,
                        double *y, double *bound)
{
    const int64_t nb = K / QK;
#pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < N; ++n) {
        for (int64_t m = 0; m < M; ++m) {
            double acc = 0.0, mag = 0.0;
            for (int64_t b = 0; b < nb; ++b) {
                const uint8_t *wb = w + (n * nb + b) * Q4_0_BYTES;
                const uint8_t *xb = xq + (m * nb + b) * Q8_1_BYTES;
                double dw = (double)orc_f16_to_f32(rd16(wb));
                double dx = (double)orc_f16_to_f32(rd16(xb));
                double tb = 0.0;
                for (int j = 0; j < QK; ++j) {
                    int nib = (j < 16) ? (wb[2 + j] & 0x0F) : (wb[2 + j - 16] >> 4);
                    double wv = dw * (double)(nib - 8);
                    double xv = dx * (double)(int8_t)xb[4 + j];
                    tb += wv * xv;
                }
                acc += tb;
                mag += fabs(tb);
            }
            y[m * N + n] = acc;
            bound[m * N + n] = mag;
        }
    }
}

/* ------------------------------------------------------------------------ */
/* Offline-packed Q4_0 ([CLOSURE] "What materially worked": the verifier's   */
/* width-6 gate/up and down projections ran on offline-packed weights).      */
/*                                                                           */
/* READING (the pages name the packing, not a format): the same 18 bytes per */
/* 32 weights, regrouped.  Requires K % 512 == 0 (nb = K/32 a multiple of    */
/* 16).  Rows form tiles of 16 (the last one ragged): for row n,             */
/* n0 = 16*(n/16), r = n - n0, rows_t = min(16, N - n0).  Two planes:        */
/*   QS, N*nb*16 bytes at 0: element j of block b of row n, with half        */
/*     h = j/16 and jj = j%16, is nibble (jj >= 8 ? high : low) of byte      */
/*       n0*nb*16 + u*(4*rows_t*16) + (g*rows_t + r)*16 + 8*v + (jj % 8)     */
/*     where u = b/4, v = (b%4)/2, g = 2*(b%2) + h;                           */
/*   D, N*nb*2 bytes at N*nb*16: the fp16 scale of block b of row n is       */
/*     element n0*nb + ((b/16)*2 + b%2)*rows_t*8 + r*8 + (b%16)/2.           */
/* The nibble codes are the Q4_0 codes (value d*(q - 8)).                    */
/* ------------------------------------------------------------------------ */

#define Q4P_TILE 16

static int64_t q4p_tile(int64_t n, int64_t N, int64_t *n0, int64_t *r)
{
    *n0 = n / Q4P_TILE * Q4P_TILE;
    *r = n - *n0;
    return (N - *n0 < Q4P_TILE) ? N - *n0 : Q4P_TILE;
}

/* byte of the QS plane holding element j of block b of row n; *hi = nibble */
static int64_t q4p_qs_at(int64_t n, int64_t b, int j, int64_t N, int64_t nb, int *hi)
{
    int64_t n0, r, rows_t = q4p_tile(n, N, &n0, &r);
    const int h = j / 16, jj = j % 16;
    const int64_t u = b / 4, v = (b % 4) / 2, g = 2 * (b % 2) + h;
    *hi = (jj >= 8);
    return n0 * nb * 16 + u * (4 * rows_t * 16) + (g * rows_t + r) * 16 + 8 * v + (jj % 8);
}

/* element of the D plane holding the scale of block b of row n */
static int64_t q4p_d_at(int64_t n, int64_t b, int64_t N, int64_t nb)
{
    int64_t n0, r, rows_t = q4p_tile(n, N, &n0, &r);
    return n0 * nb + ((b / 16) * 2 + b % 2) * rows_t * 8 + r * 8 + (b % 16) / 2;
}

int64_t orc_q4_0_pack_bytes(int64_t N, int64_t K)
{
    return N * (K / QK) * Q4_0_BYTES;
}

void orc_q4_0_pack(const uint8_t *w, int64_t N, int64_t K, uint8_t *wp)
{
    const int64_t nb = K / QK;
    uint8_t *QS = wp;
    uint8_t *D = wp + N * nb * 16;
    memset(wp, 0, (size_t)(N * nb * Q4_0_BYTES));
    for (int64_t n = 0; n < N; ++n)
        for (int64_t b = 0; b < nb; ++b) {
            const uint8_t *wb = w + (n * nb + b) * Q4_0_BYTES;
            for (int j = 0; j < QK; ++j) {
                int nib = (j < 16) ? (wb[2 + j] & 0x0F) : (wb[2 + j - 16] >> 4);
                int hi;
                int64_t at = q4p_qs_at(n, b, j, N, nb, &hi);
                QS[at] |= (uint8_t)(hi ? nib << 4 : nib);
            }
            wr16(D + 2 * q4p_d_at(n, b, N, nb), rd16(wb));
        }
}

void orc_q4_0_unpack(const uint8_t *wp, int64_t N, int64_t K, uint8_t *w)
{
    const int64_t nb = K / QK;
    const uint8_t *QS = wp;
    const uint8_t *D = wp + N * nb * 16;
    for (int64_t n = 0; n < N; ++n)
        for (int64_t b = 0; b < nb; ++b) {
            uint8_t *wb = w + (n * nb + b) * Q4_0_BYTES;
            memset(wb, 0, Q4_0_BYTES);
            wr16(wb, rd16(D + 2 * q4p_d_at(n, b, N, nb)));
            for (int j = 0; j < QK; ++j) {
                int hi;
                int64_t at = q4p_qs_at(n, b, j, N, nb, &hi);
                int nib = hi ? (QS[at] >> 4) : (QS[at] & 0x0F);
                wb[2 + (j % 16)] |= (uint8_t)((j < 16) ? nib : nib << 4);
            }
        }
}

/* The Q4_0 x Q8_1 product of orc_q4_0_q8_1_gemv, reading the packed layout:
 * same dequantized values, same order of summation. */
void orc_q4_0p_q8_1_gemv(const uint8_t *wp, int64_t N, int64_t K, const uint8_t *xq, int64_t M,
                         double *y, double *bound)
{
    const int64_t nb = K / QK;
    const uint8_t *QS = wp;
    const uint8_t *D = wp + N * nb * 16;
#pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < N; ++n) {
        for (int64_t m = 0; m < M; ++m) {
            double acc = 0.0, mag = 0.0;
            for (int64_t b = 0; b < nb; ++b) {
                const uint8_t *xb = xq + (m * nb + b) * Q8_1_BYTES;
                double dw = (double)orc_f16_to_f32(rd16(D + 2 * q4p_d_at(n, b, N, nb)));
                double dx = (double)orc_f16_to_f32(rd16(xb));
                double tb = 0.0;
                for (int j = 0; j < QK; ++j) {
                    int hi;
                    int64_t at = q4p_qs_at(n, b, j, N, nb, &hi);
                    int nib = hi ? (QS[at] >> 4) : (QS[at] & 0x0F);
                    double wv = dw * (double)(nib - 8);
                    double xv = dx * (double)(int8_t)xb[4 + j];
                    tb += wv * xv;
                }
                acc += tb;
                mag += fabs(tb);
            }
            y[m * N + n] = acc;
            bound[m * N + n] = mag;
        }
    }
}

/* ------------------------------------------------------------------------ */
/* Q6_K weights and the expanded pack ([TOP1] "Why this was slow": the       */
/* output tensor is expanded once into signed int8 quants, int8 subscales    */
/* and fp16 superblock scales; "Memory and startup": pack byte count).       */
/*                                                                           */
/* READING (GGUF Q6_K, 210 bytes per 256 values): ql[128], qh[64],           */
/* scales[16] (int8, one per 16 values), d (fp16).  Each half h (128         */
/* values) uses ql[64h..64h+63] and qh[32h..32h+31].  For l in 0..31 the     */
/* 6-bit code u of value 128h + l + 32c (c = 0..3) takes its low 4 bits from */
/* ql[64h + l + 32(c&1)] (low nibble for c < 2, high nibble for c >= 2) and  */
/* its high 2 bits from bits 2c..2c+1 of qh[32h + l].  Value =               */
/* d * scales[e/16] * (u - 32) for element e.                                */
/*                                                                           */
/* READING (pack layout; the pages give only "exact expected layout and byte */
/* count" and the total).  Three planes, each split into tiles of 64         */
/* consecutive rows (the last tile holds the N % 64 remaining rows, if any); */
/* for row n, t = n / 64, n0 = 64 t, rows_t = min(64, N - n0), r = n - n0:   */
/*   Q  int8, plane at 0:            quant k of row n at                      */
/*        n0*K + ((k/16)*rows_t + r)*16 + k%16                                */
/*      (a tile stores the 16-value piece c of all its rows, row after row,  */
/*      then piece c + 1, ...);                                              */
/*   SC int8, plane at N*K:          subscale j (= k/16) of row n at          */
/*        n0*(K/16) + ((j/16)*rows_t + r)*16 + j%16                           */
/*      (per superblock s, the 16 subscales of every row of the tile);       */
/*   D  fp16, plane at N*K + N*K/16: scale of superblock s of row n at        */
/*        element n0*(K/256) + s*rows_t + r.                                  */
/* The size is N*K + N*K/16 + 2*N*K/256 bytes.                               */
/* ------------------------------------------------------------------------ */

#define PACK_TILE 64

static int64_t tile_rows(int64_t n, int64_t N, int64_t *n0, int64_t *r)
{
    *n0 = n / PACK_TILE * PACK_TILE;
    *r = n - *n0;
    return (N - *n0 < PACK_TILE) ? N - *n0 : PACK_TILE;
}

/* byte offset of quant (n, k) in the Q plane */
static int64_t pack_q_at(int64_t n, int64_t k, int64_t N, int64_t K)
{
    int64_t n0, r, rows_t = tile_rows(n, N, &n0, &r);
    return n0 * K + ((k / 16) * rows_t + r) * 16 + k % 16;
}

/* byte offset of subscale (n, j) in the SC plane, j = k / 16 */
static int64_t pack_sc_at(int64_t n, int64_t j, int64_t N, int64_t K)
{
    int64_t n0, r, rows_t = tile_rows(n, N, &n0, &r);
    return n0 * (K / 16) + ((j / 16) * rows_t + r) * 16 + j % 16;
}

/* element index of superblock scale (n, s) in the D plane */
static int64_t pack_d_at(int64_t n, int64_t s, int64_t N, int64_t K)
{
    int64_t n0, r, rows_t = tile_rows(n, N, &n0, &r);
    return n0 * (K / QK_K) + s * rows_t + r;
}

void orc_q6k_decode(const uint8_t *raw, int64_t N, int64_t K, int8_t *q, int8_t *sc, uint16_t *d)
{
    const int64_t nsb = N * (K / QK_K);
    for (int64_t i = 0; i < nsb; ++i) {
        const uint8_t *blk = raw + i * Q6_K_BYTES;
        const uint8_t *ql = blk, *qh = blk + 128;
        const int8_t *scales = (const int8_t *)(blk + 192);
        for (int h = 0; h < 2; ++h)
            for (int l = 0; l < 32; ++l)
                for (int c = 0; c < 4; ++c) {
                    uint8_t lo_byte = ql[64 * h + l + 32 * (c & 1)];
                    int lo = (c < 2) ? (lo_byte & 0x0F) : (lo_byte >> 4);
                    int hi = (qh[32 * h + l] >> (2 * c)) & 3;
                    q[i * QK_K + 128 * h + l + 32 * c] = (int8_t)((lo | (hi << 4)) - 32);
                }
        for (int j = 0; j < 16; ++j)
            sc[i * 16 + j] = scales[j];
        d[i] = rd16(blk + 208);
    }
}

void orc_q6k_encode(const int8_t *q, const int8_t *sc, const uint16_t *d, int64_t N, int64_t K,
                    uint8_t *raw)
{
    const int64_t nsb = N * (K / QK_K);
    for (int64_t i = 0; i < nsb; ++i) {
        uint8_t *blk = raw + i * Q6_K_BYTES;
        memset(blk, 0, 192);
        for (int h = 0; h < 2; ++h)
            for (int l = 0; l < 32; ++l)
                for (int c = 0; c < 4; ++c) {
                    int u = q[i * QK_K + 128 * h + l + 32 * c] + 32; /* 0..63 */
                    uint8_t *lo_byte = &blk[64 * h + l + 32 * (c & 1)];
                    *lo_byte |= (uint8_t)((c < 2) ? (u & 0x0F) : ((u & 0x0F) << 4));
                    blk[128 + 32 * h + l] |= (uint8_t)(((u >> 4) & 3) << (2 * c));
                }
        for (int j = 0; j < 16; ++j)
            blk[192 + j] = (uint8_t)sc[i * 16 + j];
        wr16(blk + 208, d[i]);
    }
}

int64_t orc_q6k_pack_bytes(int64_t N, int64_t K)
{
    return N * K + N * (K / 16) + 2 * N * (K / QK_K);
}

void orc_q6k_pack_expand(const uint8_t *raw, int64_t N, int64_t K, uint8_t *pack)
{
    int8_t *Q = (int8_t *)pack;
    int8_t *SC = (int8_t *)(pack + N * K);
    uint8_t *D = pack + N * K + N * (K / 16);
    const int64_t ns = K / QK_K;
#pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < N; ++n) {
        for (int64_t s = 0; s < ns; ++s) {
            int8_t q[QK_K], sc[16];
            uint16_t dbits;
            orc_q6k_decode(raw + (n * ns + s) * Q6_K_BYTES, 1, QK_K, q, sc, &dbits);
            for (int e = 0; e < QK_K; ++e)
                Q[pack_q_at(n, s * QK_K + e, N, K)] = q[e];
            for (int j = 0; j < 16; ++j)
                SC[pack_sc_at(n, s * 16 + j, N, K)] = sc[j];
            wr16(D + 2 * pack_d_at(n, s, N, K), dbits);
        }
    }
}

/* logits[r][n] = sum_k Wq6[n][k] * X[r][k] over the pack's dequantized
 * values d * sc * q and the Q8_1 rows' values d_x * q_x, in binary64.
 * bound[r][n] = sum over 32-blocks of |block contribution|.
 * pack: expanded Q6_K of an [N][K] weight (layout above); xq: Q8_1
 * [rows][K/32]; logits, bound: [rows][N]. */
void orc_q6k_pack_logits(const uint8_t *pack, int64_t N, int64_t K, const uint8_t *xq,
                         int64_t rows, double *logits, double *bound)
{
    const int8_t *Q = (const int8_t *)pack;
    const int8_t *SC = (const int8_t *)(pack + N * K);
    const uint8_t *D = pack + N * K + N * (K / 16);
    const int64_t nb = K / QK;
#pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < N; ++n) {
        for (int64_t r = 0; r < rows; ++r) {
            double acc = 0.0, mag = 0.0;
            for (int64_t b = 0; b < nb; ++b) {
                const uint8_t *xb = xq + (r * nb + b) * Q8_1_BYTES;
                const int64_t k0 = b * QK;
                double dx = (double)orc_f16_to_f32(rd16(xb));
                double dw = (double)orc_f16_to_f32(rd16(D + 2 * pack_d_at(n, k0 / QK_K, N, K)));
                double tb = 0.0;
                for (int j = 0; j < QK; ++j) {
                    int64_t k = k0 + j;
                    double wv = dw * (double)SC[pack_sc_at(n, k / 16, N, K)] *
                                (double)Q[pack_q_at(n, k, N, K)];
                    double xv = dx * (double)(int8_t)xb[4 + j];
                    tb += wv * xv;
                }
                acc += tb;
                mag += fabs(tb);
            }
            logits[r * N + n] = acc;
            bound[r * N + n] = mag;
        }
    }
}

/* ------------------------------------------------------------------------ */
/* Compact Q6_K pack: the raw Q6_K bits themselves, re-tiled ([TOP1]         */
/* "Memory and startup": the expanded pack is kept beside the raw Q6_K       */
/* weights at 1,360,793,600 bytes; "Transfer to DeepSeek and future lanes":  */
/* persistent packs are ranked by time saved per GiB).  READING -- this      */
/* layout is the library's, not the pages': the 210 bytes of every           */
/* superblock, in four planes, each in the 64-row tiles of the expanded      */
/* pack (n0, r, rows_t as there):                                            */
/*   QL plane at 0:         raw byte i (0..127) of superblock s of row n at  */
/*        n0*(K/2) + ((8*s + i/16)*rows_t + r)*16 + i%16                     */
/*   QH plane at N*K/2:     raw byte 128 + i (i = 0..63) at                  */
/*        n0*(K/4) + ((4*s + i/16)*rows_t + r)*16 + i%16                     */
/*   SC plane at N*K*3/4:   raw byte 192 + i (subscale j = 16*s + i) at the  */
/*        expanded pack's SC position of (n, j)                              */
/*   D  plane at N*K*13/16: raw bytes 208..209 at the expanded D position.   */
/* Size 210 * N * K/256 bytes, the raw size.  The weights it encodes are     */
/* those of the raw superblocks (orc_q6k_decode).                            */
/* ------------------------------------------------------------------------ */

int64_t orc_q6k_compact_bytes(int64_t N, int64_t K) { return Q6_K_BYTES * N * (K / QK_K); }

/* byte offsets, within the whole pack, of raw byte `i` of superblock s of row n */
static int64_t cpk_ql_at(int64_t n, int64_t s, int64_t i, int64_t N, int64_t K)
{
    int64_t n0, r, rows_t = tile_rows(n, N, &n0, &r);
    return n0 * (K / 2) + ((8 * s + i / 16) * rows_t + r) * 16 + i % 16;
}

static int64_t cpk_qh_at(int64_t n, int64_t s, int64_t i, int64_t N, int64_t K)
{
    int64_t n0, r, rows_t = tile_rows(n, N, &n0, &r);
    return N * (K / 2) + n0 * (K / 4) + ((4 * s + i / 16) * rows_t + r) * 16 + i % 16;
}

static int64_t cpk_sc_at(int64_t n, int64_t s, int64_t i, int64_t N, int64_t K)
{
    return N * (K / 2) + N * (K / 4) + pack_sc_at(n, 16 * s + i, N, K);
}

static int64_t cpk_d_at(int64_t n, int64_t s, int64_t N, int64_t K)
{
    return N * (K / 2) + N * (K / 4) + N * (K / 16) + 2 * pack_d_at(n, s, N, K);
}

void orc_q6k_pack_compact(const uint8_t *raw, int64_t N, int64_t K, uint8_t *pack)
{
    const int64_t ns = K / QK_K;
    for (int64_t n = 0; n < N; ++n)
        for (int64_t s = 0; s < ns; ++s) {
            const uint8_t *blk = raw + (n * ns + s) * Q6_K_BYTES;
            for (int i = 0; i < 128; ++i)
                pack[cpk_ql_at(n, s, i, N, K)] = blk[i];
            for (int i = 0; i < 64; ++i)
                pack[cpk_qh_at(n, s, i, N, K)] = blk[128 + i];
            for (int i = 0; i < 16; ++i)
                pack[cpk_sc_at(n, s, i, N, K)] = blk[192 + i];
            pack[cpk_d_at(n, s, N, K)] = blk[208];
            pack[cpk_d_at(n, s, N, K) + 1] = blk[209];
        }
}

void orc_q6k_compact_unpack(const uint8_t *pack, int64_t N, int64_t K, uint8_t *raw)
{
    const int64_t ns = K / QK_K;
    for (int64_t n = 0; n < N; ++n)
        for (int64_t s = 0; s < ns; ++s) {
            uint8_t *blk = raw + (n * ns + s) * Q6_K_BYTES;
            for (int i = 0; i < 128; ++i)
                blk[i] = pack[cpk_ql_at(n, s, i, N, K)];
            for (int i = 0; i < 64; ++i)
                blk[128 + i] = pack[cpk_qh_at(n, s, i, N, K)];
            for (int i = 0; i < 16; ++i)
                blk[192 + i] = pack[cpk_sc_at(n, s, i, N, K)];
            blk[208] = pack[cpk_d_at(n, s, N, K)];
            blk[209] = pack[cpk_d_at(n, s, N, K) + 1];
        }
}

/* ------------------------------------------------------------------------ */
/* Greedy top-1 with the lowest-token-ID tie rule ([TOP1] "Exactness and     */
/* safety contracts": generic argmax and the fused reducer share one         */
/* lowest-ID finite-tie contract).  Scan ids ascending and replace the best  */
/* only on a strictly greater value, so among equal maxima the lowest id     */
/* wins; -0 and +0 compare equal.  NaN is never selected.                    */
/* ------------------------------------------------------------------------ */

void orc_top1(const double *logits, int64_t rows, int64_t N, int32_t *ids)
{
    for (int64_t r = 0; r < rows; ++r) {
        int64_t best = -1;
        double bv = 0.0;
        for (int64_t n = 0; n < N; ++n) {
            double v = logits[r * N + n];
            if (isnan(v))
                continue;
            if (best < 0 || v > bv) {
                best = n;
                bv = v;
            }
        }
        ids[r] = (int32_t)best;
    }
}

/* The fused LM-head boundary ([TOP1] "Outcome", "Why this was slow"): of an
 * [M][K] f32 activation, quantize rows row0..row0+rows-1 to Q8_1, project
 * them through the expanded Q6_K pack and reduce each to its greedy id.
 * logits/bound (each [rows][N]) are caller buffers kept for the comparator;
 * xq_out ([rows][K/32] Q8_1) likewise. */
void orc_q6k_lmhead_top1(const uint8_t *pack, int64_t N, int64_t K, const float *x, int64_t M,
                         int64_t row0, int64_t rows, uint8_t *xq_out, double *logits, double *bound,
                         int32_t *ids)
{
    (void)M;
    orc_q8_1_quantize(x + row0 * K, rows, K, xq_out);
    orc_q6k_pack_logits(pack, N, K, xq_out, rows, logits, bound);
    orc_top1(logits, rows, N, ids);
}

/* ------------------------------------------------------------------------ */
/* Verifier-layer stages between projections (a width-6 FFN block: gate and  */
/* up share one Q8_1 activation, down consumes SiLU(gate)*up requantized;    */
/* [CLOSURE] "What materially worked": width-6 gate/up and down projections; */
/* "Closed or negative paths": the down-to-next-RMS/Q8 boundary).            */
/* READING: h = SiLU(g) * u = g / (1 + exp(-g)) * u; the next layer's input  */
/* is the row RMS normalization x = y / sqrt(mean_k y^2 + eps) (no weight).  */
/* Both in binary64 from binary32 inputs.                                    */
/* ------------------------------------------------------------------------ */

void orc_silu_mul(const float *g, const float *u, int64_t n, double *h)
{
    for (int64_t i = 0; i < n; ++i) {
        double gv = (double)g[i];
        h[i] = gv / (1.0 + exp(-gv)) * (double)u[i];
    }
}

void orc_rms_norm(const float *y, int64_t M, int64_t K, double eps, double *out)
{
    for (int64_t m = 0; m < M; ++m) {
        double ss = 0.0;
        for (int64_t k = 0; k < K; ++k)
            ss += (double)y[m * K + k] * (double)y[m * K + k];
        double inv = 1.0 / sqrt(ss / (double)K + eps);
        for (int64_t k = 0; k < K; ++k)
            out[m * K + k] = (double)y[m * K + k] * inv;
    }
}

int orc_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Threads for the loops over output rows; each row's sum stays in one
 * thread in its fixed order, so results do not depend on it. */
void orc_set_num_threads(int n)
{
#ifdef _OPENMP
    if (n >= 1)
        omp_set_num_threads(n);
#else
    (void)n;
#endif
}
