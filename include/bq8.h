/*
 * bq8.h -- C ABI of libbq8: block-quantized GEMV kernels for AMD Instinct
 * MI355X (gfx950, CDNA4).
 *
 * The hot path is the width-6 speculative verifier projection and the fused
 * draft LM head of two web pages:
 *   "Qwen3.6 27B Q4_0 DFlash/SYCL closure" -- Q4_0 x Q8_1 MMVQ with direct
 *     coverage of every row count 1..17 ("What materially worked"), width-6
 *     gate/up and down projections, the down-to-next-RMS/Q8 boundary
 *     ("Closed or negative paths");
 *   "Q6_K M=6 fused DFlash top-1 production record" -- the Q6_K output
 *     weight expanded once to int8 quants + int8 subscales + fp16 superblock
 *     scales, a kernel that quantizes the useful activation rows, reuses each
 *     weight slice across all of them and reduces each row to its greedy
 *     token id without writing logits ("Why this was slow"), with the
 *     lowest-token-ID finite-tie contract ("Exactness and safety contracts");
 *   "Qwen3.6 27B B70 follow-up: Q8 activation cache, FP8 artifacts, MTP
 *     blocker" -- one exact Q8_1 activation reused by sibling Q4_0 matmuls
 *     ("Q8_1 activation cache prototype").
 *
 * Conventions for every entry point:
 *   - Pointers are DEVICE pointers unless the comment says otherwise.  The
 *     caller allocates and owns every buffer; the library allocates nothing.
 *     Between calls it keeps only device properties, cached per device, and
 *     the allocation-free head's own scratch array (q6k_lmhead_top1_noalloc).
 *     Any host thread may call, with any device current: the call runs on
 *     the current device.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *     Calls only enqueue work; results are valid once the stream reaches
 *     them.  Nothing synchronizes inside the library.
 *   - Arguments are validated on the host BEFORE anything is enqueued.  On a
 *     validation failure the call returns a nonzero status and no output
 *     byte is touched.  BQ8_ERR_HIP reports a failed launch.
 *   - fp16 fields are raw IEEE binary16 bits, little-endian.
 *   - Calls on one stream are ordered; concurrent calls on different
 *     streams must not share output or scratch buffers.
 *
 * Formats (block layouts follow the public GGUF formats the pages' .gguf
 * model files use):
 *   Q8_1  32 activations in 36 bytes: d (fp16), s (fp16), q[32] (int8);
 *         d = max|x|/127, q = x/d rounded half away from zero, s = d*sum(q).
 *   Q4_0  32 weights in 18 bytes: d (fp16), qs[16]; element j < 16 is the
 *         low nibble of qs[j], element j+16 the high nibble; value d*(q-8).
 *   Q6_K  256 weights in 210 bytes: ql[128], qh[64], scales[16] (int8),
 *         d (fp16); value d * scales[e/16] * (u - 32) for a 6-bit code u.
 *   Expanded Q6_K pack: three planes -- Q int8 quants at 0, SC int8
 *         subscales (one per 16 values) at N*K, D fp16 superblock scales at
 *         N*K + N*K/16 (total q6k_pack_bytes(N, K)) -- each split into tiles
 *         of 64 consecutive rows (the last tile holds the remaining N % 64
 *         rows).  For row n: n0 = 64*(n/64), r = n - n0, rows_t =
 *         min(64, N - n0).
 *           quant k      at byte    n0*K + ((k/16)*rows_t + r)*16 + k%16
 *           subscale j   at byte    N*K + n0*(K/16) + ((j/16)*rows_t + r)*16 + j%16
 *           scale s      at element (N*K + N*K/16)/2 + n0*(K/256) + s*rows_t + r
 *         i.e. a tile stores 16-value piece c of all its rows, row after
 *         row, then piece c + 1: lane r of a wave reads its row's piece c
 *         while the wave reads one contiguous kilobyte.
 */
#ifndef BQ8_H
#define BQ8_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define BQ8_ABI_VERSION 1

typedef int32_t bq8_status;
enum {
    BQ8_OK = 0,
    BQ8_ERR_NULL = 1,  /* a required pointer is NULL                         */
    BQ8_ERR_SHAPE = 2, /* a size is out of range or not a block multiple     */
    BQ8_ERR_ALIGN = 3, /* a pointer is not aligned as documented             */
    BQ8_ERR_SIZE = 4,  /* a byte count (pack, scratch) is not what is needed */
    BQ8_ERR_HIP = 5    /* the HIP runtime reported a launch error            */
};

/* Host.  Static, never-freed description of a status code. */
const char *bq8_status_string(bq8_status status);

/* Host.  BQ8_ABI_VERSION of the built library. */
int32_t bq8_abi_version(void);

/* ------------------------------------------------------------------------
 * Q8_1 activation quantization.
 * x:  f32 [M][K] row-major, 4-byte aligned.
 * xq: Q8_1 [M][K/32] blocks of 36 bytes, row-major by (row, block),
 *     4-byte aligned; fully overwritten.  One quantized activation may feed
 *     any number of sibling q4_0_mmvq_* calls (the Q8_1 activation cache of
 *     the follow-up page, made explicit).
 * Shape: M >= 1, K >= 32, K % 32 == 0, M*K < 2^31.
 * Subnormal amax: d = amax/127 may round to 0 (then the block is all zero)
 * or lose precision (quants are clamped to +-127).  NaN/Inf inputs are
 * outside the contract.
 * ---------------------------------------------------------------------- */
bq8_status q8_1_quantize(const float *x, int64_t M, int64_t K, void *xq, void *stream);

/* ------------------------------------------------------------------------
 * Q4_0 x Q8_1 matrix-vector products at M activation rows, one entry point
 * per M = 1..17 (the closure page's direct MMVQ coverage through rows 9-17:
 * no row count falls back to re-reading the weight once per row).
 *   y[m][n] = sum_k W[n][k] * X[m][k]
 * with W the dequantized Q4_0 weight and X the dequantized Q8_1 rows.
 * w:  Q4_0 [N][K/32] blocks of 18 bytes, row-major, 16-byte aligned.
 * xq: Q8_1 [M][K/32] (from q8_1_quantize), 16-byte aligned (the kernels
 *     copy it into LDS in 16-byte pieces).
 * y:  f32 [M][N] row-major, 4-byte aligned; fully overwritten.
 * Shape: 1 <= N < 2^31, 32 <= K <= 2^26, K % 32 == 0, N*K/32*18 < 2^40.
 * Each weight byte is read from memory once per call whatever M is.
 * Accumulation is binary32 over exact per-block integer dots, in a fixed
 * order: results are bitwise reproducible run to run, and equal weight rows
 * give bitwise equal outputs.
 * ---------------------------------------------------------------------- */
bq8_status q4_0_mmvq_m1(const void *w, int64_t N, int64_t K, const void *xq, float *y, void *stream);
bq8_status q4_0_mmvq_m2(const void *w, int64_t N, int64_t K, const void *xq, float *y, void *stream);
bq8_status q4_0_mmvq_m3(const void *w, int64_t N, int64_t K, const void *xq, float *y, void *stream);
bq8_status q4_0_mmvq_m4(const void *w, int64_t N, int64_t K, const void *xq, float *y, void *stream);
bq8_status q4_0_mmvq_m5(const void *w, int64_t N, int64_t K, const void *xq, float *y, void *stream);
bq8_status q4_0_mmvq_m6(const void *w, int64_t N, int64_t K, const void *xq, float *y, void *stream);
bq8_status q4_0_mmvq_m7(const void *w, int64_t N, int64_t K, const void *xq, float *y, void *stream);
bq8_status q4_0_mmvq_m8(const void *w, int64_t N, int64_t K, const void *xq, float *y, void *stream);
bq8_status q4_0_mmvq_m9(const void *w, int64_t N, int64_t K, const void *xq, float *y, void *stream);
bq8_status q4_0_mmvq_m10(const void *w, int64_t N, int64_t K, const void *xq, float *y, void *stream);
bq8_status q4_0_mmvq_m11(const void *w, int64_t N, int64_t K, const void *xq, float *y, void *stream);
bq8_status q4_0_mmvq_m12(const void *w, int64_t N, int64_t K, const void *xq, float *y, void *stream);
bq8_status q4_0_mmvq_m13(const void *w, int64_t N, int64_t K, const void *xq, float *y, void *stream);
bq8_status q4_0_mmvq_m14(const void *w, int64_t N, int64_t K, const void *xq, float *y, void *stream);
bq8_status q4_0_mmvq_m15(const void *w, int64_t N, int64_t K, const void *xq, float *y, void *stream);
bq8_status q4_0_mmvq_m16(const void *w, int64_t N, int64_t K, const void *xq, float *y, void *stream);
bq8_status q4_0_mmvq_m17(const void *w, int64_t N, int64_t K, const void *xq, float *y, void *stream);

/* Same as q4_0_mmvq_m<M> with M (1..17) as an argument. */
bq8_status q4_0_mmvq(const void *w, int64_t N, int64_t K, const void *xq, int64_t M, float *y,
                     void *stream);

/* ------------------------------------------------------------------------
 * Offline-packed Q4_0 (the closure page's width-6 gate/up and down
 * projections ran on offline-packed weights, "What materially worked").  The
 * pack holds the same 18 bytes per 32 weights, regrouped so that the MFMA
 * kernel's weight operand is one contiguous kilobyte per wave load.
 * Requires K % 512 == 0.  For row n: n0 = 16*(n/16), r = n - n0,
 * rows_t = min(16, N - n0), nb = K/32.
 *   QS plane (N*nb*16 bytes at 0): element j of block b of row n, with
 *     h = j/16, jj = j%16, is nibble (jj >= 8 ? high : low) of byte
 *       n0*nb*16 + u*(4*rows_t*16) + (g*rows_t + r)*16 + 8*v + jj%8,
 *     u = b/4, v = (b%4)/2, g = 2*(b%2) + h; nibble values are the Q4_0
 *     codes q (value d*(q - 8)).
 *   D plane (N*nb*2 bytes at N*nb*16): the fp16 scale of block b of row n
 *     is element n0*nb + ((b/16)*2 + b%2)*rows_t*8 + r*8 + (b%16)/2.
 * q4_0_pack_bytes: host; N*K/32*18, or -1 if the shape is invalid.
 * q4_0_pack: w Q4_0 [N][K/32] (2-byte aligned) -> wp (16-byte aligned,
 *   wp_bytes == q4_0_pack_bytes(N, K), fully overwritten).  Run once, at
 *   load time.
 * q4_0_mmvq_packed: y[m][n] = sum_k W[n][k] X[m][k] as q4_0_mmvq_m<M>, for
 *   M = 1..17, from the packed weight; xq, y as there.  Results equal the
 *   standard-layout entry points up to the binary32 summation order, which
 *   is fixed: results are reproducible bit for bit, and equal weight rows
 *   give bitwise equal outputs.
 * q4_0_mmvq_packed_ws: the same product, launched so that every CU gets the
 *   same work where that pays (M >= 9; for M <= 8 it is q4_0_mmvq_packed,
 *   bit for bit): each 16-row tile past the largest
 *   multiple of the CU count is cut into P = min(4, K/256) ranges of K
 *   (range p = chunks
 *   floor(p*C/P) .. floor((p+1)*C/P) - 1 of the C = K/256 chunks of 8
 *   blocks), computed by separate workgroups whose range sums meet in the
 *   workspace and are added in range order.  From M = 11, when N % 32 == 0
 *   and there are fewer 32-row pairs of tiles than CUs, every pair is cut
 *   instead, into P = q4_0_mmvq_packed_splits_rows(N, K, M) ranges (when
 *   that count is at least 2 and gives a workgroup per CU).  Outputs of cut
 *   tiles equal q4_0_mmvq_packed's up to the binary32 summation order, the
 *   others bit for bit; results are reproducible bit for bit.
 *   ws: device memory, 256-byte aligned, ws_bytes >= q4_0_mmvq_packed_ws_bytes();
 *   caller-owned.  Zero-fill it once before its first use: every call that
 *   completes leaves it ready for the next (its counters back at zero).
 *   Calls that overlap in time (e.g. on different streams) must not share
 *   a workspace.  ws NULL -> BQ8_ERR_NULL, ws_bytes too small ->
 *   BQ8_ERR_SIZE, ws misaligned -> BQ8_ERR_ALIGN.
 * q4_0_mmvq_packed_ws_bytes: host; the workspace q4_0_mmvq_packed_ws and
 *   q4_0_gate_up_silu_q8_1_packed_ws need on the current device (about
 *   24 KB per CU), or -1 without a device.  One workspace serves both.
 * q4_0_mmvq_packed_split: the same product with K cut into nsplit ranges of
 *   8-block chunks (range p = chunks floor(p*C/nsplit) .. floor((p+1)*C/
 *   nsplit) - 1 of the C = K/256 chunks), each computed by its own
 *   workgroups, so that a shape with few 16-row tiles still fills every CU.
 *   ypart: f32 [nsplit][M][N], 4-byte aligned; ypart[p] holds range p's
 *   sums, and y = ypart[0] + ypart[1] + ... in that order (binary32; see
 *   rms_norm_q8_1_sum).  nsplit = 1 gives q4_0_mmvq_packed's bits.
 *   1 <= nsplit <= 8, nsplit <= K/256.
 * q4_0_mmvq_packed_splits: host; the nsplit the packed stream uses for an
 *   [N][K] projection (enough ranges for at least 1024 workgroups, at most
 *   8), or -1 if the shape is invalid.  1 for [17408 x 5120], 4 for
 *   [5120 x 17408].
 * q4_0_mmvq_packed_splits_rows: host; the nsplit for a split launch of M
 *   rows on the current device.  M <= 10: q4_0_mmvq_packed_splits(N, K).
 *   M >= 11 (two 16-row tiles per workgroup when N % 32 == 0): of the
 *   counts 2..8, at most K/256, whose workgroups are all resident at once
 *   by the runtime's occupancy figure, the one that spreads them most
 *   evenly over the CUs (least ratio of the busiest CU's workgroups to the
 *   mean; the smaller count on a tie), else q4_0_mmvq_packed_splits(N, K).
 *   3 for [5120 x 17408] at M = 11..17 on MI355X.  -1 for an invalid shape
 *   or M, or when M >= 11 and no device can be queried.
 * Shape: 1 <= N < 2^31, 512 <= K <= 2^26, K % 512 == 0.
 * ---------------------------------------------------------------------- */
int64_t q4_0_pack_bytes(int64_t N, int64_t K);
bq8_status q4_0_pack(const void *w, int64_t N, int64_t K, void *wp, int64_t wp_bytes,
                     void *stream);
bq8_status q4_0_mmvq_packed(const void *wp, int64_t N, int64_t K, const void *xq, int64_t M,
                            float *y, void *stream);
bq8_status q4_0_mmvq_packed_ws(const void *wp, int64_t N, int64_t K, const void *xq, int64_t M,
                               float *y, void *ws, int64_t ws_bytes, void *stream);
int64_t q4_0_mmvq_packed_ws_bytes(void);
bq8_status q4_0_mmvq_packed_split(const void *wp, int64_t N, int64_t K, const void *xq,
                                  int64_t M, int64_t nsplit, float *ypart, void *stream);
int64_t q4_0_mmvq_packed_splits(int64_t N, int64_t K);
int64_t q4_0_mmvq_packed_splits_rows(int64_t N, int64_t K, int64_t M);

/* ------------------------------------------------------------------------
 * Joint gate/up projection with SiLU(gate)*up and its Q8_1 requantization
 * as the epilogue (the fused-head page's run identity has joint gate/up
 * enabled over its packed width-6 projections, "Strict run identity"; the
 * closure page's packed gate/up projections, "What materially worked").
 * One launch:
 *   g = W_gate X,  u = W_up X               (as q4_0_mmvq_packed)
 *   h = g / (1 + exp(-g)) * u               (binary32, as silu_mul_q8_1)
 *   hq = Q8_1(h)                            (as silu_mul_q8_1)
 * wg, wu: q4_0_pack of the gate and up weights, each Q4_0 [N][K]; 16-byte
 *   aligned.  xq: Q8_1 [M][K/32], 16-byte aligned.  hq: Q8_1 [M][N/32],
 *   4-byte aligned, fully overwritten.  g, u, h: optional f32 [M][N]
 *   (NULL to skip), receive the gate and up products and h; hq does not
 *   depend on whether they are given.  hq is bitwise the Q8_1 of the h
 *   computed here; g and u equal q4_0_mmvq_packed's up to the binary32
 *   summation order.
 * q4_0_gate_up_silu_q8_1_packed_ws: the same launch balanced over the CUs
 *   when N/32 is at least the CU count (else it is the plain launch, bit for
 *   bit): each 32-column group past the largest multiple of the CU count is cut
 *   into P = min(4, K/256) ranges of K computed by separate workgroups,
 *   whose range sums meet in the workspace (as q4_0_mmvq_packed_ws) and are
 *   added in range order before the epilogue.  For those groups g and u
 *   equal q4_0_gate_up_silu_q8_1_packed's up to the binary32 summation
 *   order, the others bit for bit; hq is the Q8_1 of the h computed here.
 *   ws, ws_bytes and their errors as q4_0_mmvq_packed_ws.
 * Shape: M = 1..17, N % 32 == 0, 32 <= N < 2^31, K as q4_0_mmvq_packed,
 *   M*K < 2^31, M*N < 2^31.
 * ---------------------------------------------------------------------- */
bq8_status q4_0_gate_up_silu_q8_1_packed(const void *wg, const void *wu, int64_t N, int64_t K,
                                         const void *xq, int64_t M, float *g, float *u, float *h,
                                         void *hq, void *stream);
bq8_status q4_0_gate_up_silu_q8_1_packed_ws(const void *wg, const void *wu, int64_t N,
                                            int64_t K, const void *xq, int64_t M, float *g,
                                            float *u, float *h, void *hq, void *ws,
                                            int64_t ws_bytes, void *stream);

/* ------------------------------------------------------------------------
 * Q6_K expansion (run once, at load time).  The fused-head page expands the
 * output tensor once into signed int8 quants, int8 subscales and fp16
 * superblock scales ("Why this was slow") and accepts the pack only with its
 * exact layout and size ("Exactness and safety contracts").
 * q6k_pack_bytes: host; N*K + N*K/16 + 2*N*K/256, or -1 if the shape is
 * invalid.  [248320 x 5120] gives 1,360,793,600 ("Memory and startup").
 * raw:  Q6_K [N][K/256] superblocks of 210 bytes, row-major, 2-byte aligned.
 * pack: expanded pack (layout above), 16-byte aligned, pack_bytes bytes,
 *       fully overwritten.
 * Shape: 1 <= N < 2^31, K >= 256, K % 256 == 0.
 * pack_bytes != q6k_pack_bytes(N, K) -> BQ8_ERR_SIZE.
 * ---------------------------------------------------------------------- */
int64_t q6k_pack_bytes(int64_t N, int64_t K);
bq8_status q6k_pack_expand(const void *raw, int64_t N, int64_t K, void *pack, int64_t pack_bytes,
                           void *stream);

/* ------------------------------------------------------------------------
 * Fused Q6_K LM-head projection + greedy top-1 ("Q6_K M=6 fused DFlash
 * top-1 production record": only decoder rows 1..5 of the six-row block are
 * projected, each weight slice is reused across all of them, and each row is
 * reduced on the device to the lowest token id among its maximal logits;
 * logits are never written to memory).
 * pack:    expanded Q6_K pack of an [N][K] weight (q6k_pack_expand).
 * x:       f32 [M][K] row-major activations, 4-byte aligned.
 * row0, rows: project rows row0 .. row0+rows-1 of x (the hot path uses
 *          M = 6, row0 = 1, rows = 5); 1 <= rows <= 8, row0 + rows <= M.
 * ids:     int32 [rows]; ids[r] is the greedy token id of row row0 + r.
 * scratch: device workspace of at least q6k_lmhead_top1_scratch_bytes(N, K,
 *          rows) bytes, 16-byte aligned (quantized rows, their 16-value
 *          sums and one key per workgroup and row); its contents on entry do
 *          not matter.  Three
 *          kernels run in stream order: quantize, fused projection + per-
 *          workgroup reduction, final reduction.  Below 3600 64-row tiles
 *          (N < 230337) each tile's K is cut into ranges computed by the
 *          waves of one workgroup and added in range order, so that narrow
 *          vocabularies (a 31040-row shard) still fill the CUs.
 * Shape: 1 <= N < 2^31 - 1, K >= 256, K % 256 == 0, N*K < 2^40.
 * Tie rule: among equal maximal logits the lowest id wins; -0 equals +0.
 * Equal weight rows give bitwise equal logits, so planted duplicate rows
 * always resolve to the lower id.
 * q6k_lmhead_top1_scratch_bytes: host; -1 if the shape is invalid.
 * ---------------------------------------------------------------------- */
int64_t q6k_lmhead_top1_scratch_bytes(int64_t N, int64_t K, int64_t rows);
bq8_status q6k_lmhead_top1(const void *pack, int64_t N, int64_t K, const float *x, int64_t M,
                           int64_t row0, int64_t rows, int32_t *ids, void *scratch,
                           int64_t scratch_bytes, void *stream);

/* ------------------------------------------------------------------------
 * q6k_lmhead_top1 without a scratch argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid allocation).  The call allocates nothing: its
 * scratch is a device array inside the library, one per GPU, of
 * BQ8_TOP1_NOALLOC_SCRATCH_BYTES (256 KiB), held by each GPU the library runs
 * on until the process ends.  Arguments, results and errors are those of
 * q6k_lmhead_top1, plus:
 *   q6k_lmhead_top1_scratch_bytes(N, K, rows) > BQ8_TOP1_NOALLOC_SCRATCH_BYTES
 *     -> BQ8_ERR_SIZE (K <= 16384 always fits, at any N and rows <= 8);
 *   the device address of the array could not be obtained -> BQ8_ERR_HIP.
 * Every call on one GPU shares that GPU's array: calls that may overlap on
 * one GPU (different streams, no ordering between them) race and must not be
 * issued.  The array's contents on entry do not matter.
 * ---------------------------------------------------------------------- */
#define BQ8_TOP1_NOALLOC_SCRATCH_BYTES 262144
bq8_status q6k_lmhead_top1_noalloc(const void *pack, int64_t N, int64_t K, const float *x,
                                   int64_t M, int64_t row0, int64_t rows, int32_t *ids,
                                   void *stream);

/* ------------------------------------------------------------------------
 * The same fused head with the outputs target-verified speculation needs
 * ("Qwen3.6 27B AutoRound Handoff", "Current next-execution plan": a
 * candidate-max head gives the true top ids and values plus per-row
 * candidate scores).  For each projected row r (0 <= r < rows):
 *   ids[r]      as q6k_lmhead_top1;
 *   top_vals[r] the binary32 logit of ids[r] (NaN when ids[r] == -1; a
 *               maximal -0 is reported as +0);
 *   cand_scores[r*ncand + c], c < ncand: the binary32 logit of vocabulary
 *               row cand_ids[r*ncand + c], the same value the top-1 search
 *               compared (so it equals top_vals[r] bitwise when the
 *               candidate is ids[r]); NaN when the id is outside [0, N).
 * Target-side use: row0 = 0, rows = M = 6 projects all six rows.
 * cand_ids: device int32 [rows][ncand]; cand_scores: device f32
 *   [rows][ncand]; both may be NULL when ncand == 0; 0 <= ncand <= 8.
 * top_vals: device f32 [rows].  4-byte alignment.  Other arguments, scratch
 *   and shape as q6k_lmhead_top1.
 * ---------------------------------------------------------------------- */
bq8_status q6k_lmhead_candidate_max(const void *pack, int64_t N, int64_t K, const float *x,
                                    int64_t M, int64_t row0, int64_t rows,
                                    const int32_t *cand_ids, int64_t ncand, int32_t *ids,
                                    float *top_vals, float *cand_scores, void *scratch,
                                    int64_t scratch_bytes, void *stream);

/* ------------------------------------------------------------------------
 * Compact Q6_K pack: the raw Q6_K bits, re-tiled, so the fused head streams
 * 210 bytes per 256 weights instead of the expanded pack's 274 (the
 * fused-head page keeps its 1,360,793,600-byte expanded pack beside the
 * raw weights, "Memory and startup", and ranks persistent packs by time
 * saved per GiB, "Transfer to DeepSeek and future lanes").  Layout, with
 * the tiles of the expanded pack (n0, r, rows_t as there):
 *   QL plane (N*K/2 bytes at 0): raw byte i (0..127) of superblock s of row
 *       n at n0*(K/2) + ((8*s + i/16)*rows_t + r)*16 + i%16;
 *   QH plane (N*K/4 bytes at N*K/2): raw byte 128 + i (i = 0..63) at
 *       n0*(K/4) + ((4*s + i/16)*rows_t + r)*16 + i%16;
 *   SC plane (N*K/16 bytes at N*K*3/4): the subscales, as the expanded SC;
 *   D plane (N*K/128 bytes at N*K*13/16): the fp16 d, as the expanded D.
 * q6k_compact_bytes: host; 210*N*K/256, or -1 if the shape is invalid
 *   (1,042,944,000 for [248320 x 5120]).
 * q6k_pack_compact: raw Q6_K [N][K/256] (2-byte aligned) -> pack (16-byte
 *   aligned, pack_bytes == q6k_compact_bytes, fully overwritten).
 * q6k_lmhead_top1_compact, q6k_lmhead_candidate_max_compact: the fused head
 *   on the compact pack, with the arguments, scratch size and results of
 *   q6k_lmhead_top1 and q6k_lmhead_candidate_max.  For the same raw weights
 *   the logits are bitwise those of the expanded pack (the 6-bit codes are
 *   rebuilt in registers and the -32 offset is applied to exact integer
 *   dots), so ids, values and scores are identical.
 * ---------------------------------------------------------------------- */
int64_t q6k_compact_bytes(int64_t N, int64_t K);
bq8_status q6k_pack_compact(const void *raw, int64_t N, int64_t K, void *pack, int64_t pack_bytes,
                            void *stream);
bq8_status q6k_lmhead_top1_compact(const void *pack, int64_t N, int64_t K, const float *x,
                                   int64_t M, int64_t row0, int64_t rows, int32_t *ids,
                                   void *scratch, int64_t scratch_bytes, void *stream);
bq8_status q6k_lmhead_candidate_max_compact(const void *pack, int64_t N, int64_t K,
                                            const float *x, int64_t M, int64_t row0,
                                            int64_t rows, const int32_t *cand_ids, int64_t ncand,
                                            int32_t *ids, float *top_vals, float *cand_scores,
                                            void *scratch, int64_t scratch_bytes, void *stream);

/* ------------------------------------------------------------------------
 * Verifier-layer glue between projections (a width-6 FFN block whose gate
 * and up projections share one Q8_1 activation and whose down projection
 * consumes SiLU(gate)*up requantized to Q8_1; the closure page's width-6
 * gate/up and down projections and its down-to-next-RMS/Q8 boundary).
 *
 * silu_mul_q8_1: h = g / (1 + exp(-g)) * u elementwise, then hq = Q8_1(h).
 *   g, u: f32 [M][N] row-major; h: optional f32 [M][N] copy of h (NULL to
 *   skip); hq: Q8_1 [M][N/32].  Shape: M >= 1, N >= 32, N % 32 == 0,
 *   M*N < 2^31.  4-byte alignment.
 * rms_norm_q8_1: x = y / sqrt(mean_k(y^2) + eps) per row, then xq = Q8_1(x).
 *   y: f32 [M][K]; x: optional f32 [M][K] copy (NULL to skip); xq: Q8_1
 *   [M][K/32].  Shape: 1 <= M <= 64, 32 <= K <= 32768, K % 32 == 0;
 *   eps > 0.  4-byte alignment.
 * rms_norm_q8_1_sum: the same step on y = yparts[0] + ... + yparts[nparts-1]
 *   (f32 [nparts][M][K], added in part order in binary32, 1 <= nparts <= 8):
 *   the down-to-next-RMS/Q8 boundary of a split down projection.  y, x, xq
 *   are each optional (at least one given): y receives the summed rows, x the
 *   normalized rows, xq their Q8_1 blocks.  With nparts == 1 and y NULL it is
 *   rms_norm_q8_1.
 * ---------------------------------------------------------------------- */
bq8_status silu_mul_q8_1(const float *g, const float *u, int64_t M, int64_t N, float *h, void *hq,
                         void *stream);
bq8_status rms_norm_q8_1(const float *y, int64_t M, int64_t K, float eps, float *x, void *xq,
                         void *stream);
bq8_status rms_norm_q8_1_sum(const float *yparts, int64_t nparts, int64_t M, int64_t K, float eps,
                             float *y, float *x, void *xq, void *stream);

/* ------------------------------------------------------------------------
 * Width-M verifier FFN stream over `layers` layers, enqueued from native
 * code (five launches per layer on standard weights, no host
 * synchronization; the closure page's width-6 gate/up and down projections
 * and down-to-next-RMS/Q8 boundary, and the follow-up page's shared Q8_1
 * activation for sibling matmuls).
 * Per layer l:
 *   xq = Q8_1(x0)                        if l == 0   (q8_1_quantize)
 *   xq = rms_norm_q8_1(y, eps)           otherwise
 *   g  = q4_0_mmvq(w_gate[l], xq)        f32 [M][ffn]
 *   u  = q4_0_mmvq(w_up[l],   xq)        f32 [M][ffn]
 *   hq = silu_mul_q8_1(g, u)             Q8_1 [M][ffn/32]
 *   y  = q4_0_mmvq(w_down[l], hq)        f32 [M][hidden]
 * w_gate, w_up, w_down: HOST arrays of `layers` DEVICE pointers; gate and up
 *   are Q4_0 [ffn][hidden/32], down is Q4_0 [hidden][ffn/32]; 16-byte
 *   aligned.
 * x0: f32 [M][hidden] input of layer 0, 4-byte aligned (read only).
 * y:  f32 [M][hidden], 4-byte aligned; on completion the down output of the
 *   last layer (it is also each layer's intermediate).
 * work: device workspace of at least offsets[4] bytes from
 *   q4_0_ffn_stream_layout, 256-byte aligned.  On completion it holds the
 *   last layer's stage buffers: xq at offsets[0], g at offsets[1], u at
 *   offsets[2], hq at offsets[3].  The rest of it is internal.
 * Shape: 1 <= M <= 17, hidden and ffn multiples of 32, 32 <= hidden <= 32768,
 *   32 <= ffn <= 2^26, M*ffn < 2^31, 1 <= layers <= 2^20, eps > 0.
 * Every layer's pointers are checked before anything is enqueued.
 * q4_0_ffn_stream_layout: host; writes the four stage offsets and the total
 *   work-area size to offsets[0..4].  On a device the total also has room,
 *   after the stages, for the workspace of q4_0_mmvq_packed_ws_bytes(),
 *   which the packed pass below uses.
 * ---------------------------------------------------------------------- */
bq8_status q4_0_ffn_stream_layout(int64_t M, int64_t hidden, int64_t ffn, int64_t *offsets);
bq8_status q4_0_ffn_stream(const void *const *w_gate, const void *const *w_up,
                           const void *const *w_down, int64_t layers, int64_t M, int64_t hidden,
                           int64_t ffn, const float *x0, float eps, float *y, void *work,
                           int64_t work_bytes, void *stream);

/* The same pass on offline-packed weights (q4_0_pack of each matrix), three
 * launches per layer plus one at the end:
 *   xq = rms_norm_q8_1_sum(parts, P)              if l > 0
 *   hq = q4_0_gate_up_silu_q8_1_packed(w_gate[l], w_up[l], xq)
 *   parts = q4_0_mmvq_packed_split(w_down[l], hq, P)
 * with P = q4_0_mmvq_packed_splits(hidden, ffn), and after the last layer
 * y = the sum of its parts (rms_norm_q8_1_sum with only y).  y is written
 * only by that last step; the g and u stage buffers are not written.  When
 * work_bytes also covers the workspace (the layout's total on a device), the
 * joint launches are q4_0_gate_up_silu_q8_1_packed_ws on it, its counters
 * cleared once at the start of the pass by a kernel; with a work area that
 * holds the stages only, they are q4_0_gate_up_silu_q8_1_packed.
 * hidden and ffn must also be multiples of 512. */
bq8_status q4_0_ffn_stream_packed(const void *const *w_gate, const void *const *w_up,
                                  const void *const *w_down, int64_t layers, int64_t M,
                                  int64_t hidden, int64_t ffn, const float *x0, float eps,
                                  float *y, void *work, int64_t work_bytes, void *stream);

/* ------------------------------------------------------------------------
 * Measurement: a read-only HBM probe.
 *
 * Not a step of the method: the streaming ceiling that the weight-streaming
 * kernels are compared with, beside the 8 TB/s nominal peak of MI355X.
 * Reads bytes of buf (device, 16-byte aligned, bytes a multiple of 16) once
 * with 16-byte nontemporal loads, the way the products read their weights,
 * on `workgroups` workgroups of 256 threads with `unroll` (1, 2, 4 or 8)
 * loads in flight per thread, and writes one XOR of every 32-bit word read
 * per wave: out (device, caller-owned) receives 4 * workgroups uint32 words.
 * Asynchronous on stream; nothing else is written.
 * Errors: null pointers -> NULL; bytes < 16 or not a multiple of 16,
 *   workgroups outside 1..2^20, another unroll -> SHAPE; buf not 16-byte or
 *   out not 4-byte aligned -> ALIGN.
 * ---------------------------------------------------------------------- */
bq8_status bq8_hbm_read_probe(const void *buf, int64_t bytes, int64_t workgroups, int64_t unroll,
                              uint32_t *out, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* BQ8_H */
