// Q6_K expansion, the compact Q6_K pack, and the fused Q6_K LM-head
// projection with greedy top-1 (and its candidate-max outputs) on either.
//
// "Q6_K M=6 fused DFlash top-1 production record":
//   "Why this was slow" -- the Q6_K output tensor is expanded once into signed
//     int8 quants, int8 subscales and fp16 superblock scales; a kernel then
//     quantizes the useful activation rows, reuses each weight slice across
//     all of them and reduces to greedy ids without writing logits;
//   "Outcome" -- only decoder rows 1..5 of the six-row block are projected;
//   "Exactness and safety contracts" -- lowest-token-ID finite-tie rule, and
//     the exact pack layout and byte count;
//   "Memory and startup" -- the pack size for [5120, 248320].
// Formats: include/bq8.h.
//
// Pack layout (Q, SC and D planes split into tiles of 64 consecutive rows,
// the last tile ragged; include/bq8.h gives the offsets): within a tile the
// Q plane stores 16-value piece c of every row, row after row, then piece
// c + 1, so the 64 rows' piece c is one contiguous kilobyte.
//
// Top-1 mapping on gfx950: one wave per 64-row tile, lane <-> row.  Lane r
// loads its own 16-byte pieces; each load instruction of the wave reads one
// contiguous kilobyte, and the values land directly in the registers where
// they are used (no LDS staging).  The R quantized activation rows --
// identical for every lane -- come through scalar loads as v_dot4 operands.
// Per 32 values and activation row: 8 x v_dot4 give the two 16-value integer
// dots, which the two int8 subscales combine exactly in int32 (24-bit
// multiplies); the result, widened to binary32, is scaled by the row's d_x
// into a per-superblock sum, and d_w scales that sum once per superblock.
// The order of operations is the same for every row, so equal weight rows
// give bitwise equal logits.  Narrow vocabularies (under 3600 tiles, such as
// one GPU's 31040-row shard) have too few tiles to fill the CUs one wave per
// tile; there the waves of a workgroup share a tile, each summing one range
// of its superblocks, and the range sums are added in range order in LDS.
// Each lane keeps, per activation row, a 64-bit
// key
//     (order-preserving bits of the logit) << 32 | (0xFFFFFFFF - id)
// whose maximum is the largest logit with the lowest id among ties.  Keys
// meet by wave butterflies, then in LDS, then in one slot per workgroup in
// the caller's scratch; a one-workgroup kernel on the same stream reduces
// the slots and writes the ids.  Stream order, not a device-wide fence,
// publishes the slots: a per-workgroup release fence at device scope costs
// an L2 write-back on this multi-XCD part and doubled the kernel time.  No
// logit ever reaches memory, and max over integers makes the result
// independent of scheduling.
//
// Candidate-max: the lane that computes a candidate's vocabulary row stores
// that logit; the final kernel also decodes the winning key back to its
// logit.  "Qwen3.6 27B AutoRound Handoff", "Current next-execution plan":
// target-verified speculation needs the top ids and values and per-row
// candidate scores.
//
// Compact pack (include/bq8.h): the raw Q6_K bytes re-tiled like the
// expanded planes (ql, qh, subscales, scales); the same kernel rebuilds the
// 6-bit codes in registers and gives bitwise the expanded pack's logits.
// "Memory and startup": the expanded pack is kept beside the raw weights.
#include "bq8_dev.h"

#include <atomic>

namespace bq8 {

// ------------------------------------------------------------- expansion
constexpr int PACK_TILE = 64;

// Tile of row n: first row n0, rows in the tile, index of n in the tile.
__device__ __forceinline__ int tile_of(int n, int N, int &n0, int &r)
{
    n0 = n / PACK_TILE * PACK_TILE;
    r = n - n0;
    return (N - n0 < PACK_TILE) ? N - n0 : PACK_TILE;
}

// One wave per (superblock s, row n), rows fastest, so neighbouring waves
// fill neighbouring 16-byte pieces of the tiled planes.  Lane l produces the
// four codes 4l..4l+3 of the superblock: value e lies in half h = e/128;
// within it, c = (e%128)/32 picks the low (c < 2) or high nibble of
// ql[64h + 32(c&1) + l'] and bits 2c..2c+1 of qh[32h + l'], with l' = e%32.
__global__ __launch_bounds__(256) void q6k_expand_kernel(const uint8_t *__restrict__ raw, int N,
                                                         int K, int8_t *__restrict__ Q,
                                                         int8_t *__restrict__ SC,
                                                         uint16_t *__restrict__ D)
{
    const int lane = threadIdx.x & 63;
    const int64_t wave_id = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) >> 6;
    const int64_t nwaves = ((int64_t)gridDim.x * blockDim.x) >> 6;
    const int ns = K / QK_K;
    const int64_t total = (int64_t)N * ns;
    const int e = 4 * lane;
    const int h = e >> 7;
    const int c = (e & 127) >> 5;
    const int l0 = e & 31;
    const int ql_off = 64 * h + 32 * (c & 1) + l0;
    const int qh_off = 128 + 32 * h + l0;
    const int lo_shift = (c < 2) ? 0 : 4;
    const int hi_shift = 2 * c;
    for (int64_t i = wave_id; i < total; i += nwaves) {
        const int s = (int)(i / N);
        const int n = (int)(i - (int64_t)s * N);
        int n0, r;
        const int rows_t = tile_of(n, N, n0, r);
        const uint8_t *blk = raw + ((int64_t)n * ns + s) * Q6_K_BYTES;
        uint32_t packed = 0;
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const uint32_t lo = (blk[ql_off + t] >> lo_shift) & 0x0Fu;
            const uint32_t hi = (blk[qh_off + t] >> hi_shift) & 0x03u;
            const uint32_t code = lo | (hi << 4);
            packed |= ((code - 32u) & 0xFFu) << (8 * t);
        }
        // value e of superblock s is in piece 16 s + e/16 at byte e%16
        const int64_t piece = (int64_t)s * 16 + (e >> 4);
        *reinterpret_cast<uint32_t *>(Q + (int64_t)n0 * K + (piece * rows_t + r) * 16 + (e & 15)) =
            packed;
        if (lane < 4) {
            const uint8_t *sc = blk + 192 + 4 * lane;
            *reinterpret_cast<uint32_t *>(SC + (int64_t)n0 * (K / 16) +
                                          ((int64_t)s * rows_t + r) * 16 + 4 * lane) =
                (uint32_t)sc[0] | ((uint32_t)sc[1] << 8) | ((uint32_t)sc[2] << 16) |
                ((uint32_t)sc[3] << 24);
        }
        if (lane == 4)
            D[(int64_t)n0 * ns + (int64_t)s * rows_t + r] = (uint16_t)(blk[208] | (blk[209] << 8));
    }
}

// ------------------------------------------------------------- top-1
constexpr int TOP1_THREADS = 256;
constexpr int TOP1_WAVES = TOP1_THREADS / WAVE;
constexpr int TOP1_MAX_GRID = 1024;
constexpr int TOP1_MAX_ROWS = 8;
constexpr int TOP1_SPLIT_MAX_WAVES = 16;

__device__ __forceinline__ uint64_t make_key(float v, uint32_t id)
{
    if (v == 0.0f)
        v = 0.0f; // -0 ties with +0
    uint32_t u = __builtin_bit_cast(uint32_t, v);
    u = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
    return ((uint64_t)u << 32) | (uint64_t)(0xFFFFFFFFu - id);
}

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t k)
{
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
        const uint32_t lo = __shfl_xor((uint32_t)k, off, 64);
        const uint32_t hi = __shfl_xor((uint32_t)(k >> 32), off, 64);
        const uint64_t o = ((uint64_t)hi << 32) | lo;
        k = o > k ? o : k;
    }
    return k;
}

// Rows 0..R-1 of x (starting at row0) -> the Q8_1 quants and scales in
// scratch, block-major so that one superblock's activations for every row
// are contiguous: quants int8 [nb][R][32], scales f32 [nb][R] (the fp16 d of
// the block, widened exactly).  Also sets the nscores candidate scores to
// NaN; the fused kernel overwrites those whose id names a vocabulary row.
// With sx, also -32 x the sum of each 16-value half of every block's quants,
// int32 [nb][R][2] (the compact layout's -32 offset correction).
__global__ __launch_bounds__(256) void q6k_top1_prep_kernel(const float *__restrict__ x, int R,
                                                            int nb, int8_t *__restrict__ xq8,
                                                            float *__restrict__ dx,
                                                            int32_t *__restrict__ sx,
                                                            float *__restrict__ scores,
                                                            int nscores)
{
    const int gid = blockIdx.x * blockDim.x + threadIdx.x;
    if (gid < nscores)
        scores[gid] = __builtin_nanf("");
    const int blk = gid >> 5; // row-major (r, b) over the R rows of x
    const int j = gid & 31;
    const bool valid = blk < R * nb;
    const float v = valid ? x[(size_t)blk * QK + j] : 0.0f;
    float d;
    const int q = q8_1_block_quant(v, d);
    const int hs = row16_sum(q); // sum over the lane's 16-value half
    if (valid) {
        const int r = blk / nb, b = blk - r * nb;
        xq8[((size_t)b * R + r) * QK + j] = (int8_t)q;
        if (j == 0)
            dx[(size_t)b * R + r] = h2f(f2h(d));
        if (sx && (j & 15) == 0)
            sx[((size_t)b * R + r) * 2 + (j >> 4)] = -32 * hs;
    }
}

// The logits of this lane's weight row of the 64-row tile at n0 (the last
// row repeated in a ragged tile) over superblocks sb0 .. sb1 - 1 (sb1 >
// sb0), for the R activation rows: acc[i] = sum over those superblocks of
// d_w * (sum of the 16-value sub-block dots times their subscales), added
// superblock by superblock in order.
template <int R, bool COMPACT>
__device__ __forceinline__ void q6k_tile_logits(const int8_t *__restrict__ Q,
                                                const int8_t *__restrict__ QH,
                                                const int8_t *__restrict__ SC,
                                                const uint16_t *__restrict__ D, int N, int K,
                                                int n0, int sb0, int sb1,
                                                const int8_t *__restrict__ xq8,
                                                const float *__restrict__ dx,
                                                const int32_t *__restrict__ sx, float (&acc)[R])
{
    const int lane = threadIdx.x & 63;
    const int nsb = K / QK_K;
    const int rows_t = (N - n0 < PACK_TILE) ? N - n0 : PACK_TILE;
    const int r = lane < rows_t ? lane : rows_t - 1; // ragged tile: repeat the last row
    const int8_t *qt = Q + (size_t)n0 * (COMPACT ? K / 2 : K);
    const int8_t *ht = COMPACT ? QH + (size_t)n0 * (K / 4) : nullptr;
    const int8_t *st = SC + (size_t)n0 * (K / 16);
    const uint16_t *dt = D + (size_t)n0 * nsb;
#pragma unroll
    for (int i = 0; i < R; ++i)
        acc[i] = 0.0f;

    // expanded: pieces 16 sb + 8 half .. +7 of this lane's row (128
    // quants); compact: ql pieces 8 sb + 4 half .. +3 in v[0..3], qh
    // pieces 4 sb + 2 half .. +1 in v[4..5]
    auto load_half = [&](u32x4(&v)[8], int sb, int half) {
        if constexpr (COMPACT) {
#pragma unroll
            for (int j = 0; j < 4; ++j)
                v[j] = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(
                    qt + ((size_t)(sb * 8 + half * 4 + j) * rows_t + r) * 16));
#pragma unroll
            for (int j = 0; j < 2; ++j)
                v[4 + j] = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(
                    ht + ((size_t)(sb * 4 + half * 2 + j) * rows_t + r) * 16));
        } else {
            const int c0 = sb * 16 + half * 8;
#pragma unroll
            for (int j = 0; j < 8; ++j)
                v[j] = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(
                    qt + ((size_t)(c0 + j) * rows_t + r) * 16));
        }
    };
    // 32-blocks 4 half .. 4 half + 3 of the superblock, every activation row
    auto compute_half = [&](const u32x4(&v)[8], int half, const u32x4 &scw,
                            const int8_t *xs, const float *ds, const int32_t *xsum,
                            float(&accsb)[R]) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int bl = half * 4 + j;
            const uint32_t scword = scw[bl >> 1];
            const int sca = __builtin_amdgcn_sbfe(scword, 16 * (bl & 1), 8);
            const int scb = __builtin_amdgcn_sbfe(scword, 16 * (bl & 1) + 8, 8);
            // the block's 32 weights as 8 words of 4 signed bytes
            int w[8];
            if constexpr (COMPACT) {
                // code of value l (0..31) of block 4 half + j: low (j < 2)
                // or high nibble of ql byte 32 (j & 1) + l of the half,
                // bits 2j..2j+1 of its qh byte l
#pragma unroll
                for (int k = 0; k < 8; ++k) {
                    const uint32_t qlw = v[2 * (j & 1) + (k >> 2)][k & 3];
                    const uint32_t qhw = v[4 + (k >> 2)][k & 3];
                    const uint32_t lo = ((j < 2) ? qlw : (qlw >> 4)) & 0x0F0F0F0Fu;
                    w[k] = (int)(lo | (((qhw >> (2 * j)) & 0x03030303u) << 4));
                }
            } else {
#pragma unroll
                for (int k = 0; k < 8; ++k)
                    w[k] = (int)v[2 * j + (k >> 2)][k & 3];
            }
#pragma unroll
            for (int i = 0; i < R; ++i) {
                const int *xb = reinterpret_cast<const int *>(xs + (bl * R + i) * QK);
                // codes 0..63 stand for q + 32
                int sa = dot4(w[0], xb[0], COMPACT ? xsum[(bl * R + i) * 2] : 0);
                sa = dot4(w[1], xb[1], sa);
                sa = dot4(w[2], xb[2], sa);
                sa = dot4(w[3], xb[3], sa);
                int sbv = dot4(w[4], xb[4], COMPACT ? xsum[(bl * R + i) * 2 + 1] : 0);
                sbv = dot4(w[5], xb[5], sbv);
                sbv = dot4(w[6], xb[6], sbv);
                sbv = dot4(w[7], xb[7], sbv);
                // |sa|, |sbv| <= 16 * 32 * 127 < 2^23: exact 24-bit products
                const int I = __mul24(sa, sca) + __mul24(sbv, scb);
                accsb[i] = fmaf((float)I, ds[bl * R + i], accsb[i]);
            }
        }
    };

    // Both halves of the next superblock are in flight while one is
    // computed.  Loads are issued without branches (a wait-count join after
    // a skipped load would make later waits conservative): after the last
    // superblock of the range the prefetch repeats its addresses (cache
    // hits, never used).
    u32x4 va[8], vb[8];
    load_half(va, sb0, 0);
    load_half(vb, sb0, 1);
    u32x4 scw = *reinterpret_cast<const u32x4 *>(st + ((size_t)sb0 * rows_t + r) * 16);
    uint32_t dbits = dt[(size_t)sb0 * rows_t + r];
    for (int sb = sb0; sb < sb1; ++sb) {
        const int sbn = (sb + 1 < sb1) ? sb + 1 : sb;
        const u32x4 scw_next =
            *reinterpret_cast<const u32x4 *>(st + ((size_t)sbn * rows_t + r) * 16);
        const uint32_t dbits_next = dt[(size_t)sbn * rows_t + r];
        const int8_t *xs = xq8 + (size_t)sb * 8 * R * QK;
        const float *ds = dx + (size_t)sb * 8 * R;
        const int32_t *xsum = COMPACT ? sx + (size_t)sb * 8 * R * 2 : nullptr;
        float accsb[R];
#pragma unroll
        for (int i = 0; i < R; ++i)
            accsb[i] = 0.0f;
        compute_half(va, 0, scw, xs, ds, xsum, accsb);
        load_half(va, sbn, 0);
        compute_half(vb, 1, scw, xs, ds, xsum, accsb);
        load_half(vb, sbn, 1);
        const float dw = h2f(dbits);
#pragma unroll
        for (int i = 0; i < R; ++i)
            acc[i] = fmaf(accsb[i], dw, acc[i]);
        scw = scw_next;
        dbits = dbits_next;
    }
}

// Folds the logits acc[i] of vocabulary row n_raw (< N) into the running
// best keys of the R activation rows, and stores the candidate scores it
// names: per activation row i, the logits of vocabulary rows cand[i*ncand +
// c] (c < ncand) go to scores[i*ncand + c] from the one lane that computes
// them -- the same binary32 values the keys are made of.
template <int R>
__device__ __forceinline__ void q6k_fold(const float (&acc)[R], int n_raw,
                                         const int32_t *__restrict__ cand, int ncand,
                                         float *__restrict__ scores, uint64_t (&best)[R])
{
#pragma unroll
    for (int i = 0; i < R; ++i) {
        const float v = acc[i];
        if (!__builtin_isnan(v)) {
            const uint64_t k = make_key(v, (uint32_t)n_raw);
            best[i] = k > best[i] ? k : best[i];
        }
    }
    for (int c = 0; c < ncand; ++c)
#pragma unroll
        for (int i = 0; i < R; ++i)
            if (n_raw == cand[i * ncand + c])
                scores[i * ncand + c] = acc[i];
}

// Greedy top-1 over the vocabulary, one wave per 64-row tile: lane l owns
// weight row n0 + l and computes its logits over all of K, the wave keeps
// the best key per activation row, and the workgroup's maximum goes to
// slots[blockIdx.x][i] (cand / ncand / scores as in q6k_fold).
// COMPACT: the weight comes as the compact pack's ql (Q) and qh (QH) planes
// instead of the expanded int8 quants; per 32-block the 6-bit codes 0..63
// are rebuilt in registers and dotted as int8 into accumulators that start
// at -32 x sum(x quants) of their 16-value half (sx), which gives the
// expanded kernel's integer exactly.
template <int R, bool COMPACT>
__global__ __launch_bounds__(TOP1_THREADS) __attribute__((amdgpu_waves_per_eu(4))) void
q6k_top1_kernel(const int8_t *__restrict__ Q, const int8_t *__restrict__ QH,
                const int8_t *__restrict__ SC, const uint16_t *__restrict__ D, int N, int K,
                const int8_t *__restrict__ xq8, const float *__restrict__ dx,
                const int32_t *__restrict__ sx, uint64_t *__restrict__ slots,
                const int32_t *__restrict__ cand, int ncand, float *__restrict__ scores)
{
    __shared__ uint64_t wave_best[TOP1_WAVES][R];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int ntiles = (N + PACK_TILE - 1) / PACK_TILE;

    uint64_t best[R];
#pragma unroll
    for (int i = 0; i < R; ++i)
        best[i] = 0;
    for (int t = blockIdx.x * TOP1_WAVES + wave; t < ntiles; t += gridDim.x * TOP1_WAVES) {
        const int n0 = t * PACK_TILE;
        float acc[R];
        q6k_tile_logits<R, COMPACT>(Q, QH, SC, D, N, K, n0, 0, K / QK_K, xq8, dx, sx, acc);
        if (n0 + lane < N)
            q6k_fold(acc, n0 + lane, cand, ncand, scores, best);
    }

#pragma unroll
    for (int i = 0; i < R; ++i) {
        const uint64_t k = wave_max_u64(best[i]);
        if (lane == 0)
            wave_best[wave][i] = k;
    }
    __syncthreads();
    if (threadIdx.x < R) {
        uint64_t k = 0;
#pragma unroll
        for (int w = 0; w < TOP1_WAVES; ++w)
            k = wave_best[w][threadIdx.x] > k ? wave_best[w][threadIdx.x] : k;
        slots[(size_t)blockIdx.x * R + threadIdx.x] = k;
    }
}

// The same top-1 with every tile's superblocks cut into S ranges, for
// vocabularies too narrow to give each CU enough waves with whole tiles (a
// 31040-row shard of the 248320-row head has 485 tiles).  The workgroup's S
// waves share one tile at a time; wave w computes superblocks w*nsb/S ..
// (w+1)*nsb/S - 1 (S <= nsb, so no range is empty), the S partial logits
// are added in range order in LDS, and wave 0 folds the sums into its keys
// and candidate scores.  slots[blockIdx.x][i] as in q6k_top1_kernel.
template <int R, bool COMPACT>
__global__ __launch_bounds__(TOP1_SPLIT_MAX_WAVES * WAVE) __attribute__((amdgpu_waves_per_eu(4)))
void q6k_top1_split_kernel(const int8_t *__restrict__ Q, const int8_t *__restrict__ QH,
                           const int8_t *__restrict__ SC, const uint16_t *__restrict__ D, int N,
                           int K, const int8_t *__restrict__ xq8, const float *__restrict__ dx,
                           const int32_t *__restrict__ sx, uint64_t *__restrict__ slots,
                           const int32_t *__restrict__ cand, int ncand,
                           float *__restrict__ scores)
{
    __shared__ float part[TOP1_SPLIT_MAX_WAVES][R][WAVE];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int S = __builtin_amdgcn_readfirstlane(blockDim.x >> 6);
    const int nsb = K / QK_K;
    const int ntiles = (N + PACK_TILE - 1) / PACK_TILE;
    const int sb0 = wave * nsb / S, sb1 = (wave + 1) * nsb / S;

    uint64_t best[R];
#pragma unroll
    for (int i = 0; i < R; ++i)
        best[i] = 0;
    for (int t = blockIdx.x; t < ntiles; t += gridDim.x) {
        const int n0 = t * PACK_TILE;
        float acc[R];
        q6k_tile_logits<R, COMPACT>(Q, QH, SC, D, N, K, n0, sb0, sb1, xq8, dx, sx, acc);
#pragma unroll
        for (int i = 0; i < R; ++i)
            part[wave][i][lane] = acc[i];
        __syncthreads();
        if (wave == 0) {
#pragma unroll
            for (int i = 0; i < R; ++i)
                for (int w = 1; w < S; ++w)
                    acc[i] += part[w][i][lane];
            if (n0 + lane < N)
                q6k_fold(acc, n0 + lane, cand, ncand, scores, best);
        }
        __syncthreads(); // part is rewritten by the next tile
    }
    if (wave == 0) {
#pragma unroll
        for (int i = 0; i < R; ++i) {
            const uint64_t k = wave_max_u64(best[i]);
            if (lane == 0)
                slots[(size_t)blockIdx.x * R + i] = k;
        }
    }
}

// One workgroup: the maximum key of each row over every slot -> ids, and
// (if vals) the logit the key was made of.  Each thread takes every 256th
// slot and all R rows of it at once, so the loads are independent and the
// kernel waits on memory once.
template <int R>
__global__ __launch_bounds__(TOP1_THREADS) void q6k_top1_final_kernel(
    const uint64_t *__restrict__ slots, int nslots, int32_t *__restrict__ ids,
    float *__restrict__ vals)
{
    __shared__ uint64_t wave_best[TOP1_WAVES][R];
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    uint64_t k[R];
#pragma unroll
    for (int i = 0; i < R; ++i)
        k[i] = 0;
    for (int g = threadIdx.x; g < nslots; g += TOP1_THREADS) {
#pragma unroll
        for (int i = 0; i < R; ++i) {
            const uint64_t v = slots[(size_t)g * R + i];
            k[i] = v > k[i] ? v : k[i];
        }
    }
#pragma unroll
    for (int i = 0; i < R; ++i) {
        const uint64_t m = wave_max_u64(k[i]);
        if (lane == 0)
            wave_best[wave][i] = m;
    }
    __syncthreads();
    if (threadIdx.x < R) {
        uint64_t m = 0;
#pragma unroll
        for (int w = 0; w < TOP1_WAVES; ++w)
            m = wave_best[w][threadIdx.x] > m ? wave_best[w][threadIdx.x] : m;
        // no finite logit at all -> -1
        ids[threadIdx.x] = (m == 0) ? -1 : (int32_t)(0xFFFFFFFFu - (uint32_t)m);
        if (vals) {
            // invert the order-preserving map of make_key (-0 came in as +0)
            const uint32_t u = (uint32_t)(m >> 32);
            const uint32_t bits = (u & 0x80000000u) ? (u & 0x7FFFFFFFu) : ~u;
            vals[threadIdx.x] = (m == 0) ? __builtin_nanf("") : __builtin_bit_cast(float, bits);
        }
    }
}

// Superblock ranges per tile: 1 (one wave per whole tile) when the
// vocabulary has at least TOP1_SPLIT_BELOW tiles (the 248320-row head has
// 3880), else the smallest divisor S >= 4 of the superblock count (S <= 16)
// that gives at least TOP1_SPLIT_WAVES waves, or the largest divisor up to
// 16 (1 if there is none).  Measured at K = 5120 with rows 1..5 (µs per call,
// expanded pack, unsplit -> split): 31040 rows 135 -> 46 (S = 10), 65536 rows
// 146 -> 67, 131000 rows 162 -> 121, 229376 rows 211 -> 204 (S = 4); at
// 248320 rows the unsplit kernel is faster (220 against 228 with S = 4).
// Two ranges measured worse than four at every width.
constexpr int64_t TOP1_SPLIT_BELOW = 3600;
constexpr int64_t TOP1_SPLIT_WAVES = 4096;

static int top1_splits(int64_t N, int64_t K)
{
    const int64_t tiles = (N + WAVE - 1) / WAVE, nsb = K / QK_K;
    if (tiles >= TOP1_SPLIT_BELOW)
        return 1;
    int best = 1;
    for (int d = 2; d <= TOP1_SPLIT_MAX_WAVES && d <= nsb; ++d) {
        if (nsb % d != 0)
            continue;
        best = d;
        if (d >= 4 && tiles * d >= TOP1_SPLIT_WAVES)
            break;
    }
    return best;
}

// Workgroups of the fused kernel (= key slots per activation row): one per
// four tiles, or one per tile when the tiles are split, at most
// TOP1_MAX_GRID.
static int64_t top1_grid(int64_t N, int64_t K)
{
    const int64_t tiles = (N + WAVE - 1) / WAVE;
    int64_t g = top1_splits(N, K) > 1 ? tiles : (tiles + TOP1_WAVES - 1) / TOP1_WAVES;
    return g > TOP1_MAX_GRID ? TOP1_MAX_GRID : g;
}

static bool top1_shape_ok(int64_t N, int64_t K)
{
    return N >= 1 && N < (int64_t(1) << 31) - 1 && K >= QK_K && K % QK_K == 0 &&
           N * K < (int64_t(1) << 40) && K < (int64_t(1) << 24);
}

static int64_t round256(int64_t v) { return (v + 255) / 256 * 256; }

// Scratch: quants int8 [nb][rows][32] | scales f32 [nb][rows] | one u64 key
// per (workgroup, row); each area starts on a 256-byte boundary.
static int64_t xq8_area(int64_t K, int64_t rows) { return round256(rows * K); }
static int64_t dx_area(int64_t K, int64_t rows) { return round256(rows * (K / QK) * 4); }
static int64_t sx_area(int64_t K, int64_t rows) { return round256(rows * (K / QK) * 2 * 4); }

template <int R, bool COMPACT>
static void launch_top1(const int8_t *Q, const int8_t *QH, const int8_t *SC, const uint16_t *D,
                        int N, int K, const int8_t *xq8, const float *dx, const int32_t *sx,
                        uint64_t *slots, int32_t *ids, float *vals, const int32_t *cand,
                        int ncand, float *scores, int grid, int splits, hipStream_t s)
{
    if (splits > 1)
        hipLaunchKernelGGL((q6k_top1_split_kernel<R, COMPACT>), dim3(grid), dim3(WAVE * splits),
                           0, s, Q, QH, SC, D, N, K, xq8, dx, sx, slots, cand, ncand, scores);
    else
        hipLaunchKernelGGL((q6k_top1_kernel<R, COMPACT>), dim3(grid), dim3(TOP1_THREADS), 0, s, Q,
                           QH, SC, D, N, K, xq8, dx, sx, slots, cand, ncand, scores);
    hipLaunchKernelGGL(q6k_top1_final_kernel<R>, dim3(1), dim3(TOP1_THREADS), 0, s, slots, grid,
                       ids, vals);
}

template <bool COMPACT>
static void launch_top1_rows(int rows, const int8_t *Q, const int8_t *QH, const int8_t *SC,
                             const uint16_t *D, int N, int K, const int8_t *xq8, const float *dx,
                             const int32_t *sx, uint64_t *slots, int32_t *ids, float *vals,
                             const int32_t *cand, int ncand, float *scores, int grid, int splits,
                             hipStream_t s)
{
#define BQ8_TOP1_CASE(r)                                                                           \
    case r:                                                                                        \
        launch_top1<r, COMPACT>(Q, QH, SC, D, N, K, xq8, dx, sx, slots, ids, vals, cand, ncand,    \
                                scores, grid, splits, s);                                          \
        break;
    switch (rows) {
        BQ8_TOP1_CASE(1)
        BQ8_TOP1_CASE(2)
        BQ8_TOP1_CASE(3)
        BQ8_TOP1_CASE(4)
        BQ8_TOP1_CASE(5)
        BQ8_TOP1_CASE(6)
        BQ8_TOP1_CASE(7)
        BQ8_TOP1_CASE(8)
    }
#undef BQ8_TOP1_CASE
}

constexpr int TOP1_MAX_CAND = 8;

// Everything but argument checks: prep, fused kernel, final reduction.
// compact: pack is the compact layout (ql | qh | subscales | scales planes),
// else the expanded one (quants | subscales | scales).
static bq8_status lmhead_run(const void *pack, bool compact, int64_t N, int64_t K, const float *x,
                             int64_t row0, int64_t rows, const int32_t *cand, int64_t ncand,
                             int32_t *ids, float *vals, float *scores, void *scratch,
                             hipStream_t s)
{
    const int8_t *Q = (const int8_t *)pack;
    const int8_t *QH = compact ? Q + N * (K / 2) : nullptr;
    const int8_t *SC = compact ? Q + N * (K / 2) + N * (K / 4) : Q + N * K;
    const uint16_t *D = (const uint16_t *)(SC + N * (K / 16));
    uint8_t *base = (uint8_t *)scratch;
    int8_t *xq8 = (int8_t *)base;
    float *dx = (float *)(base + xq8_area(K, rows));
    int32_t *sx = (int32_t *)(base + xq8_area(K, rows) + dx_area(K, rows));
    uint64_t *slots =
        (uint64_t *)(base + xq8_area(K, rows) + dx_area(K, rows) + sx_area(K, rows));
    const int nb = (int)(K / QK);
    const int nblocks = (int)rows * nb;
    const int grid = (int)top1_grid(N, K);
    const int splits = top1_splits(N, K);
    const int nc = (int)ncand;
    (void)hipGetLastError();
    hipLaunchKernelGGL(q6k_top1_prep_kernel, dim3((nblocks * 32 + 255) / 256), dim3(256), 0, s,
                       x + row0 * K, (int)rows, nb, xq8, dx, compact ? sx : nullptr, scores,
                       (int)(rows * ncand));
    if (hipGetLastError() != hipSuccess)
        return BQ8_ERR_HIP;
    const int n = (int)N, k = (int)K, r = (int)rows;
    if (compact)
        launch_top1_rows<true>(r, Q, QH, SC, D, n, k, xq8, dx, sx, slots, ids, vals, cand, nc,
                               scores, grid, splits, s);
    else
        launch_top1_rows<false>(r, Q, QH, SC, D, n, k, xq8, dx, sx, slots, ids, vals, cand, nc,
                                scores, grid, splits, s);
    return launch_status();
}

// Compact pack, one thread per (row, superblock, 16-byte piece): pieces
// 0..7 of ql, 0..3 of qh, the 16 subscales (that thread also moves d).  The
// raw superblocks are 2-byte aligned, so pieces are read as halfwords.
__global__ __launch_bounds__(256) void q6k_compact_kernel(const uint8_t *__restrict__ raw, int N,
                                                          int K, uint8_t *__restrict__ QL,
                                                          uint8_t *__restrict__ QH,
                                                          uint8_t *__restrict__ SCP,
                                                          uint16_t *__restrict__ DP)
{
    const int ns = K / QK_K;
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= (int64_t)N * ns * 13)
        return;
    const int part = (int)(i % 13);
    const int64_t ns_i = i / 13;
    const int n = (int)(ns_i / ns), sb = (int)(ns_i - (int64_t)n * ns);
    int n0, r;
    const int rows_t = tile_of(n, N, n0, r);
    const uint8_t *blk = raw + ((int64_t)n * ns + sb) * Q6_K_BYTES;
    int src;
    uint8_t *dst;
    if (part < 8) {
        src = 16 * part;
        dst = QL + (int64_t)n0 * (K / 2) + ((int64_t)(8 * sb + part) * rows_t + r) * 16;
    } else if (part < 12) {
        src = 128 + 16 * (part - 8);
        dst = QH + (int64_t)n0 * (K / 4) + ((int64_t)(4 * sb + part - 8) * rows_t + r) * 16;
    } else {
        src = 192;
        dst = SCP + (int64_t)n0 * (K / 16) + ((int64_t)sb * rows_t + r) * 16;
        DP[(int64_t)n0 * ns + (int64_t)sb * rows_t + r] =
            *reinterpret_cast<const uint16_t *>(blk + 208);
    }
    const uint16_t *hw = reinterpret_cast<const uint16_t *>(blk + src);
    u32x4 v;
#pragma unroll
    for (int w = 0; w < 4; ++w)
        v[w] = (uint32_t)hw[2 * w] | ((uint32_t)hw[2 * w + 1] << 16);
    *reinterpret_cast<u32x4 *>(dst) = v;
}

} // namespace bq8

using namespace bq8;

BQ8_EXPORT int64_t q6k_pack_bytes(int64_t N, int64_t K)
{
    if (N < 1 || K < QK_K || K % QK_K != 0 || N > (int64_t(1) << 40) / K)
        return -1;
    return N * K + N * (K / 16) + 2 * N * (K / QK_K);
}

BQ8_EXPORT bq8_status q6k_pack_expand(const void *raw, int64_t N, int64_t K, void *pack,
                                      int64_t pack_bytes, void *stream)
{
    if (!raw || !pack)
        return BQ8_ERR_NULL;
    if (N < 1 || N >= (int64_t(1) << 31) || q6k_pack_bytes(N, K) < 0)
        return BQ8_ERR_SHAPE;
    if (!aligned(raw, 2) || !aligned(pack, 16))
        return BQ8_ERR_ALIGN;
    if (pack_bytes != q6k_pack_bytes(N, K))
        return BQ8_ERR_SIZE;
    const int64_t nsb = N * (K / QK_K);
    int8_t *Q = (int8_t *)pack;
    int8_t *SC = Q + N * K;
    uint16_t *D = (uint16_t *)(SC + N * (K / 16));
    int64_t grid = (nsb + 3) / 4; // 4 waves per workgroup, one superblock each
    if (grid > 65536)
        grid = 65536;
    (void)hipGetLastError();
    hipLaunchKernelGGL(q6k_expand_kernel, dim3((unsigned)grid), dim3(256), 0, (hipStream_t)stream,
                       (const uint8_t *)raw, (int)N, (int)K, Q, SC, D);
    return launch_status();
}

BQ8_EXPORT int64_t q6k_lmhead_top1_scratch_bytes(int64_t N, int64_t K, int64_t rows)
{
    if (!top1_shape_ok(N, K) || rows < 1 || rows > TOP1_MAX_ROWS)
        return -1;
    return xq8_area(K, rows) + dx_area(K, rows) + sx_area(K, rows) +
           top1_grid(N, K) * rows * (int64_t)sizeof(uint64_t);
}

BQ8_EXPORT bq8_status q6k_lmhead_top1(const void *pack, int64_t N, int64_t K, const float *x,
                                      int64_t M, int64_t row0, int64_t rows, int32_t *ids,
                                      void *scratch, int64_t scratch_bytes, void *stream)
{
    if (!pack || !x || !ids || !scratch)
        return BQ8_ERR_NULL;
    if (!top1_shape_ok(N, K) || rows < 1 || rows > TOP1_MAX_ROWS || M < 1 || row0 < 0 ||
        row0 + rows > M || M * K >= (int64_t(1) << 31))
        return BQ8_ERR_SHAPE;
    if (!aligned(pack, 16) || !aligned(x, 4) || !aligned(ids, 4) || !aligned(scratch, 16))
        return BQ8_ERR_ALIGN;
    if (scratch_bytes < q6k_lmhead_top1_scratch_bytes(N, K, rows))
        return BQ8_ERR_SIZE;
    return lmhead_run(pack, false, N, K, x, row0, rows, nullptr, 0, ids, nullptr, nullptr,
                      scratch, (hipStream_t)stream);
}

static bq8_status candidate_max(const void *pack, bool compact, int64_t N, int64_t K,
                                const float *x, int64_t M, int64_t row0, int64_t rows,
                                const int32_t *cand_ids, int64_t ncand, int32_t *ids,
                                float *top_vals, float *cand_scores, void *scratch,
                                int64_t scratch_bytes, void *stream)
{
    if (!pack || !x || !ids || !top_vals || !scratch || (ncand > 0 && (!cand_ids || !cand_scores)))
        return BQ8_ERR_NULL;
    if (!top1_shape_ok(N, K) || rows < 1 || rows > TOP1_MAX_ROWS || M < 1 || row0 < 0 ||
        row0 + rows > M || M * K >= (int64_t(1) << 31) || ncand < 0 || ncand > TOP1_MAX_CAND)
        return BQ8_ERR_SHAPE;
    if (!aligned(pack, 16) || !aligned(x, 4) || !aligned(ids, 4) || !aligned(top_vals, 4) ||
        !aligned(scratch, 16) || (ncand > 0 && (!aligned(cand_ids, 4) || !aligned(cand_scores, 4))))
        return BQ8_ERR_ALIGN;
    if (scratch_bytes < q6k_lmhead_top1_scratch_bytes(N, K, rows))
        return BQ8_ERR_SIZE;
    return lmhead_run(pack, compact, N, K, x, row0, rows, ncand > 0 ? cand_ids : nullptr, ncand,
                      ids, top_vals, ncand > 0 ? cand_scores : nullptr, scratch,
                      (hipStream_t)stream);
}

BQ8_EXPORT bq8_status q6k_lmhead_candidate_max(const void *pack, int64_t N, int64_t K,
                                               const float *x, int64_t M, int64_t row0,
                                               int64_t rows, const int32_t *cand_ids,
                                               int64_t ncand, int32_t *ids, float *top_vals,
                                               float *cand_scores, void *scratch,
                                               int64_t scratch_bytes, void *stream)
{
    return candidate_max(pack, false, N, K, x, M, row0, rows, cand_ids, ncand, ids, top_vals,
                         cand_scores, scratch, scratch_bytes, stream);
}

BQ8_EXPORT int64_t q6k_compact_bytes(int64_t N, int64_t K)
{
    if (N < 1 || N >= (int64_t(1) << 31) || K < QK_K || K % QK_K != 0 ||
        N > (int64_t(1) << 40) / K)
        return -1;
    return N * (K / QK_K) * Q6_K_BYTES;
}

BQ8_EXPORT bq8_status q6k_pack_compact(const void *raw, int64_t N, int64_t K, void *pack,
                                       int64_t pack_bytes, void *stream)
{
    if (!raw || !pack)
        return BQ8_ERR_NULL;
    if (q6k_compact_bytes(N, K) < 0 || N * (K / QK_K) * 13 >= (int64_t(1) << 40))
        return BQ8_ERR_SHAPE;
    if (!aligned(raw, 2) || !aligned(pack, 16))
        return BQ8_ERR_ALIGN;
    if (pack_bytes != q6k_compact_bytes(N, K))
        return BQ8_ERR_SIZE;
    uint8_t *QL = (uint8_t *)pack;
    uint8_t *QH = QL + N * (K / 2);
    uint8_t *SCP = QH + N * (K / 4);
    uint16_t *DP = (uint16_t *)(SCP + N * (K / 16));
    const int64_t items = N * (K / QK_K) * 13;
    (void)hipGetLastError();
    hipLaunchKernelGGL(q6k_compact_kernel, dim3((unsigned)((items + 255) / 256)), dim3(256), 0,
                       (hipStream_t)stream, (const uint8_t *)raw, (int)N, (int)K, QL, QH, SCP,
                       DP);
    return launch_status();
}

BQ8_EXPORT bq8_status q6k_lmhead_top1_compact(const void *pack, int64_t N, int64_t K,
                                              const float *x, int64_t M, int64_t row0,
                                              int64_t rows, int32_t *ids, void *scratch,
                                              int64_t scratch_bytes, void *stream)
{
    if (!pack || !x || !ids || !scratch)
        return BQ8_ERR_NULL;
    if (!top1_shape_ok(N, K) || rows < 1 || rows > TOP1_MAX_ROWS || M < 1 || row0 < 0 ||
        row0 + rows > M || M * K >= (int64_t(1) << 31))
        return BQ8_ERR_SHAPE;
    if (!aligned(pack, 16) || !aligned(x, 4) || !aligned(ids, 4) || !aligned(scratch, 16))
        return BQ8_ERR_ALIGN;
    if (scratch_bytes < q6k_lmhead_top1_scratch_bytes(N, K, rows))
        return BQ8_ERR_SIZE;
    return lmhead_run(pack, true, N, K, x, row0, rows, nullptr, 0, ids, nullptr, nullptr,
                      scratch, (hipStream_t)stream);
}

BQ8_EXPORT bq8_status q6k_lmhead_candidate_max_compact(const void *pack, int64_t N, int64_t K,
                                                       const float *x, int64_t M, int64_t row0,
                                                       int64_t rows, const int32_t *cand_ids,
                                                       int64_t ncand, int32_t *ids,
                                                       float *top_vals, float *cand_scores,
                                                       void *scratch, int64_t scratch_bytes,
                                                       void *stream)
{
    return candidate_max(pack, true, N, K, x, M, row0, rows, cand_ids, ncand, ids, top_vals,
                         cand_scores, scratch, scratch_bytes, stream);
}

// ------------------------------------------------- allocation-free head
namespace bq8 {
namespace noalloc {
// The scratch of q6k_lmhead_top1_noalloc.  Each GPU the library runs on has
// its own copy, held until the process ends.  On the host this name is only
// a stand-in: host code uses the device address noalloc_scratch() looks up.
static __device__ __align__(256) uint8_t scratch[BQ8_TOP1_NOALLOC_SCRATCH_BYTES];
} // namespace noalloc

// This GPU's address of noalloc::scratch, looked up once per device with that
// device current (hipGetSymbolAddress); nullptr if the runtime refuses.
static void *noalloc_scratch()
{
    static std::atomic<void *> addr[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64)
        return nullptr;
    void *p = addr[dev].load(std::memory_order_acquire);
    if (!p) {
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(noalloc::scratch)) != hipSuccess || !p)
            return nullptr;
        addr[dev].store(p, std::memory_order_release);
    }
    return p;
}
} // namespace bq8

BQ8_EXPORT bq8_status q6k_lmhead_top1_noalloc(const void *pack, int64_t N, int64_t K,
                                              const float *x, int64_t M, int64_t row0,
                                              int64_t rows, int32_t *ids, void *stream)
{
    if (!pack || !x || !ids)
        return BQ8_ERR_NULL;
    if (!top1_shape_ok(N, K) || rows < 1 || rows > TOP1_MAX_ROWS || M < 1 || row0 < 0 ||
        row0 + rows > M || M * K >= (int64_t(1) << 31))
        return BQ8_ERR_SHAPE;
    if (!aligned(pack, 16) || !aligned(x, 4) || !aligned(ids, 4))
        return BQ8_ERR_ALIGN;
    if (q6k_lmhead_top1_scratch_bytes(N, K, rows) > BQ8_TOP1_NOALLOC_SCRATCH_BYTES)
        return BQ8_ERR_SIZE;
    void *scr = noalloc_scratch();
    if (!scr)
        return BQ8_ERR_HIP;
    // every area of the scratch is written before it is read within the
    // call (quantized rows by the first kernel, one key per workgroup by the
    // second), so nothing needs clearing
    return lmhead_run(pack, false, N, K, x, row0, rows, nullptr, 0, ids, nullptr, nullptr, scr,
                      (hipStream_t)stream);
}

BQ8_EXPORT const char *bq8_status_string(bq8_status status)
{
    switch (status) {
    case BQ8_OK: return "ok";
    case BQ8_ERR_NULL: return "a required pointer is NULL";
    case BQ8_ERR_SHAPE: return "a size is out of range or not a block multiple";
    case BQ8_ERR_ALIGN: return "a pointer is not aligned as documented";
    case BQ8_ERR_SIZE: return "a byte count (pack or scratch) is not what is needed";
    case BQ8_ERR_HIP: return "the HIP runtime reported a launch error";
    default: return "unknown status";
    }
}

BQ8_EXPORT int32_t bq8_abi_version(void) { return BQ8_ABI_VERSION; }
