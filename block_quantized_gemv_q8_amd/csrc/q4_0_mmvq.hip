// Q4_0 x Q8_1 matrix-vector product at M = 1..17 activation rows.
//
// "Qwen3.6 27B Q4_0 DFlash/SYCL closure", "What materially worked": direct
// MMVQ coverage of every row count through 17 removed repeated full-weight
// reads; "Why the objectives were missed": the width-6 target verifier
// dominates each speculative cycle.  Each weight byte therefore crosses HBM
// exactly once per call, whatever M is, and is reused for all M rows from
// registers.
//
// Mapping on gfx950 (wave64):
//   * lane  <-> weight row n: a workgroup owns 64 consecutive rows;
//   * wave  <-> a slice of K: the S waves of a workgroup take the row's
//     8-block chunks (144 bytes, 16-byte aligned when K % 256 == 0)
//     round-robin, so one call launches ceil(N/64) * S waves -- enough to
//     cover 256 CUs even when N is only a few thousand rows;
//   * the M activation rows of the current block are the same for every
//     lane of a wave, so the compiler reads them with scalar loads into
//     SGPRs, where v_dot4 takes them as an operand at no VGPR/LDS cost.
// Per block and row: 8 x v_dot4_i32_i8 give the exact int32 dot
// sum_j (q_w - 8) * q_x; it is scaled by d_w * d_x (an exact binary32
// product of two fp16 values) and accumulated in binary32.  The S partial
// sums of a row meet in LDS and are added in wave order, so results are
// deterministic and equal rows give equal outputs.
#include "bq8_dev.h"
#include "bq8_host.h"

#include <utility>

namespace bq8 {

// 32-bit word at byte offset `off` (a compile-time constant after
// unrolling) of a register array holding 16-byte-aligned memory.
template <int OFF>
__device__ __forceinline__ uint32_t word_at(const uint32_t *w)
{
    if constexpr (OFF % 4 == 0)
        return w[OFF / 4];
    else
        return __builtin_amdgcn_alignbyte(w[OFF / 4 + 1], w[OFF / 4], OFF % 4);
}

// Accumulate one Q4_0 block (scale bits `dbits`, nibble words qs[0..3])
// against block `b` of every activation row.  Each nibble q is placed in the
// high half of a byte with its top bit flipped, which is the signed byte
// 16*(q - 8); the int32 dot is therefore 16x the exact block dot, and the
// caller scales the finished sums by 1/16 (exact: a power of two).
template <int M>
__device__ __forceinline__ void block_dot(uint32_t dbits, const uint32_t qs[4],
                                          const uint8_t *__restrict__ xq, int nb, int b,
                                          float acc[M])
{
    int lo[4], hi[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        lo[i] = (int)(((qs[i] << 4) & 0xF0F0F0F0u) ^ 0x80808080u); // elements 4i .. 4i+3
        hi[i] = (int)((qs[i] & 0xF0F0F0F0u) ^ 0x80808080u);        // elements 16+4i .. 16+4i+3
    }
    const float dw = h2f(dbits);
#pragma unroll
    for (int m = 0; m < M; ++m) {
        const uint32_t *xb =
            reinterpret_cast<const uint32_t *>(xq + ((size_t)m * nb + b) * Q8_1_BYTES);
        int s = dot4(lo[0], (int)xb[1], 0);
        s = dot4(lo[1], (int)xb[2], s);
        s = dot4(lo[2], (int)xb[3], s);
        s = dot4(lo[3], (int)xb[4], s);
        s = dot4(hi[0], (int)xb[5], s);
        s = dot4(hi[1], (int)xb[6], s);
        s = dot4(hi[2], (int)xb[7], s);
        s = dot4(hi[3], (int)xb[8], s);
        const float scale = dw * h2f(xb[0]);
        acc[m] = fmaf((float)s, scale, acc[m]);
    }
}

template <int J, int M>
__device__ __forceinline__ void chunk_block(const uint32_t *wd, const uint8_t *__restrict__ xq,
                                            int nb, int b, float acc[M])
{
    constexpr int o = J * Q4_0_BYTES;
    const uint32_t dword = wd[o / 4];
    const uint32_t dbits = (o % 4 == 0) ? dword : (dword >> 16);
    uint32_t qs[4];
    qs[0] = word_at<o + 2>(wd);
    qs[1] = word_at<o + 6>(wd);
    qs[2] = word_at<o + 10>(wd);
    qs[3] = word_at<o + 14>(wd);
    block_dot<M>(dbits, qs, xq, nb, b, acc);
}

template <int M, int... J>
__device__ __forceinline__ void chunk_all(const uint32_t *wd, const uint8_t *__restrict__ xq, int nb,
                                          int b0, float acc[M], std::integer_sequence<int, J...>)
{
    (chunk_block<J, M>(wd, xq, nb, b0 + J, acc), ...);
}


constexpr int CHUNK_BYTES = 8 * Q4_0_BYTES;           // 144: eight blocks, 16-byte aligned
constexpr int CHUNK_PIECES = CHUNK_BYTES / 16;         // 9 x 16 bytes
constexpr int STAGE_BYTES = WAVE * CHUNK_BYTES;        // 64 rows x 144 bytes per wave

// ALIGNED (K % 256 == 0, w 16-byte aligned): a wave stages the 144-byte
// chunk c of its 64 rows through LDS.  The 576 16-byte pieces are loaded
// with nine 128-bit loads in which nine consecutive lanes read one row's
// contiguous 144 bytes (each load instruction touches ~7 rows instead of
// 64), written to LDS in the same order (so LDS holds [row][144 bytes]),
// then every lane reads back its own row.
// Otherwise (any K % 32 == 0) each lane reads its row's blocks directly
// with 16-bit loads (always aligned).
template <int M, bool ALIGNED>
__global__ __launch_bounds__(1024) void q4_0_mmvq_dot4_kernel(const uint8_t *__restrict__ w,
                                                              int N, int nb,
                                                              const uint8_t *__restrict__ xq,
                                                              float *__restrict__ y)
{
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int S = __builtin_amdgcn_readfirstlane(blockDim.x >> 6);
    const int n0 = blockIdx.x * WAVE;
    const size_t row_bytes = (size_t)nb * Q4_0_BYTES;

    float acc[M];
#pragma unroll
    for (int m = 0; m < M; ++m)
        acc[m] = 0.0f;

    if constexpr (ALIGNED) {
        uint8_t *stage = smem + (size_t)wave * STAGE_BYTES;
        const uint8_t *tile = w + (size_t)n0 * row_bytes;
        // per-lane byte offsets (within the tile) of the nine pieces it loads;
        // rows past N repeat row N-1 so every load stays in bounds
        uint32_t goff[CHUNK_PIECES];
#pragma unroll
        for (int j = 0; j < CHUNK_PIECES; ++j) {
            const int p = j * WAVE + lane;
            const int r = p / CHUNK_PIECES;
            const int q = p - r * CHUNK_PIECES;
            const int rr = (n0 + r < N) ? r : (N - 1 - n0);
            goff[j] = (uint32_t)(rr * row_bytes) + 16u * (uint32_t)q;
        }
        const int nchunks = nb >> 3;
        for (int c = wave; c < nchunks; c += S) {
            const uint8_t *src = tile + (size_t)c * CHUNK_BYTES;
            u32x4 v[CHUNK_PIECES];
#pragma unroll
            for (int j = 0; j < CHUNK_PIECES; ++j)
                v[j] = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(src + goff[j]));
            wave_lds_sync();
#pragma unroll
            for (int j = 0; j < CHUNK_PIECES; ++j)
                reinterpret_cast<u32x4 *>(stage)[j * WAVE + lane] = v[j];
            wave_lds_sync();
            uint32_t wd[36];
#pragma unroll
            for (int i = 0; i < CHUNK_PIECES; ++i) {
                const u32x4 t = reinterpret_cast<const u32x4 *>(stage + lane * CHUNK_BYTES)[i];
                wd[4 * i + 0] = t[0];
                wd[4 * i + 1] = t[1];
                wd[4 * i + 2] = t[2];
                wd[4 * i + 3] = t[3];
            }
            chunk_all<M>(wd, xq, nb, c * 8, acc, std::make_integer_sequence<int, 8>{});
        }
    } else {
        const int n = (n0 + lane < N) ? n0 + lane : N - 1;
        const uint8_t *row = w + (size_t)n * row_bytes;
        for (int b = wave; b < nb; b += S) {
            const uint16_t *p = reinterpret_cast<const uint16_t *>(row + (size_t)b * Q4_0_BYTES);
            uint32_t qs[4];
#pragma unroll
            for (int i = 0; i < 4; ++i)
                qs[i] = (uint32_t)p[1 + 2 * i] | ((uint32_t)p[2 + 2 * i] << 16);
            block_dot<M>(p[0], qs, xq, nb, b, acc);
        }
    }

    // partial sums of the S waves meet in LDS (reusing the staging area)
    __syncthreads();
    float *partial = reinterpret_cast<float *>(smem); // [S][M][64]
#pragma unroll
    for (int m = 0; m < M; ++m)
        partial[(wave * M + m) * WAVE + lane] = acc[m];
    __syncthreads();
    for (int idx = threadIdx.x; idx < M * WAVE; idx += blockDim.x) {
        const int m = idx / WAVE;
        const int l = idx % WAVE;
        float s = 0.0f;
        for (int v = 0; v < S; ++v)
            s += partial[(v * M + m) * WAVE + l];
        const int nn = n0 + l;
        if (nn < N)
            y[(size_t)m * N + nn] = s * 0.0625f;
    }
}

// ---------------------------------------------------------------- MFMA
// Padded int8 MFMA, v_mfma_i32_16x16x64_i8 (D[16][16] += A[16][64] *
// B[64][16]), used block-diagonally so one instruction produces the exact
// integer dots of 16 weight rows x 2 blocks x 8 activation rows:
//   B column n = weight row n of the 16-row tile; k in [0,32) is block
//     8G+j of the chunk, k in [32,64) is block 8G+j+4 (same 2-byte alignment);
//   A row i = (blk, m) = (i/8, i%8) holds activation row 8s+m of block
//     8G+j+4*blk in its own half of k and zeros in the other half (and zeros
//     past M); s = 0..ceil(M/8)-1 selects a set of eight activation rows,
//     each set one MFMA sharing the same B.
// Lane l (c = l%16, g = l/16) supplies B column c, k-group g: 16 signed bytes
// 16*(q-8) made from qs[8h..8h+7] (h = g%2) of block 8G+j+4*(g/2) -- eight
// low nibbles, then eight high nibbles -- and A row c, k-group g: the
// matching activation bytes q[8h..8h+7], q[16+8h..16+8h+7] (or zeros).  The k
// order inside a block is the same on both sides, so D[(blk,m)][n] = 16 * I.
// Output lane l holds D rows 4g..4g+3 = block 8G+j+4*(g/2), m = 4h..4h+3 of
// column c: exactly the block whose weight scale the lane read, so each of
// its sums is scaled by d_w * d_x[m] and accumulated in binary32.  Lanes l
// and l+32 hold the two halves of the chunk and are added at the end; then
// the S waves' sums meet in LDS in wave order.
//
// Streaming: the S waves of a workgroup share one 16-row tile and take its
// CB-block chunks round-robin.  A chunk is 16 rows x CB*18 contiguous bytes
// (CB = 32: 576-byte runs, the longest that divide the usual K) plus the
// chunk's CB Q8_1 blocks of every activation row; both are loaded as 16-byte
// pieces (consecutive lanes along each contiguous run), written to the
// wave's LDS stage, and read back in MFMA operand order.  The next chunk's
// loads are issued before the current chunk is computed, and compute reads
// only LDS, so the wait for one chunk never waits for the next.

template <int M, int CB, int NST>
struct MfmaShape {
    static constexpr int MS = (M + 7) / 8;                   // MFMAs per block pair
    static constexpr int RUN = CB * Q4_0_BYTES;              // weight bytes per row per chunk
    static constexpr int XRUN = CB * Q8_1_BYTES;             // activation bytes per row per chunk
    static constexpr int WPIECES = 16 * RUN / 16;            // 16 rows of weights
    static constexpr int XPIECES = M * XRUN / 16;            // M rows of activations
    static constexpr int PIECES = WPIECES + XPIECES;
    static constexpr int LOADS = (PIECES + WAVE - 1) / WAVE; // DMA instructions per chunk
    static constexpr int DXOFF = LOADS * WAVE * 16;          // f32 d_x [CB][8*MS] after the pieces
    static constexpr int STAGE = DXOFF + CB * 8 * MS * 4;    // bytes per stage
    static constexpr int WAVE_LDS = NST * STAGE;             // bytes per wave
};

// One workgroup owns a 16-row tile; its S waves take the tile's CB-block
// chunks round-robin.  A chunk is staged in LDS as a list of 16-byte pieces:
// first the tile's 16 rows x CB*18 contiguous weight bytes (consecutive lanes
// along each row run), then the chunk's CB Q8_1 blocks of each activation
// row.  The pieces travel by global_load_lds_dwordx4 -- global memory straight
// into LDS, 64 lanes x 16 bytes per instruction -- into an NST-stage ring per
// wave, so NST-1 chunks are in flight while one is computed and no VGPRs hold
// data in transit.  Every load is issued unconditionally (past the wave's
// last chunk it repeats the last chunk's addresses: cache hits, never used)
// so the wait counts stay exact.
template <int M, int CB, int NST>
__global__ __launch_bounds__(512) void q4_0_mmvq_mfma_kernel(const uint8_t *__restrict__ w,
                                                              int N, int nb,
                                                              const uint8_t *__restrict__ xq,
                                                              float *__restrict__ y)
{
    using SH = MfmaShape<M, CB, NST>;
    constexpr int MS = SH::MS, LOADS = SH::LOADS;
    static_assert(CB % 8 == 0 && (SH::RUN % 16) == 0 && (SH::XRUN % 16) == 0, "chunk shape");
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int S = __builtin_amdgcn_readfirstlane(blockDim.x >> 6);
    const int n0 = blockIdx.x * 16;
    const size_t row_bytes = (size_t)nb * Q4_0_BYTES;
    uint8_t *ring = smem + (size_t)wave * SH::WAVE_LDS;

    const int c16 = lane & 15;
    const int g = lane >> 4;
    const int h = g & 1;
    const int hb = g >> 1;
    bool a_on[MS];
    uint32_t aoff[MS]; // offset of this lane's A row (activation row 8s + c16%8) in a stage
#pragma unroll
    for (int s = 0; s < MS; ++s) {
        const int m = 8 * s + (c16 & 7);
        a_on[s] = ((c16 >> 3) == hb) && (m < M);
        aoff[s] = (uint32_t)SH::WPIECES * 16 + (uint32_t)(a_on[s] ? m : 0) * SH::XRUN;
    }
    // per-lane source of piece p = 64j + lane at chunk c: base[j] + c * step[j]
    const uint8_t *base[LOADS];
    uint32_t step[LOADS];
    {
        const uint8_t *tile = w + (size_t)n0 * row_bytes;
#pragma unroll
        for (int j = 0; j < LOADS; ++j) {
            const int p = j * WAVE + lane;
            if (p < SH::WPIECES) {
                const int r = p / (SH::RUN / 16);
                const int q = p - r * (SH::RUN / 16);
                const int rr = (n0 + r < N) ? r : (N - 1 - n0);
                base[j] = tile + (size_t)rr * row_bytes + 16 * q;
                step[j] = SH::RUN;
            } else if (p < SH::PIECES) {
                const int px = p - SH::WPIECES;
                const int m = px / (SH::XRUN / 16);
                const int q = px - m * (SH::XRUN / 16);
                base[j] = xq + (size_t)m * nb * Q8_1_BYTES + 16 * q;
                step[j] = SH::XRUN;
            } else {
                base[j] = tile; // padding slot: a valid address, never read back
                step[j] = SH::RUN;
            }
        }
    }
    auto issue = [&](int c, int st) {
        uint8_t *dst = ring + st * SH::STAGE;
#pragma unroll
        for (int j = 0; j < LOADS; ++j)
            __builtin_amdgcn_global_load_lds((global_void_t *)(base[j] + (size_t)c * step[j]),
                                             (lds_void_t *)(dst + j * WAVE * 16), 16, 0, 0);
    };

    float acc[MS][4];
#pragma unroll
    for (int s = 0; s < MS; ++s)
#pragma unroll
        for (int r = 0; r < 4; ++r)
            acc[s][r] = 0.0f;

    auto compute = [&](int st) {
        const uint8_t *stage = ring + st * SH::STAGE;
        float *dxs = reinterpret_cast<float *>(ring + st * SH::STAGE + SH::DXOFF);
        // d_x of the chunk's blocks as f32: dxs[b*8*MS + m], 0 past M
#pragma unroll
        for (int i = lane; i < CB * 8 * MS; i += WAVE) {
            const int b = i / (8 * MS), m = i - (i / (8 * MS)) * (8 * MS);
            const uint16_t bits = *reinterpret_cast<const uint16_t *>(
                stage + SH::WPIECES * 16 + (m < M ? m : 0) * SH::XRUN + b * Q8_1_BYTES);
            dxs[i] = (m < M) ? h2f(bits) : 0.0f;
        }
        wave_lds_sync();
#pragma unroll
        for (int G = 0; G < CB / 8; ++G) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int bl = 8 * G + j + 4 * hb; // this lane's block within the chunk
                i32x4 A[MS];
                float dx[MS][4];
#pragma unroll
                for (int s = 0; s < MS; ++s) {
                    const uint32_t *xb =
                        reinterpret_cast<const uint32_t *>(stage + aoff[s] + bl * Q8_1_BYTES);
                    const int a0 = (int)xb[1 + 2 * h], a1 = (int)xb[2 + 2 * h];
                    const int a2 = (int)xb[5 + 2 * h], a3 = (int)xb[6 + 2 * h];
                    A[s][0] = a_on[s] ? a0 : 0;
                    A[s][1] = a_on[s] ? a1 : 0;
                    A[s][2] = a_on[s] ? a2 : 0;
                    A[s][3] = a_on[s] ? a3 : 0;
                    const float *dxp = dxs + bl * 8 * MS + 8 * s + 4 * h;
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        dx[s][r] = dxp[r];
                }
                // block bl of staged row c16: d at byte o = 18*bl, qs at o + 2
                const uint8_t *bp = stage + c16 * SH::RUN + Q4_0_BYTES * bl;
                uint32_t x0, x1, dbits;
                if (j & 1) { // o = 2 mod 4: qs 4-byte aligned, d in the high half before it
                    const uint32_t *pw = reinterpret_cast<const uint32_t *>(bp - 2);
                    dbits = pw[0] >> 16;
                    x0 = pw[1 + 2 * h];
                    x1 = pw[2 + 2 * h];
                } else {     // o = 0 mod 4: d in the low half, qs start 2 bytes in
                    const uint32_t *pw = reinterpret_cast<const uint32_t *>(bp);
                    dbits = pw[0];
                    const uint32_t a0 = pw[2 * h], a1 = pw[2 * h + 1], a2 = pw[2 * h + 2];
                    x0 = __builtin_amdgcn_alignbyte(a1, a0, 2);
                    x1 = __builtin_amdgcn_alignbyte(a2, a1, 2);
                }
                i32x4 B;
                B[0] = (int)(((x0 << 4) & 0xF0F0F0F0u) ^ 0x80808080u);
                B[1] = (int)(((x1 << 4) & 0xF0F0F0F0u) ^ 0x80808080u);
                B[2] = (int)((x0 & 0xF0F0F0F0u) ^ 0x80808080u);
                B[3] = (int)((x1 & 0xF0F0F0F0u) ^ 0x80808080u);
                const float dw = h2f(dbits);
#pragma unroll
                for (int s = 0; s < MS; ++s) {
                    const i32x4 D = __builtin_amdgcn_mfma_i32_16x16x64_i8(
                        A[s], B, (i32x4){0, 0, 0, 0}, 0, 0, 0);
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        acc[s][r] = fmaf((float)D[r], dw * dx[s][r], acc[s][r]);
                }
            }
        }
        wave_lds_sync();
    };

    // Chunks wave, wave+S, ...; the wave's k-th chunk lives in stage k % NST.
    // The compiler does not order LDS reads after these DMA loads, so the
    // wait is explicit: before computing chunk k, exactly (NST-1)*LOADS
    // younger DMA instructions (chunks k+1 .. k+NST-1) may still be
    // outstanding and every older one -- chunk k's -- must have landed.
    constexpr int YOUNGER = (NST - 1) * LOADS;
    static_assert(YOUNGER <= 63, "vmcnt field");
    constexpr int WAIT_IMM = waitcnt_vmcnt(YOUNGER);
    const int nchunks = nb / CB;
    if (wave < nchunks) {
        const int mine = (nchunks - wave + S - 1) / S; // this wave's chunk count
#pragma unroll
        for (int k = 0; k < NST - 1; ++k)
            issue(wave + S * (k < mine ? k : mine - 1), k);
        for (int k = 0; k < mine; ++k) {
            const int kn = k + NST - 1;
            issue(wave + S * (kn < mine ? kn : mine - 1), kn % NST);
            __builtin_amdgcn_s_waitcnt(WAIT_IMM);
            compute(k % NST);
        }
    }

    // the two chunk halves (lanes l and l+32), then the S waves in order
#pragma unroll
    for (int s = 0; s < MS; ++s)
#pragma unroll
        for (int r = 0; r < 4; ++r)
            acc[s][r] += __shfl_xor(acc[s][r], 32, 64);
    __builtin_amdgcn_s_waitcnt(0); // no load may still be writing the LDS reused below
    __syncthreads();
    constexpr int SLOTS = MS * 4;
    float *partial = reinterpret_cast<float *>(smem); // [S][SLOTS][32]
    if (lane < 32) {
#pragma unroll
        for (int s = 0; s < MS; ++s)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                partial[(wave * SLOTS + s * 4 + r) * 32 + lane] = acc[s][r];
    }
    __syncthreads();
    for (int idx = threadIdx.x; idx < SLOTS * 32; idx += blockDim.x) {
        const int slot = idx >> 5, l = idx & 31;
        const int s = slot >> 2, r = slot & 3;
        const int m = 8 * s + 4 * (l >> 4) + r;
        const int nn = n0 + (l & 15);
        float sacc = 0.0f;
        for (int v = 0; v < S; ++v)
            sacc += partial[(v * SLOTS + slot) * 32 + l];
        if (m < M && nn < N)
            y[(size_t)m * N + nn] = sacc * 0.0625f;
    }
}

// Waves per workgroup of the dot4 kernel: enough workgroups x waves to give
// every CU several waves, never more waves than K-units, at most 16 waves
// (1024 threads: 16 x 9216 bytes of staging fit gfx950's 160 KB of LDS), and
// at most 128 partial rows of LDS (S * M <= 128).
static int pick_splits(int64_t N, int64_t units, int M, int64_t lds_limit, bool staged)
{
    const int64_t tiles = (N + WAVE - 1) / WAVE;
    const int64_t target_waves = 256 * 8;
    int64_t s = (target_waves + tiles - 1) / tiles;
    if (s > 16)
        s = 16;
    if (s > units)
        s = units;
    if (s > 128 / M)
        s = 128 / M;
    if (staged && s > lds_limit / STAGE_BYTES)
        s = lds_limit / STAGE_BYTES;
    return (int)(s < 1 ? 1 : s);
}

// Waves per workgroup for the MFMA kernel: four (measured best on the
// ffn_up and down shapes for every M, against 1..8), fewer when the row has
// fewer chunks or LDS cannot hold four rings.
template <int M, int CB, int NST>
static int mfma_waves(int64_t N, int nb, int64_t limit)
{
    (void)N;
    int64_t s = 4;
    if (s > nb / CB)
        s = nb / CB;
    while (s > 1 && s * MfmaShape<M, CB, NST>::WAVE_LDS > limit)
        --s;
    return (int)(s < 1 ? 1 : s);
}

template <int M, int CB, int NST>
static bq8_status launch_mfma(const void *w, int64_t N, int nb, const void *xq, float *y,
                              hipStream_t stream, int64_t limit, int waves)
{
    using SH = MfmaShape<M, CB, NST>;
    const int64_t tiles = (N + 15) / 16;
    const int s = waves > 0 ? waves : mfma_waves<M, CB, NST>(N, nb, limit);
    const int64_t ring = (int64_t)s * SH::WAVE_LDS;
    const int64_t partial = (int64_t)s * SH::MS * 4 * 32 * (int64_t)sizeof(float);
    const int64_t lds = ring > partial ? ring : partial;
    if (!allow_dynamic_lds((const void *)q4_0_mmvq_mfma_kernel<M, CB, NST>, limit))
        return BQ8_ERR_HIP;
    hipLaunchKernelGGL((q4_0_mmvq_mfma_kernel<M, CB, NST>), dim3((unsigned)tiles), dim3(WAVE * s),
                       (size_t)lds, stream, (const uint8_t *)w, (int)N, nb, (const uint8_t *)xq, y);
    return launch_status();
}

template <int M>
static bq8_status mmvq_launch(const void *w, int64_t N, int64_t K, const void *xq, float *y,
                              void *stream)
{
    if (!w || !xq || !y)
        return BQ8_ERR_NULL;
    if (N < 1 || N >= (int64_t(1) << 31) || K < QK || K % QK != 0 ||
        N * (K / QK) * Q4_0_BYTES >= (int64_t(1) << 40) || K > (int64_t(1) << 26) ||
        (int64_t)M * K >= (int64_t(1) << 31))
        return BQ8_ERR_SHAPE;
    if (!aligned(w, 16) || !aligned(xq, 16) || !aligned(y, 4))
        return BQ8_ERR_ALIGN;
    const int nb = (int)(K / QK);
    const bool al = (K % 256 == 0);
    const int64_t limit = device_lds_limit();
    hipStream_t s = (hipStream_t)stream;
    (void)hipGetLastError();
    {
        // MFMA path for K a multiple of 256: 8-block chunks in a ring of two
        // stages.  A third stage grows each wave's ring by a chunk of M
        // activation rows and, from M = 7, leaves fewer workgroups per CU:
        // two builds in one process, interleaved, three stages against two,
        // down [5120 x 17408] M = 7 / 9 / 13 / 16 / 17: 20.3 / 24.4 / 26.9 /
        // 41.0 / 52.7 against 19.5 / 24.1 / 25.5 / 27.6 / 33.9 us; ffn_up
        // [17408 x 5120] M = 7 / 9 / 13 / 16 / 17: 18.4 / 23.3 / 25.5 / 38.8 /
        // 48.5 against 16.5 / 19.6 / 21.4 / 25.0 / 31.8 us
        constexpr int NST = 2;
        if (al && MfmaShape<M, 8, NST>::WAVE_LDS <= limit)
            return launch_mfma<M, 8, NST>(w, N, nb, xq, y, s, limit, 0);
    }
    const int64_t dlimit = al ? limit : 65536;
    const int S = pick_splits(N, al ? nb / 8 : nb, M, dlimit, al);
    const dim3 grid((unsigned)((N + WAVE - 1) / WAVE));
    const dim3 block(WAVE * S);
    const size_t partial_bytes = (size_t)S * M * WAVE * sizeof(float);
    const size_t stage_bytes = al ? (size_t)S * STAGE_BYTES : 0;
    const size_t lds = partial_bytes > stage_bytes ? partial_bytes : stage_bytes;
    if (al) {
        if (!allow_dynamic_lds((const void *)q4_0_mmvq_dot4_kernel<M, true>, limit))
            return BQ8_ERR_HIP;
        hipLaunchKernelGGL((q4_0_mmvq_dot4_kernel<M, true>), grid, block, lds, s,
                           (const uint8_t *)w, (int)N, nb, (const uint8_t *)xq, y);
    } else
        hipLaunchKernelGGL((q4_0_mmvq_dot4_kernel<M, false>), grid, block, lds, s,
                           (const uint8_t *)w, (int)N, nb, (const uint8_t *)xq, y);
    return launch_status();
}

} // namespace bq8

using namespace bq8;

#define BQ8_MMVQ_ENTRY(MM)                                                                           \
    BQ8_EXPORT bq8_status q4_0_mmvq_m##MM(const void *w, int64_t N, int64_t K, const void *xq,       \
                                          float *y, void *stream)                                    \
    {                                                                                                \
        return mmvq_launch<MM>(w, N, K, xq, y, stream);                                              \
    }

BQ8_MMVQ_ENTRY(1)
BQ8_MMVQ_ENTRY(2)
BQ8_MMVQ_ENTRY(3)
BQ8_MMVQ_ENTRY(4)
BQ8_MMVQ_ENTRY(5)
BQ8_MMVQ_ENTRY(6)
BQ8_MMVQ_ENTRY(7)
BQ8_MMVQ_ENTRY(8)
BQ8_MMVQ_ENTRY(9)
BQ8_MMVQ_ENTRY(10)
BQ8_MMVQ_ENTRY(11)
BQ8_MMVQ_ENTRY(12)
BQ8_MMVQ_ENTRY(13)
BQ8_MMVQ_ENTRY(14)
BQ8_MMVQ_ENTRY(15)
BQ8_MMVQ_ENTRY(16)
BQ8_MMVQ_ENTRY(17)

BQ8_EXPORT bq8_status q4_0_mmvq(const void *w, int64_t N, int64_t K, const void *xq, int64_t M,
                                float *y, void *stream)
{
    switch (M) {
    case 1: return q4_0_mmvq_m1(w, N, K, xq, y, stream);
    case 2: return q4_0_mmvq_m2(w, N, K, xq, y, stream);
    case 3: return q4_0_mmvq_m3(w, N, K, xq, y, stream);
    case 4: return q4_0_mmvq_m4(w, N, K, xq, y, stream);
    case 5: return q4_0_mmvq_m5(w, N, K, xq, y, stream);
    case 6: return q4_0_mmvq_m6(w, N, K, xq, y, stream);
    case 7: return q4_0_mmvq_m7(w, N, K, xq, y, stream);
    case 8: return q4_0_mmvq_m8(w, N, K, xq, y, stream);
    case 9: return q4_0_mmvq_m9(w, N, K, xq, y, stream);
    case 10: return q4_0_mmvq_m10(w, N, K, xq, y, stream);
    case 11: return q4_0_mmvq_m11(w, N, K, xq, y, stream);
    case 12: return q4_0_mmvq_m12(w, N, K, xq, y, stream);
    case 13: return q4_0_mmvq_m13(w, N, K, xq, y, stream);
    case 14: return q4_0_mmvq_m14(w, N, K, xq, y, stream);
    case 15: return q4_0_mmvq_m15(w, N, K, xq, y, stream);
    case 16: return q4_0_mmvq_m16(w, N, K, xq, y, stream);
    case 17: return q4_0_mmvq_m17(w, N, K, xq, y, stream);
    default: return BQ8_ERR_SHAPE;
    }
}
