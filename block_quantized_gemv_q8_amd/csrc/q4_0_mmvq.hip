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
// against block `b` of every activation row.
template <int M>
__device__ __forceinline__ void block_dot(uint32_t dbits, const uint32_t qs[4],
                                          const uint8_t *__restrict__ xq, int nb, int b,
                                          float acc[M])
{
    int lo[4], hi[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        lo[i] = nib_minus8(qs[i] & 0x0F0F0F0Fu);        // elements 4i .. 4i+3
        hi[i] = nib_minus8((qs[i] >> 4) & 0x0F0F0F0Fu); // elements 16+4i .. 16+4i+3
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

// ALIGNED: K % 256 == 0 and w 16-byte aligned, so every 8-block chunk of a
// row is a 16-byte-aligned 144-byte run read with nine 128-bit loads.
// Otherwise every block is read with 16-bit loads (always aligned).
template <int M, bool ALIGNED>
__global__ __launch_bounds__(1024) void q4_0_mmvq_dot4_kernel(const uint8_t *__restrict__ w,
                                                              int N, int nb,
                                                              const uint8_t *__restrict__ xq,
                                                              float *__restrict__ y)
{
    extern __shared__ float partial[]; // [S][M][64]
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int S = __builtin_amdgcn_readfirstlane(blockDim.x >> 6);
    int n = blockIdx.x * WAVE + lane;
    const bool active = n < N;
    if (!active)
        n = N - 1; // keep every load in bounds; the store is skipped
    const uint8_t *row = w + (size_t)n * nb * Q4_0_BYTES;

    float acc[M];
#pragma unroll
    for (int m = 0; m < M; ++m)
        acc[m] = 0.0f;

    if constexpr (ALIGNED) {
        const int nchunks = nb >> 3;
        for (int c = wave; c < nchunks; c += S) {
            const u32x4 *p = reinterpret_cast<const u32x4 *>(row + (size_t)c * 144);
            uint32_t wd[36];
#pragma unroll
            for (int i = 0; i < 9; ++i) {
                const u32x4 v = __builtin_nontemporal_load(p + i);
                wd[4 * i + 0] = v[0];
                wd[4 * i + 1] = v[1];
                wd[4 * i + 2] = v[2];
                wd[4 * i + 3] = v[3];
            }
            chunk_all<M>(wd, xq, nb, c * 8, acc, std::make_integer_sequence<int, 8>{});
        }
    } else {
        for (int b = wave; b < nb; b += S) {
            const uint16_t *p = reinterpret_cast<const uint16_t *>(row + (size_t)b * Q4_0_BYTES);
            uint32_t qs[4];
#pragma unroll
            for (int i = 0; i < 4; ++i)
                qs[i] = (uint32_t)p[1 + 2 * i] | ((uint32_t)p[2 + 2 * i] << 16);
            block_dot<M>(p[0], qs, xq, nb, b, acc);
        }
    }

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
        const int nn = blockIdx.x * WAVE + l;
        if (nn < N)
            y[(size_t)m * N + nn] = s;
    }
}

// Waves per workgroup: enough workgroups x waves to give every CU several
// waves, never more waves than K-units, at most 16 waves (1024 threads), and
// at most 128 partial rows of LDS (S * M <= 128).
static int pick_splits(int64_t N, int64_t units, int M)
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
    return (int)(s < 1 ? 1 : s);
}

template <int M>
static bq8_status mmvq_launch(const void *w, int64_t N, int64_t K, const void *xq, float *y,
                              void *stream)
{
    if (!w || !xq || !y)
        return BQ8_ERR_NULL;
    if (N < 1 || N >= (int64_t(1) << 31) || K < QK || K % QK != 0 ||
        N * (K / QK) * Q4_0_BYTES >= (int64_t(1) << 40) || K / QK >= (int64_t(1) << 31) ||
        (int64_t)M * K >= (int64_t(1) << 31))
        return BQ8_ERR_SHAPE;
    if (!aligned(w, 16) || !aligned(xq, 4) || !aligned(y, 4))
        return BQ8_ERR_ALIGN;
    const int nb = (int)(K / QK);
    const bool al = (K % 256 == 0);
    const int S = pick_splits(N, al ? nb / 8 : nb, M);
    const dim3 grid((unsigned)((N + WAVE - 1) / WAVE));
    const dim3 block(WAVE * S);
    const size_t lds = (size_t)S * M * WAVE * sizeof(float);
    (void)hipGetLastError();
    if (al)
        hipLaunchKernelGGL((q4_0_mmvq_dot4_kernel<M, true>), grid, block, lds, (hipStream_t)stream,
                           (const uint8_t *)w, (int)N, nb, (const uint8_t *)xq, y);
    else
        hipLaunchKernelGGL((q4_0_mmvq_dot4_kernel<M, false>), grid, block, lds, (hipStream_t)stream,
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
