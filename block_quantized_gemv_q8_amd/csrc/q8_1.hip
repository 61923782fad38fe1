// Q8_1 activation quantization and the verifier-layer glue that ends in a
// Q8_1 requantization (SiLU(gate)*up, and the weightless RMS step feeding the
// next layer).
//
// "Qwen3.6 27B B70 follow-up: Q8 activation cache, FP8 artifacts, MTP
// blocker", section "Q8_1 activation cache prototype": one exact Q8_1
// activation is reused by sibling Q4_0 matmuls.  "Qwen3.6 27B Q4_0
// DFlash/SYCL closure", "Closed or negative paths": the down-to-next-RMS/Q8
// boundary.  Block format and arithmetic: include/bq8.h.
//
// Layout on the device: 32 adjacent lanes own one 32-value block, one value
// per lane, so a wave64 quantizes two blocks; amax and sum(q) are butterfly
// reductions inside each 32-lane half.  The work is a few hundred KB at most,
// so the kernels are launch-latency bound, not bandwidth bound.
#include "bq8_dev.h"

namespace bq8 {

__global__ __launch_bounds__(256) void q8_1_quantize_kernel(const float *__restrict__ x,
                                                            int nblocks,
                                                            uint8_t *__restrict__ xq)
{
    const int gid = blockIdx.x * blockDim.x + threadIdx.x;
    const int blk = gid >> 5;
    const int j = gid & 31;
    const bool valid = blk < nblocks;
    const float v = valid ? x[(size_t)blk * QK + j] : 0.0f;
    q8_1_block_store(v, j, valid, xq + (size_t)blk * Q8_1_BYTES);
}

__global__ __launch_bounds__(256) void silu_mul_q8_1_kernel(const float *__restrict__ g,
                                                            const float *__restrict__ u,
                                                            int nblocks, float *__restrict__ h,
                                                            uint8_t *__restrict__ hq)
{
    const int gid = blockIdx.x * blockDim.x + threadIdx.x;
    const int blk = gid >> 5;
    const int j = gid & 31;
    const bool valid = blk < nblocks;
    float v = 0.0f;
    if (valid) {
        const size_t i = (size_t)blk * QK + j;
        const float gv = g[i];
        v = gv / (1.0f + expf(-gv)) * u[i];
        if (h)
            h[i] = v;
    }
    q8_1_block_store(v, j, valid, hq + (size_t)blk * Q8_1_BYTES);
}

// One workgroup of 1024 threads per row.  The 32 groups of 32 lanes own
// blocks g, g + 32, g + 64, ... (VPT blocks each); every thread loads its
// VPT values once, up front, into registers, so the row costs one memory
// round trip.  With nparts > 1 the row is the sum of nparts partial rows
// (part p at y + p * part_stride), added in part order; ysum, if given,
// receives it.  Sum of squares with a fixed reduction tree (per-thread
// partials in block order, a wave butterfly, the 16 waves in index order),
// so the result does not depend on scheduling; then each group quantizes its
// blocks from the registers.
constexpr int RMS_THREADS = 1024;
constexpr int RMS_GROUPS = RMS_THREADS / QK;
constexpr int RMS_MAX_K = RMS_GROUPS * 32 * QK; // 32 blocks per group

template <int VPT, int NP>
__global__ __launch_bounds__(RMS_THREADS) void rms_norm_q8_1_kernel(
    const float *__restrict__ y, size_t part_stride, int K, float eps, float *__restrict__ ysum,
    float *__restrict__ x, uint8_t *__restrict__ xq)
{
    __shared__ float wave_sums[RMS_THREADS / WAVE];
    // workgroup (m, q): row m; every workgroup of the row forms the row's sum
    // of squares the same way, and group grp writes and quantizes only its
    // block grp + RMS_GROUPS * q (five workgroups per row at K = 5120
    // instead of one quantizing five blocks per group in turn: 4.4 against
    // 5.6 us for the four-part sum; the bits are the same)
    const int m = blockIdx.x;
    const int q = blockIdx.y;
    const int nb = K / QK;
    const int grp = threadIdx.x >> 5;
    const int j = threadIdx.x & 31;
    const float *row = y + (size_t)m * K;
    // Every part's values are loaded before the first add (one memory round
    // trip) when they fit in registers, else one part after another;
    // out-of-range blocks read the row's last block and are dropped.
    float v[VPT];
    if constexpr (VPT * NP <= 64) {
        float t[NP][VPT];
#pragma unroll
        for (int p = 0; p < NP; ++p)
#pragma unroll
            for (int i = 0; i < VPT; ++i) {
                const int b = grp + RMS_GROUPS * i;
                t[p][i] = row[(size_t)p * part_stride + (b < nb ? b : nb - 1) * QK + j];
            }
#pragma unroll
        for (int i = 0; i < VPT; ++i) {
            v[i] = t[0][i];
#pragma unroll
            for (int p = 1; p < NP; ++p)
                v[i] += t[p][i];
        }
    } else {
#pragma unroll
        for (int i = 0; i < VPT; ++i) {
            const int b = grp + RMS_GROUPS * i;
            v[i] = row[(b < nb ? b : nb - 1) * QK + j];
        }
#pragma unroll 1
        for (int p = 1; p < NP; ++p)
#pragma unroll
            for (int i = 0; i < VPT; ++i) {
                const int b = grp + RMS_GROUPS * i;
                v[i] += row[(size_t)p * part_stride + (b < nb ? b : nb - 1) * QK + j];
            }
    }
#pragma unroll
    for (int i = 0; i < VPT; ++i)
        if (grp + RMS_GROUPS * i >= nb)
            v[i] = 0.0f;
    if (ysum) {
#pragma unroll
        for (int i = 0; i < VPT; ++i) {
            const int b = grp + RMS_GROUPS * i;
            if (i == q && b < nb)
                ysum[(size_t)m * K + b * QK + j] = v[i];
        }
    }
    if (!x && !xq)
        return; // uniform: only the sum was asked for
    float ss = 0.0f;
#pragma unroll
    for (int i = 0; i < VPT; ++i)
        ss = fmaf(v[i], v[i], ss);
#pragma unroll
    for (int off = 32; off > 0; off >>= 1)
        ss += __shfl_xor(ss, off, 64);
    if ((threadIdx.x & 63) == 0)
        wave_sums[threadIdx.x >> 6] = ss;
    __syncthreads();
    float tot = 0.0f;
#pragma unroll
    for (int w = 0; w < RMS_THREADS / WAVE; ++w)
        tot += wave_sums[w];
    const float inv = 1.0f / sqrtf(tot / (float)K + eps);

    uint8_t *out = xq ? xq + (size_t)m * nb * Q8_1_BYTES : nullptr;
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
        if (i != q) // uniform per workgroup
            continue;
        const int b = grp + RMS_GROUPS * i;
        const bool valid = b < nb;
        const float val = v[i] * inv;
        if (valid && x)
            x[(size_t)m * K + b * QK + j] = val;
        q8_1_block_store(val, j, valid && out, out ? out + (size_t)b * Q8_1_BYTES : nullptr);
    }
}

template <int VPT, int NP>
static void launch_rms_np(const float *y, int64_t M, int64_t K, float eps, float *ysum, float *x,
                          void *xq, hipStream_t s)
{
    const unsigned per_row = (unsigned)((K / QK + RMS_GROUPS - 1) / RMS_GROUPS);
    hipLaunchKernelGGL((rms_norm_q8_1_kernel<VPT, NP>), dim3((unsigned)M, per_row),
                       dim3(RMS_THREADS), 0, s, y, (size_t)(M * K), (int)K, eps, ysum, x,
                       (uint8_t *)xq);
}

template <int VPT>
static void launch_rms(const float *y, int nparts, int64_t M, int64_t K, float eps, float *ysum,
                       float *x, void *xq, hipStream_t s)
{
    switch (nparts) {
    case 1: launch_rms_np<VPT, 1>(y, M, K, eps, ysum, x, xq, s); break;
    case 2: launch_rms_np<VPT, 2>(y, M, K, eps, ysum, x, xq, s); break;
    case 3: launch_rms_np<VPT, 3>(y, M, K, eps, ysum, x, xq, s); break;
    case 4: launch_rms_np<VPT, 4>(y, M, K, eps, ysum, x, xq, s); break;
    case 5: launch_rms_np<VPT, 5>(y, M, K, eps, ysum, x, xq, s); break;
    case 6: launch_rms_np<VPT, 6>(y, M, K, eps, ysum, x, xq, s); break;
    case 7: launch_rms_np<VPT, 7>(y, M, K, eps, ysum, x, xq, s); break;
    default: launch_rms_np<VPT, 8>(y, M, K, eps, ysum, x, xq, s); break;
    }
}

static bq8_status rms_sum(const float *y, int64_t nparts, int64_t M, int64_t K, float eps,
                          float *ysum, float *x, void *xq, void *stream)
{
    if (!y || (!ysum && !x && !xq))
        return BQ8_ERR_NULL;
    if (M < 1 || M > 64 || K < QK || K % QK != 0 || K > RMS_MAX_K || !(eps > 0.0f) ||
        nparts < 1 || nparts > 8)
        return BQ8_ERR_SHAPE;
    if (!aligned(y, 4) || (xq && !aligned(xq, 4)) || (x && !aligned(x, 4)) ||
        (ysum && !aligned(ysum, 4)))
        return BQ8_ERR_ALIGN;
    (void)hipGetLastError();
    const int64_t per_group = (K / QK + RMS_GROUPS - 1) / RMS_GROUPS;
    const int np = (int)nparts;
    hipStream_t s = (hipStream_t)stream;
    if (per_group <= 2)
        launch_rms<2>(y, np, M, K, eps, ysum, x, xq, s);
    else if (per_group <= 4)
        launch_rms<4>(y, np, M, K, eps, ysum, x, xq, s);
    else if (per_group <= 8)
        launch_rms<8>(y, np, M, K, eps, ysum, x, xq, s);
    else if (per_group <= 16)
        launch_rms<16>(y, np, M, K, eps, ysum, x, xq, s);
    else
        launch_rms<32>(y, np, M, K, eps, ysum, x, xq, s);
    return launch_status();
}

} // namespace bq8

using namespace bq8;

BQ8_EXPORT bq8_status q8_1_quantize(const float *x, int64_t M, int64_t K, void *xq, void *stream)
{
    if (!x || !xq)
        return BQ8_ERR_NULL;
    if (M < 1 || K < QK || K % QK != 0 || M * K >= (int64_t(1) << 31))
        return BQ8_ERR_SHAPE;
    if (!aligned(x, 4) || !aligned(xq, 4))
        return BQ8_ERR_ALIGN;
    const int nblocks = (int)(M * K / QK);
    const int threads = 256;
    const int grid = (int)((M * K + threads - 1) / threads);
    (void)hipGetLastError();
    hipLaunchKernelGGL(q8_1_quantize_kernel, dim3(grid), dim3(threads), 0, (hipStream_t)stream, x,
                       nblocks, (uint8_t *)xq);
    return launch_status();
}

BQ8_EXPORT bq8_status silu_mul_q8_1(const float *g, const float *u, int64_t M, int64_t N, float *h,
                                    void *hq, void *stream)
{
    if (!g || !u || !hq)
        return BQ8_ERR_NULL;
    if (M < 1 || N < QK || N % QK != 0 || M * N >= (int64_t(1) << 31))
        return BQ8_ERR_SHAPE;
    if (!aligned(g, 4) || !aligned(u, 4) || !aligned(hq, 4) || (h && !aligned(h, 4)))
        return BQ8_ERR_ALIGN;
    const int nblocks = (int)(M * N / QK);
    const int threads = 256;
    const int grid = (int)((M * N + threads - 1) / threads);
    (void)hipGetLastError();
    hipLaunchKernelGGL(silu_mul_q8_1_kernel, dim3(grid), dim3(threads), 0, (hipStream_t)stream, g, u,
                       nblocks, h, (uint8_t *)hq);
    return launch_status();
}

BQ8_EXPORT bq8_status rms_norm_q8_1(const float *y, int64_t M, int64_t K, float eps, float *x,
                                    void *xq, void *stream)
{
    if (!xq)
        return BQ8_ERR_NULL;
    return rms_sum(y, 1, M, K, eps, nullptr, x, xq, stream);
}

BQ8_EXPORT bq8_status rms_norm_q8_1_sum(const float *yparts, int64_t nparts, int64_t M, int64_t K,
                                        float eps, float *y, float *x, void *xq, void *stream)
{
    return rms_sum(yparts, nparts, M, K, eps, y, x, xq, stream);
}
