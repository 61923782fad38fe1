// Read-only HBM probe: the practical streaming ceiling the weight-streaming
// kernels are measured against, beside the 8 TB/s nominal peak.  It reads a
// buffer once with 16-byte nontemporal loads, as the products read their
// weights, and folds every word into one XOR per wave, so it writes next to
// nothing.  Thread t of a grid of T threads reads words t, t + T, t + 2T, ...,
// U of them in flight per loop trip: each wave instruction reads one
// contiguous kilobyte and consecutive waves read adjacent kilobytes.
#include "bq8_dev.h"

namespace bq8 {

constexpr int PROBE_THREADS = 256;

template <int U>
__global__ __launch_bounds__(PROBE_THREADS) void hbm_read_probe_kernel(
    const u32x4 *__restrict__ buf, int64_t n16, uint32_t *__restrict__ out)
{
    const int64_t T = (int64_t)gridDim.x * PROBE_THREADS;
    int64_t i = (int64_t)blockIdx.x * PROBE_THREADS + threadIdx.x;
    uint32_t acc = 0u;
    for (; i + (U - 1) * T < n16; i += U * T) {
        u32x4 v[U];
#pragma unroll
        for (int u = 0; u < U; ++u)
            v[u] = __builtin_nontemporal_load(buf + i + u * T);
#pragma unroll
        for (int u = 0; u < U; ++u)
            acc ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
    }
    for (; i < n16; i += T) {
        const u32x4 v = __builtin_nontemporal_load(buf + i);
        acc ^= v[0] ^ v[1] ^ v[2] ^ v[3];
    }
    // XOR is order-free: the wave's fold needs no fixed tree
#pragma unroll
    for (int off = 32; off > 0; off >>= 1)
        acc ^= (uint32_t)__shfl_xor((int)acc, off, 64);
    if ((threadIdx.x & 63) == 0)
        out[(int64_t)blockIdx.x * (PROBE_THREADS / WAVE) + (threadIdx.x >> 6)] = acc;
}

} // namespace bq8

using namespace bq8;

BQ8_EXPORT bq8_status bq8_hbm_read_probe(const void *buf, int64_t bytes, int64_t workgroups,
                                         int64_t unroll, uint32_t *out, void *stream)
{
    if (!buf || !out)
        return BQ8_ERR_NULL;
    if (bytes < 16 || bytes % 16 != 0 || workgroups < 1 || workgroups > (int64_t(1) << 20) ||
        (unroll != 1 && unroll != 2 && unroll != 4 && unroll != 8))
        return BQ8_ERR_SHAPE;
    if (!aligned(buf, 16) || !aligned(out, 4))
        return BQ8_ERR_ALIGN;
    const int64_t n16 = bytes / 16;
    const u32x4 *b = static_cast<const u32x4 *>(buf);
    const dim3 grid((unsigned)workgroups), block(PROBE_THREADS);
    hipStream_t s = (hipStream_t)stream;
    (void)hipGetLastError();
    switch (unroll) {
    case 1: hipLaunchKernelGGL(hbm_read_probe_kernel<1>, grid, block, 0, s, b, n16, out); break;
    case 2: hipLaunchKernelGGL(hbm_read_probe_kernel<2>, grid, block, 0, s, b, n16, out); break;
    case 4: hipLaunchKernelGGL(hbm_read_probe_kernel<4>, grid, block, 0, s, b, n16, out); break;
    default: hipLaunchKernelGGL(hbm_read_probe_kernel<8>, grid, block, 0, s, b, n16, out); break;
    }
    return launch_status();
}
