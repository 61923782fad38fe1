// Internal device helpers shared by the libbq8 kernels (gfx950 / CDNA4).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "bq8.h"

// Entry points of the C ABI; everything else stays hidden.
#define BQ8_EXPORT extern "C" __attribute__((visibility("default")))

namespace bq8 {

constexpr int QK = 32;          // values per Q4_0 / Q8_1 block
constexpr int QK_K = 256;       // values per Q6_K superblock
constexpr int Q4_0_BYTES = 18;  // fp16 d + 16 nibble bytes
constexpr int Q8_1_BYTES = 36;  // fp16 d + fp16 s + 32 int8
constexpr int Q6_K_BYTES = 210; // ql[128] qh[64] scales[16] fp16 d
constexpr int WAVE = 64;

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(1))) void global_void_t;

// Order this wave's LDS writes before its reads of other lanes' data (a
// wave's LDS operations complete in order; the fences stop the compiler from
// moving accesses across).
__device__ __forceinline__ void wave_lds_sync()
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// s_waitcnt immediate for gfx9-family encodings: vmcnt = `vm` (6 bits split
// across two fields), expcnt and lgkmcnt left at their maximum (no wait).
constexpr int waitcnt_vmcnt(int vm)
{
    return (vm & 0xF) | (0x7 << 4) | (0xF << 8) | ((vm >> 4) << 14);
}

// Exact binary16 -> binary32 of raw bits (v_cvt_f32_f16).
__device__ __forceinline__ float h2f(uint32_t bits)
{
    _Float16 h = __builtin_bit_cast(_Float16, (uint16_t)(bits & 0xFFFFu));
    return (float)h;
}

// Round-to-nearest-even binary32 -> binary16 bits (v_cvt_f16_f32 under the
// default rounding mode; fp16 denormals are kept).
__device__ __forceinline__ uint32_t f2h(float f)
{
    return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)f);
}

// Signed int8 x4 dot product with int32 accumulate (v_dot4_i32_i8).
__device__ __forceinline__ int dot4(int a, int b, int c)
{
    return __builtin_amdgcn_sdot4(a, b, c, false);
}

// Four unsigned nibble values (0..15, one per byte) -> four signed bytes
// holding value - 8.  Adding 0x78 keeps every byte below 0x88, so no carry
// crosses a byte; flipping bit 7 then subtracts 128: (x + 120) - 128 = x - 8.
__device__ __forceinline__ int nib_minus8(uint32_t nibbles)
{
    return (int)((nibbles + 0x78787878u) ^ 0x80808080u);
}

// Lane exchanges for reductions whose result does not depend on the order
// of their operands (max of floats, sums of integers), so any exchange
// pattern gives the same bits.  Inside a row of 16 lanes they are DPP moves
// (ALU latency, no LDS round trip): swap neighbours, swap pairs, mirror in 8,
// mirror in 16 -- after the four steps every lane of the row holds the row's
// result.  The two rows of a 32-lane group then meet through ds_swizzle
// (lane ^ 16 inside each group of 32).  Every lane of the group must be
// active.
template <int CTRL>
__device__ __forceinline__ int dpp_move(int v)
{
    return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xF, 0xF, false);
}
constexpr int DPP_SWAP1 = 0xB1;      // quad_perm [1, 0, 3, 2]
constexpr int DPP_SWAP2 = 0x4E;      // quad_perm [2, 3, 0, 1]
constexpr int DPP_HALF_MIRROR = 0x141;
constexpr int DPP_MIRROR = 0x140;
__device__ __forceinline__ int swizzle_xor16(int v)
{
    return __builtin_amdgcn_ds_swizzle(v, 0x401F); // and 0x1F, or 0, xor 0x10
}
__device__ __forceinline__ float as_f(int v) { return __builtin_bit_cast(float, v); }
__device__ __forceinline__ int as_i(float v) { return __builtin_bit_cast(int, v); }

// max over each 32-lane group, for N independent values side by side
template <int N>
__device__ __forceinline__ void group32_max(float (&a)[N])
{
#pragma unroll
    for (int i = 0; i < N; ++i)
        a[i] = fmaxf(a[i], as_f(dpp_move<DPP_SWAP1>(as_i(a[i]))));
#pragma unroll
    for (int i = 0; i < N; ++i)
        a[i] = fmaxf(a[i], as_f(dpp_move<DPP_SWAP2>(as_i(a[i]))));
#pragma unroll
    for (int i = 0; i < N; ++i)
        a[i] = fmaxf(a[i], as_f(dpp_move<DPP_HALF_MIRROR>(as_i(a[i]))));
#pragma unroll
    for (int i = 0; i < N; ++i)
        a[i] = fmaxf(a[i], as_f(dpp_move<DPP_MIRROR>(as_i(a[i]))));
#pragma unroll
    for (int i = 0; i < N; ++i)
        a[i] = fmaxf(a[i], as_f(swizzle_xor16(as_i(a[i]))));
}

// integer sum over each row of 16 lanes
__device__ __forceinline__ int row16_sum(int s)
{
    s += dpp_move<DPP_SWAP1>(s);
    s += dpp_move<DPP_SWAP2>(s);
    s += dpp_move<DPP_HALF_MIRROR>(s);
    s += dpp_move<DPP_MIRROR>(s);
    return s;
}

// Quantize N 32-value Q8_1 blocks held by the 32 adjacent lanes of a group,
// value v[i] of block i in this lane (lane32 = lane index within the group),
// side by side.  Arithmetic in binary32: amax over the block, d = amax / 127
// (correctly rounded division), q = x / d rounded half away from zero and
// clamped to +-127 (d == 0 gives q = 0).  q[i] receives this lane's quant,
// d[i] the binary32 scale (the block stores it rounded to fp16).
template <int N>
__device__ __forceinline__ void q8_1_blocks_quant(const float (&v)[N], float (&d)[N], int (&q)[N])
{
    float a[N];
#pragma unroll
    for (int i = 0; i < N; ++i)
        a[i] = fabsf(v[i]);
    group32_max(a);
#pragma unroll
    for (int i = 0; i < N; ++i) {
        d[i] = a[i] / 127.0f;
        const bool live = d[i] != 0.0f;
        int qi = (int)roundf(v[i] / (live ? d[i] : 1.0f));
        qi = qi > 127 ? 127 : (qi < -127 ? -127 : qi);
        q[i] = live ? qi : 0;
    }
}

__device__ __forceinline__ int q8_1_block_quant(float v, float &d)
{
    const float vv[1] = {v};
    float dd[1];
    int q[1];
    q8_1_blocks_quant(vv, dd, q);
    d = dd[0];
    return q[0];
}

// The Q8_1 blocks of q8_1_blocks_quant: every lane writes its quant, lane 0
// of the group writes d and s = d * sum(q) (binary32 product, then fp16).
// blk[i] points at block i's 36 output bytes; blocks with valid[i] false
// are computed and not stored.
template <int N>
__device__ __forceinline__ void q8_1_blocks_store(const float (&v)[N], int lane32,
                                                  const bool (&valid)[N], uint8_t *const (&blk)[N])
{
    float d[N];
    int q[N];
    q8_1_blocks_quant(v, d, q);
    int s[N];
#pragma unroll
    for (int i = 0; i < N; ++i)
        s[i] = row16_sum(q[i]);
#pragma unroll
    for (int i = 0; i < N; ++i)
        s[i] += swizzle_xor16(s[i]);
#pragma unroll
    for (int i = 0; i < N; ++i) {
        if (!valid[i])
            continue;
        blk[i][4 + lane32] = (uint8_t)(int8_t)q[i];
        if (lane32 == 0) {
            float sf = d[i] * (float)s[i];
            // s is the binary32 product rounded to fp16.  Without this
            // barrier the compiler turns multiply-then-convert into one
            // v_fma_mixlo_f16, which rounds the exact product to fp16 once
            // and differs from the twice-rounded value in rare ties.
            __asm__ volatile("" : "+v"(sf));
            *reinterpret_cast<uint32_t *>(blk[i]) = f2h(d[i]) | (f2h(sf) << 16);
        }
    }
}

__device__ __forceinline__ void q8_1_block_store(float v, int lane32, bool valid, uint8_t *blk)
{
    const float vv[1] = {v};
    const bool ok[1] = {valid};
    uint8_t *const b[1] = {blk};
    q8_1_blocks_store(vv, lane32, ok, b);
}

inline bool aligned(const void *p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

inline bq8_status launch_status()
{
    return hipGetLastError() == hipSuccess ? BQ8_OK : BQ8_ERR_HIP;
}

} // namespace bq8
