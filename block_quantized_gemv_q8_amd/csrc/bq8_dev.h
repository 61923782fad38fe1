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

// max over each 32-lane group
__device__ __forceinline__ float group32_max(float a)
{
    a = fmaxf(a, as_f(dpp_move<DPP_SWAP1>(as_i(a))));
    a = fmaxf(a, as_f(dpp_move<DPP_SWAP2>(as_i(a))));
    a = fmaxf(a, as_f(dpp_move<DPP_HALF_MIRROR>(as_i(a))));
    a = fmaxf(a, as_f(dpp_move<DPP_MIRROR>(as_i(a))));
    return fmaxf(a, as_f(swizzle_xor16(as_i(a))));
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

// Quantize one 32-value Q8_1 block held one value per lane by 32 adjacent
// lanes (lane32 = lane index within the group).  Arithmetic in binary32:
// amax over the block, d = amax / 127 (correctly rounded division),
// q = x / d rounded half away from zero and clamped to +-127 (d == 0 gives
// q = 0).  Returns this lane's quant; `d` receives the binary32 scale (the
// block stores it rounded to fp16).
__device__ __forceinline__ int q8_1_block_quant(float v, float &d)
{
    const float a = group32_max(fabsf(v));
    d = a / 127.0f;
    int q = 0;
    if (d != 0.0f) {
        q = (int)roundf(v / d);
        q = q > 127 ? 127 : (q < -127 ? -127 : q);
    }
    return q;
}

// The Q8_1 block of q8_1_block_quant: every lane writes its quant, lane 0
// of the group writes d and s = d * sum(q) (binary32 product, then fp16).
// `blk` points at the block's 36 output bytes.
__device__ __forceinline__ void q8_1_block_store(float v, int lane32, bool valid, uint8_t *blk)
{
    float d;
    const int q = q8_1_block_quant(v, d);
    int s = row16_sum(q);
    s += swizzle_xor16(s);
    if (valid) {
        blk[4 + lane32] = (uint8_t)(int8_t)q;
        if (lane32 == 0) {
            float sf = d * (float)s;
            // s is the binary32 product rounded to fp16.  Without this
            // barrier the compiler turns multiply-then-convert into one
            // v_fma_mixlo_f16, which rounds the exact product to fp16 once
            // and differs from the twice-rounded value in rare ties.
            __asm__ volatile("" : "+v"(sf));
            *reinterpret_cast<uint32_t *>(blk) = f2h(d) | (f2h(sf) << 16);
        }
    }
}

inline bool aligned(const void *p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

// Leading bytes of a packed-launch workspace (q4_0_mmvq_packed_ws,
// q4_0_gate_up_silu_q8_1_packed_ws) that hold its counters, one uint32 per
// CU rounded up to 256 bytes; range sums follow.
inline int64_t pk_ws_count_bytes(int64_t cus) { return (cus * 4 + 255) / 256 * 256; }

inline bq8_status launch_status()
{
    return hipGetLastError() == hipSuccess ? BQ8_OK : BQ8_ERR_HIP;
}

} // namespace bq8
