// Offline-packed Q4_0 and its M = 1..17 matrix-vector product.
//
// "Qwen3.6 27B Q4_0 DFlash/SYCL closure", "What materially worked": the
// verifier's width-6 gate/up and down projections ran on offline-packed
// weights.  This pack keeps the 18 bytes per 32 weights and regroups them so
// that the MFMA kernel's weight operand arrives straight from memory into
// registers: in each 16-row tile, the 16 rows' nibbles for one (4-block
// group, lane group) are 256 contiguous bytes, so one wave load instruction
// (16 bytes per lane) reads one contiguous kilobyte and every lane receives
// exactly the nibbles of its MFMA B operand -- no LDS staging, no byte
// realignment of the 18-byte blocks.  Layout (K % 512 == 0; include/bq8.h):
//
//   tile of row n: n0 = 16*(n/16), r = n - n0, rows_t = min(16, N - n0)
//   QS plane (N*nb*16 bytes at 0): element j of block b of row n, with
//     h = j/16, jj = j%16, is nibble (jj >= 8 ? high : low) of byte
//       n0*nb*16 + u*(4*rows_t*16) + (g*rows_t + r)*16 + 8*v + jj%8
//     where u = b/4, v = (b%4)/2, g = 2*(b%2) + h;
//   D plane (N*nb*2 bytes at N*nb*16): scale of block b of row n at element
//       n0*nb + ((b/16)*2 + b%2)*rows_t*8 + r*8 + (b%16)/2.
//
// The product is the one of q4_0_mmvq.hip (block-diagonal int8 MFMA, exact
// per-block integer dots, d_w * d_x scaling and binary32 accumulation in a
// fixed order); only where the operands come from differs.  Three launches
// share its main loop (pk_accumulate): the product (q4_0_mmvq_packed), the
// same product with K cut into ranges written as partial sums
// (q4_0_mmvq_packed_split, for shapes with few row tiles), and the joint
// gate/up launch with the SiLU*up + Q8_1 epilogue
// (q4_0_gate_up_silu_q8_1_packed).
#include "bq8_dev.h"
#include "bq8_host.h"

namespace bq8 {

constexpr int PK_TILE = 16;
constexpr int PK_CB = 8; // blocks per chunk: two 4-block groups

__device__ __forceinline__ int pk_tile(int n, int N, int &n0, int &r)
{
    n0 = n / PK_TILE * PK_TILE;
    r = n - n0;
    return (N - n0 < PK_TILE) ? N - n0 : PK_TILE;
}

// ------------------------------------------------------------- packing
// One thread per (row, block): the block's 32 codes go to two 8-byte pieces
// (one per half), its scale to the D plane.
__global__ __launch_bounds__(256) void q4_0_pack_kernel(const uint8_t *__restrict__ w, int N,
                                                        int nb, uint8_t *__restrict__ QS,
                                                        uint16_t *__restrict__ D)
{
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= (int64_t)N * nb)
        return;
    const int n = (int)(i / nb), b = (int)(i - (int64_t)n * nb);
    int n0, r;
    const int rows_t = pk_tile(n, N, n0, r);
    const uint8_t *blk = w + i * Q4_0_BYTES;
    uint8_t qs[16];
#pragma unroll
    for (int j = 0; j < 16; ++j)
        qs[j] = blk[2 + j];
    const int u = b / 4, v = (b % 4) / 2;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        // element 16h + jj: code of qs[jj] (low nibble, h = 0) or (high, h = 1)
        uint32_t word[2] = {0u, 0u};
#pragma unroll
        for (int jj = 0; jj < 16; ++jj) {
            const uint32_t code = h ? (qs[jj] >> 4) : (qs[jj] & 0x0Fu);
            const int byte = jj % 8;
            const int shift = 8 * (byte % 4) + (jj >= 8 ? 4 : 0);
            word[byte / 4] |= code << shift;
        }
        const int g = 2 * (b % 2) + h;
        uint32_t *dst = reinterpret_cast<uint32_t *>(
            QS + (int64_t)n0 * nb * 16 + (int64_t)u * (4 * rows_t * 16) + (g * rows_t + r) * 16 +
            8 * v);
        dst[0] = word[0];
        dst[1] = word[1];
    }
    D[(int64_t)n0 * nb + ((b / 16) * 2 + b % 2) * rows_t * 8 + r * 8 + (b % 16) / 2] =
        (uint16_t)(blk[0] | (blk[1] << 8));
}

// --------------------------------------------------------------- product
// One workgroup owns a 16-row tile; its S waves take the tile's 8-block
// chunks round-robin.  Per chunk a wave loads, straight into registers, its
// lane's 2 x 16 bytes of packed nibbles and 8 bytes of scales, and stages the
// chunk's M Q8_1 activation blocks in LDS (global_load_lds, 16 bytes per
// lane) together with their scales as binary32.  The registers are double
// buffered: chunk k+1 is issued before chunk k is computed, and the only
// wait in the loop is for chunk k itself.
//
// MFMA mapping (v_mfma_i32_16x16x64_i8, one per block pair (2t, 2t+1) of the
// chunk): B lane l holds weight row c16 = l%16, k range 16*(l/16) .. +15,
// i.e. half h = (l/16)%2 of block 2t + hb, hb = l/32 -- exactly the lane's
// 8 packed bytes, unpacked to 16 signed bytes 16*(q - 8); A row c16 holds
// activation row m = c16%8 (+8s) for block c16/8, zero outside its block's k
// range (lanes outside it read a zeroed LDS row).  Results are 16x the exact
// dots (scaled by 1/16 at the end, exact).
//
// Which activation row an A row holds: MFMA s of a block pair covers rows
// 2X*s .. 2X*s + 2X - 1 of each block, X = ceil(M / (2*MS)) of them per
// 4-row group.  A row c16 (group g = c16/4 = 2*block + h, position
// x = c16%4) holds row m = 2X*s + X*h + x when x < X (pk_row), and output
// lane l keeps that row's sum in acc[..][s][x] for its h = (l/16)%2.  With
// X < 4 the positions x >= X are never formed (M = 6: X = 3; M = 1, 2:
// X = 1; M = 17: X = 3 in 3 MFMAs instead of 4 positions); M = 8 and 16 give
// the plain m = 8s + 4h + x.  Which row sits where does not change any sum.
template <int M>
struct PkShape {
    static constexpr int MS = (M + 7) / 8;
    static constexpr int X = (M + 2 * MS - 1) / (2 * MS);    // rows per 4-row group
    static constexpr int XRUN = PK_CB * Q8_1_BYTES;          // activation bytes per row per chunk
    static constexpr int XPIECES = M * XRUN / 16;
    static constexpr int LOADS = (XPIECES + WAVE - 1) / WAVE; // DMA instructions per chunk
    static constexpr int DXOFF = LOADS * WAVE * 16;           // f32 d_x [PK_CB][8*MS]
    static constexpr int STAGE = DXOFF + PK_CB * 8 * MS * 4;
    static constexpr int ZOFF = 2 * STAGE;                    // XRUN zero bytes after the ring
    static constexpr int WAVE_LDS = ZOFF + XRUN;
};

// Activation row of (MFMA s, 4-row group half h, position x); it exists when
// x < X and the row is below M.
template <int M>
__device__ __forceinline__ int pk_row(int s, int h, int x)
{
    return 2 * PkShape<M>::X * s + PkShape<M>::X * h + x;
}
template <int M>
__device__ __forceinline__ bool pk_row_ok(int s, int h, int x)
{
    return x < PkShape<M>::X && pk_row<M>(s, h, x) < M;
}

// acc[s][x] += 16 I * d_w * d_x for one tile's block pair: Dm[s] the MFMA
// products (16x the exact integer dots), dbits the lane's block's fp16 d_w,
// dx[s] the activation rows' d_x.
template <int M>
__device__ __forceinline__ void pk_scale_tile(float (&acc)[PkShape<M>::MS][4],
                                              const i32x4 (&Dm)[PkShape<M>::MS], uint32_t dbits,
                                              const f32x4 (&dx)[PkShape<M>::MS])
{
    const float dw = h2f(dbits);
#pragma unroll
    for (int s = 0; s < PkShape<M>::MS; ++s)
#pragma unroll
        for (int x = 0; x < PkShape<M>::X; ++x)
            acc[s][x] = fmaf((float)Dm[s][x], dw * dx[s][x], acc[s][x]);
}

// The main loop shared by the products: this wave's partial sums over its
// chunks for NT 16-row tiles that read the same activation rows.  Tile i's
// packed nibbles start at tile[i], its scales at dtile[i]; every tile has
// rows_t rows; chunk c of tile i starts at tile[i] + c * chunk_stride bytes
// and its scales at dtile[i] + (c/2) * dgroup_stride elements (+4 for odd
// c).  The wave sums chunks c0 + wave, c0 + wave + S, ... below c0 + nc.  The activations are staged once per chunk and each A operand feeds NT
// MFMAs.  ring is this wave's LDS (at least PkShape<M>::WAVE_LDS bytes).
// acc[i][s][x] of lanes l and l + 32 are the two blocks' shares of the sum
// for weight row l%16 of tile i and activation row pk_row(s, (l/16)%2, x), 16x
// the exact value.
template <int M, int NT>
__device__ __forceinline__ void pk_accumulate(const uint8_t *const (&tile)[NT],
                                              const uint16_t *const (&dtile)[NT], int rows_t,
                                              size_t chunk_stride, size_t dgroup_stride, int nb,
                                              int c0, int nc, const uint8_t *__restrict__ xq,
                                              uint8_t *ring, float (&acc)[NT][PkShape<M>::MS][4])
{
    using SH = PkShape<M>;
    constexpr int MS = SH::MS, LOADS = SH::LOADS;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int S = __builtin_amdgcn_readfirstlane(blockDim.x >> 6);
    uint8_t *zero = ring + SH::ZOFF;

    const int c16 = lane & 15;
    const int g = lane >> 4;
    const int h = g & 1;
    const int hb = g >> 1;
    const int r = c16 < rows_t ? c16 : rows_t - 1; // ragged tile: repeat the last row
    bool a_on[MS];
    uint32_t aoff[MS];
#pragma unroll
    for (int s = 0; s < MS; ++s) {
        const int ha = (c16 >> 2) & 1, xa = c16 & 3;
        const int m = pk_row<M>(s, ha, xa);
        a_on[s] = ((c16 >> 3) == hb) && pk_row_ok<M>(s, ha, xa);
        aoff[s] = (uint32_t)(a_on[s] ? m : 0) * SH::XRUN;
    }
    // Addresses are a uniform per-chunk base (scalar registers) plus a fixed
    // 32-bit per-lane offset, so the loads take the saddr + voffset form.
    // activation pieces: piece p = 64j + lane of a chunk is 16 bytes of row m
    uint32_t xoff[LOADS];
#pragma unroll
    for (int j = 0; j < LOADS; ++j) {
        const int p = j * WAVE + lane;
        if (p < SH::XPIECES) {
            const int m = p / (SH::XRUN / 16);
            const int q = p - m * (SH::XRUN / 16);
            xoff[j] = (uint32_t)m * (uint32_t)nb * Q8_1_BYTES + 16u * (uint32_t)q;
        } else {
            xoff[j] = 0u; // padding slot: a valid address, never read back
        }
    }
    // weights: this lane's piece of 4-block group u at tile + u * group_bytes + woff
    const uint32_t woff = (uint32_t)(g * rows_t + r) * 16u;
    const size_t group_bytes = (size_t)4 * rows_t * 16;
    // scales: this lane's blocks (parity hb) of 16-block group q at
    // dtile + q * dgroup_stride + doff, doff in elements
    const uint32_t doff = (uint32_t)(hb * rows_t + r) * 8u;

    auto issue = [&](int c, int st, u32x4(&wv)[NT][2], uint32_t(&dv)[NT][2]) {
        uint8_t *dst = ring + st * SH::STAGE;
        const uint8_t *xc = xq + (size_t)c * SH::XRUN;
#pragma unroll
        for (int j = 0; j < LOADS; ++j)
            __builtin_amdgcn_global_load_lds((global_void_t *)(xc + xoff[j]),
                                             (lds_void_t *)(dst + j * WAVE * 16), 16, 0, 0);
#pragma unroll
        for (int i = 0; i < NT; ++i) {
            const uint8_t *wc0 = tile[i] + (size_t)c * chunk_stride;
            wv[i][0] = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(wc0 + woff));
            wv[i][1] = __builtin_nontemporal_load(
                reinterpret_cast<const u32x4 *>(wc0 + group_bytes + woff));
        }
#pragma unroll
        for (int i = 0; i < NT; ++i) {
            // blocks 8c + 2i + hb, i = 0..3: elements 4*(c%2) .. +3 of group c/2
            const uint16_t *dc = dtile[i] + (size_t)(c >> 1) * dgroup_stride + (c & 1) * 4;
            const uint32_t *dq = reinterpret_cast<const uint32_t *>(dc + doff);
            dv[i][0] = dq[0];
            dv[i][1] = dq[1];
        }
    };

#pragma unroll
    for (int i = 0; i < NT; ++i)
#pragma unroll
        for (int s = 0; s < MS; ++s)
#pragma unroll
            for (int x = 0; x < 4; ++x)
                acc[i][s][x] = 0.0f;

    auto compute = [&](int st, const u32x4(&wv)[NT][2], const uint32_t(&dv)[NT][2]) {
        const uint8_t *stage = ring + st * SH::STAGE;
        float *dxs = reinterpret_cast<float *>(ring + st * SH::STAGE + SH::DXOFF);
        // d_x of the chunk's blocks as f32: dxs[b*8*MS + m], 0 past M
#pragma unroll
        for (int i = lane; i < PK_CB * 8 * MS; i += WAVE) {
            // entry 8s + 4h + x of block b: d of row pk_row(s, h, x)
            const int b = i / (8 * MS), j = i - (i / (8 * MS)) * (8 * MS);
            const int sj = j >> 3, hj = (j >> 2) & 1, xj = j & 3;
            const bool ok = pk_row_ok<M>(sj, hj, xj);
            const uint16_t bits = *reinterpret_cast<const uint16_t *>(
                stage + (ok ? pk_row<M>(sj, hj, xj) : 0) * SH::XRUN + b * Q8_1_BYTES);
            dxs[i] = ok ? h2f(bits) : 0.0f;
        }
        // per-lane parts of the LDS addresses, folded once per chunk: block
        // offset 36*hb, element half 16*h past the 4 header bytes
        const uint8_t *abase[MS];
#pragma unroll
        for (int s = 0; s < MS; ++s)
            abase[s] = (a_on[s] ? stage + aoff[s] : zero) + Q8_1_BYTES * hb + 4 + 16 * h;
        const float *dxl = dxs + hb * 8 * MS + 4 * h;
        wave_lds_sync();
#pragma unroll
        for (int t = 0; t < PK_CB / 2; ++t) {
            // this lane's block within the chunk is 2t + hb
            i32x4 A[MS];
            f32x4 dx[MS];
#pragma unroll
            for (int s = 0; s < MS; ++s) {
                const uint32_t *xb =
                    reinterpret_cast<const uint32_t *>(abase[s] + 2 * t * Q8_1_BYTES);
                A[s][0] = (int)xb[0];
                A[s][1] = (int)xb[1];
                A[s][2] = (int)xb[2];
                A[s][3] = (int)xb[3];
                dx[s] = *reinterpret_cast<const f32x4 *>(dxl + 2 * t * 8 * MS + 8 * s);
            }
            // every tile's MFMAs first, then their scaling, so that the
            // products' latency overlaps the next tile's unpacking -- except
            // with four tiles and two or more MFMAs a tile (the joint launch
            // from M = 9), where holding every product costs the registers of
            // a wave per SIMD: there each tile is scaled after its own MFMAs
            // (joint M = 9 25.7 -> 23.7 us, 168 VGPRs instead of 180; the
            // order of the additions is the same)
            constexpr bool EACH = NT >= 4 && MS >= 2;
            i32x4 Dm[EACH ? 1 : NT][MS];
#pragma unroll
            for (int i = 0; i < NT; ++i) {
                const int di = EACH ? 0 : i;
                // 8 packed bytes: byte i < 4 holds elements i (low) and 8+i
                // (high), byte 4+i elements 4+i and 12+i, of the lane's
                // 16-element range
                const uint32_t w0 = wv[i][t >> 1][2 * (t & 1)];
                const uint32_t w1 = wv[i][t >> 1][2 * (t & 1) + 1];
                i32x4 B;
                B[0] = (int)(((w0 << 4) & 0xF0F0F0F0u) ^ 0x80808080u);
                B[1] = (int)(((w1 << 4) & 0xF0F0F0F0u) ^ 0x80808080u);
                B[2] = (int)((w0 & 0xF0F0F0F0u) ^ 0x80808080u);
                B[3] = (int)((w1 & 0xF0F0F0F0u) ^ 0x80808080u);
#pragma unroll
                for (int s = 0; s < MS; ++s)
                    Dm[di][s] = __builtin_amdgcn_mfma_i32_16x16x64_i8(A[s], B, (i32x4){0, 0, 0, 0},
                                                                      0, 0, 0);
                if constexpr (EACH)
                    pk_scale_tile<M>(acc[i], Dm[0], dv[i][t >> 1] >> (16 * (t & 1)), dx);
            }
            if constexpr (!EACH) {
#pragma unroll
                for (int i = 0; i < NT; ++i)
                    pk_scale_tile<M>(acc[i], Dm[i], dv[i][t >> 1] >> (16 * (t & 1)), dx);
            }
        }
        wave_lds_sync();
    };

    if (wave < nc) {
        const int mine = (nc - wave + S - 1) / S;
        u32x4 wn[NT][2], wc[NT][2];
        uint32_t dn[NT][2], dc[NT][2];
        issue(c0 + wave, 0, wn, dn);
        // The zero row is first read by the first compute, so it is written
        // after the first issue: nothing but address setup goes before the
        // loads (ffn_up M = 6 10.69 -> 10.51 us, down 4 K ranges M = 1
        // 10.49 -> 10.12 us; no M slower).
        for (int i = lane; i < SH::XRUN / 4; i += WAVE)
            reinterpret_cast<uint32_t *>(zero)[i] = 0u;
        for (int k = 0; k < mine; ++k) {
            // Taking chunk k out of the prefetch registers waits for exactly
            // its loads (nothing younger is in flight yet); the explicit wait
            // also covers its activation DMA, which the compiler does not track.
#pragma unroll
            for (int i = 0; i < NT; ++i) {
                wc[i][0] = wn[i][0];
                wc[i][1] = wn[i][1];
                dc[i][0] = dn[i][0];
                dc[i][1] = dn[i][1];
            }
            __builtin_amdgcn_s_waitcnt(waitcnt_vmcnt(0));
            // no prefetch past the wave's last chunk: a repeated chunk would
            // be fetched from HBM again (the weight loads are nontemporal).
            // The loads go out at raised wave priority, so that other waves'
            // compute on the SIMD does not hold them back.
            __builtin_amdgcn_s_setprio(3);
            if (k + 1 < mine)
                issue(c0 + wave + S * (k + 1), (k + 1) & 1, wn, dn);
            __builtin_amdgcn_s_setprio(0);
            compute(k & 1, wc, dc);
        }
    }
}

// LDS bytes per wave: its ring, which after the wave's last chunk holds its
// sums -- float [NT][2][MS*4][32], half h = lane / 32 holding lane 32h + l's
// sums, the two blocks of each pair.  Only the wave itself touches its ring,
// and its last chunk's reads and copies are done before it writes there, so
// no barrier is needed before the write.
template <int M, int NT>
constexpr int pk_wave_stride()
{
    constexpr int sums = NT * 2 * PkShape<M>::MS * 4 * 32 * 4;
    return PkShape<M>::WAVE_LDS > sums ? PkShape<M>::WAVE_LDS : sums;
}

template <int NT, int MS>
__device__ __forceinline__ void pk_store_partials(const float (&acc)[NT][MS][4], uint8_t *ring,
                                                  int lane)
{
    constexpr int SLOTS = MS * 4;
    float *p = reinterpret_cast<float *>(ring);
    const int half = lane >> 5, l = lane & 31;
#pragma unroll
    for (int i = 0; i < NT; ++i)
#pragma unroll
        for (int s = 0; s < MS; ++s)
#pragma unroll
            for (int x = 0; x < 4; ++x)
                p[((i * 2 + half) * SLOTS + s * 4 + x) * 32 + l] = acc[i][s][x];
}

// Wave v's sum for one (tile, slot, lane) with its pair added, lane l then
// l + 32, as one value.
template <int NT, int MS>
__device__ __forceinline__ float pk_partial_sum(const uint8_t *smem, int stride, int v, int i,
                                                int slot, int l)
{
    constexpr int SLOTS = MS * 4;
    const float *p = reinterpret_cast<const float *>(smem + (size_t)v * stride) +
                     (i * 2 * SLOTS + slot) * 32 + l;
    return p[0] + p[SLOTS * 32];
}

// The meeting's reads: the P range sums at p, p + stride, ... (agent-scope
// atomic loads, all issued before the first add; P <= 4), added in range
// order from +0.
__device__ __forceinline__ float pk_range_sum(const float *p, size_t stride, int P)
{
    float v[4];
#pragma unroll
    for (int r = 0; r < 4; ++r)
        v[r] = __hip_atomic_load(p + (size_t)(r < P ? r : 0) * stride, __ATOMIC_RELAXED,
                                 __HIP_MEMORY_SCOPE_AGENT);
    float sacc = 0.0f;
#pragma unroll
    for (int r = 0; r < 4; ++r)
        if (r < P)
            sacc += v[r];
    return sacc;
}

// Two such sums, all 2P loads issued first.
__device__ __forceinline__ void pk_range_sum2(const float *p, const float *q, size_t stride,
                                              int P, float &sp, float &sq)
{
    float v[4], w[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const size_t o = (size_t)(r < P ? r : 0) * stride;
        v[r] = __hip_atomic_load(p + o, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        w[r] = __hip_atomic_load(q + o, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    sp = 0.0f;
    sq = 0.0f;
#pragma unroll
    for (int r = 0; r < 4; ++r)
        if (r < P) {
            sp += v[r];
            sq += w[r];
        }
}

// y[m][n] for one 16-row tile; the tile's S waves take its 8-block chunks
// round-robin and their sums are added in wave order.  Workgroup b works in
// one of three ways:
//   nsplit > 1: range p = b / tiles of tile b % tiles (chunks p*C/nsplit ..
//     (p+1)*C/nsplit - 1 of the C = nb/8), its sums to y + p*M*N;
//   b < whole: the whole tile b, its sums to y;
//   otherwise (CU balance, nsplit = 1): range j % P of tile whole + j / P,
//     j = b - whole, with the tile's chunks cut into P ranges as above.  The
//     tiles past the last multiple of the CU count are cut this way so that
//     every CU gets the same work.  Their workgroups come last: the whole
//     tiles, the longer work, start first.  A cut range's sums go to
//     ws_sum[j][SLOTS*32]; the workgroup then counts itself in
//     ws_count[j / P], and the one that brings the count to P adds the P
//     range sums in range order, writes y and sets the count back to 0 for
//     the next call.
// The range sums and the count are agent-scope atomic stores, loads and adds
// (global_store / global_load with the device-scope bit, global_atomic_add),
// coherent across the XCDs' L2 caches without an L2 write-back: each writer
// waits for its stores to complete (vmcnt(0)) before it counts itself, and
// the last workgroup issues its loads after its count has returned.
//
// KIND fixes at compile time what a workgroup has to decide, since every
// instruction before a wave's first load delays the whole stream.  With
// N % 16 == 0 every tile is full and the chunk strides are constants
// (PK_FULL_WHOLE: workgroup b is tile b; PK_FULL_SPLIT: the split launch).
// PK_ANY decides all of it at run time: a ragged last tile, the cut
// launch, and every launch at M >= 9.  Measured against PK_ANY (two builds
// in one process, interleaved), ffn_up: M = 1 / 6 / 8 10.29 / 10.66 / 10.97
// against 10.42 / 11.13 / 11.28 us; down, 4 K ranges: M = 1 10.59 against
// 10.74 us.  At M >= 9 the specialized kernels were slower (ffn_up M = 17
// 19.24 against 18.30 us), so those stay general.  The results are bitwise
// those of PK_ANY: only address arithmetic differs.
enum { PK_ANY = 0, PK_FULL_WHOLE = 1, PK_FULL_SPLIT = 2 };

template <int M, int KIND, int NT>
__global__ __launch_bounds__(512) void q4_0_mmvq_packed_kernel(
    const uint8_t *__restrict__ QS, const uint16_t *__restrict__ D, int N, int nb, int nsplit,
    int P, int whole, const uint8_t *__restrict__ xq, float *__restrict__ y,
    float *__restrict__ ws_sum, uint32_t *__restrict__ ws_count)
{
    constexpr int MS = PkShape<M>::MS;
    constexpr int SLOTS = MS * 4;
    constexpr int UNIT = NT * SLOTS * 32; // sums of one workgroup's unit (NT tiles)
    constexpr int STRIDE = pk_wave_stride<M, NT>();
    // NT > 1 is launched only with N % (16 NT) == 0
    constexpr bool FULL = KIND != PK_ANY || NT > 1;
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int S = __builtin_amdgcn_readfirstlane(blockDim.x >> 6);
    const int units = (N + PK_TILE * NT - 1) / (PK_TILE * NT);
    const int nch = nb / PK_CB;
    int t = blockIdx.x, c0 = 0, c1 = nch, j = -1;
    if (KIND == PK_FULL_SPLIT || (KIND == PK_ANY && nsplit > 1)) {
        // p * nch < 2^21 (p < 8, nch <= 2^18): 32-bit arithmetic suffices
        const int p = (int)blockIdx.x / units;
        t = blockIdx.x - p * units;
        c0 = p * nch / nsplit;
        c1 = (p + 1) * nch / nsplit;
        y += (size_t)p * M * N;
    } else if (KIND == PK_ANY) {
        if ((int)blockIdx.x >= whole) {
            j = blockIdx.x - whole;
            const int p = j % P;
            t = whole + j / P;
            c0 = p * nch / P;
            c1 = (p + 1) * nch / P;
        }
    }
    const int n0 = t * PK_TILE * NT;
    const int rows_t = FULL ? PK_TILE : ((N - n0 < PK_TILE) ? N - n0 : PK_TILE);
    const uint8_t *tile[NT];
    const uint16_t *dtile[NT];
#pragma unroll
    for (int i = 0; i < NT; ++i) {
        tile[i] = QS + (size_t)(n0 + PK_TILE * i) * nb * 16;
        dtile[i] = D + (size_t)(n0 + PK_TILE * i) * nb;
    }
    float acc[NT][MS][4];
    pk_accumulate<M, NT>(tile, dtile, rows_t, (size_t)8 * rows_t * 16, (size_t)2 * rows_t * 8, nb,
                         c0, c1 - c0, xq, smem + (size_t)wave * STRIDE, acc);
    pk_store_partials<NT, MS>(acc, smem + (size_t)wave * STRIDE, lane);
    __syncthreads();
    // output idx = (i * SLOTS + slot) * 32 + l, slot = 4s + x: tile i,
    // activation row pk_row(s, l/16, x), weight row n0 + 16i + l%16
    auto wave_sum = [&](int idx) {
        const int i = idx / (SLOTS * 32), slot = (idx >> 5) % SLOTS, l = idx & 31;
        float sacc = 0.0f;
        for (int v = 0; v < S; ++v)
            sacc += pk_partial_sum<NT, MS>(smem, STRIDE, v, i, slot, l);
        return sacc;
    };
    auto store_y = [&](int idx, float sacc) {
        const int i = idx / (SLOTS * 32), slot = (idx >> 5) % SLOTS, l = idx & 31;
        const int m = pk_row<M>(slot >> 2, l >> 4, slot & 3);
        const int nn = n0 + PK_TILE * i + (l & 15);
        if (pk_row_ok<M>(slot >> 2, l >> 4, slot & 3) && nn < N)
            y[(size_t)m * N + nn] = sacc * 0.0625f;
    };
    if (KIND == PK_FULL_WHOLE || KIND == PK_FULL_SPLIT || j < 0) {
        for (int idx = threadIdx.x; idx < UNIT; idx += blockDim.x)
            store_y(idx, wave_sum(idx));
        return;
    }
    float *rsum = ws_sum + (size_t)(j - j % P) * UNIT; // the unit's P range sums
    for (int idx = threadIdx.x; idx < UNIT; idx += blockDim.x)
        __hip_atomic_store(rsum + (size_t)(j % P) * UNIT + idx, wave_sum(idx), __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    // the partial sums have been read: wave 0's first LDS word then tells the
    // workgroup whether it arrived last
    int *last = reinterpret_cast<int *>(smem);
    if (threadIdx.x == 0)
        *last = __hip_atomic_fetch_add(ws_count + j / P, 1u, __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT) == (uint32_t)(P - 1);
    __syncthreads();
    if (!*last)
        return;
    for (int idx = threadIdx.x; idx < UNIT; idx += blockDim.x)
        store_y(idx, pk_range_sum(rsum + idx, UNIT, P));
    if (threadIdx.x == 0)
        __hip_atomic_store(ws_count + j / P, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// The joint launch's epilogue for 32-column group grp (columns n0 .. n0+31):
// one 32-lane group per activation row m, lane c is column n0 + c;
// sums(half, slot, l, sg, su) gives the gate and up tiles' sums (tiles
// 2grp + half of each) at the accumulator position of (m, c).
template <int M, typename Sum>
__device__ __forceinline__ void gate_up_epilogue(Sum sum, int N, int n0, int grp,
                                                 float *__restrict__ g, float *__restrict__ u,
                                                 float *__restrict__ h, uint8_t *__restrict__ hq)
{
    const int groups = blockDim.x >> 5;
    const int c = threadIdx.x & 31;
    const int half = c >> 4; // tile 2grp + half of each matrix
    for (int m0 = 0; m0 < M; m0 += groups) {
        const int m = m0 + (int)(threadIdx.x >> 5);
        const bool valid = m < M;
        const int mc = valid ? m : M - 1;
        // the accumulator position of row mc (pk_row inverted)
        constexpr int X = PkShape<M>::X;
        const int sm = mc / (2 * X), hm = (mc - 2 * X * sm) / X, xm = mc - 2 * X * sm - X * hm;
        const int slot = sm * 4 + xm;
        const int l = 16 * hm + (c & 15);
        float sg, su;
        sum(half, slot, l, sg, su);
        const float gv = sg * 0.0625f, uv = su * 0.0625f;
        const float hv = gv / (1.0f + expf(-gv)) * uv;
        const size_t o = (size_t)mc * N + n0 + c;
        if (valid) {
            if (g)
                g[o] = gv;
            if (u)
                u[o] = uv;
            if (h)
                h[o] = hv;
        }
        q8_1_block_store(hv, c, valid, hq + ((size_t)mc * (N / QK) + grp) * Q8_1_BYTES);
    }
}

// Gate and up projections of one Q8_1 activation with the SiLU(gate) * up
// product and its Q8_1 requantization as the epilogue ("Q6_K M=6 fused
// DFlash top-1 production record", "Strict run identity": joint gate/up over
// the packed width-6 projections).  Workgroup p owns
// output columns 32p .. 32p+31 of both matrices (N % 32 == 0, so its four
// 16-row tiles -- gate 2p, 2p+1, up 2p, 2p+1 -- are full); its waves take the
// 8-block chunks round-robin with all four tiles per chunk, so each staged
// activation block and each A operand serves four MFMAs.  The 32 columns are
// one Q8_1 block of h per activation row, quantized where it is computed; g,
// u and h never reach memory unless asked for.  Per column and row, g and u
// are the sums of the plain product (same per-wave order, waves added in
// order), h = g / (1 + exp(-g)) * u in binary32, then the Q8_1 block of h.
//
// CU balance (ws_sum != NULL): workgroups b < whole own group b as above;
// the groups past the last multiple of the CU count are cut into P K ranges
// (range r = chunks r*C/P .. (r+1)*C/P - 1), workgroup whole + j taking range
// j % P of group whole + j / P.  A range's four tiles' sums go to
// ws_sum[j][4][SLOTS*32] as agent-scope atomic stores; the workgroup waits
// for them (vmcnt(0)) and counts itself in ws_count[j / P]; the one that
// brings the count to P adds the P ranges' sums in range order, runs the
// epilogue above on them and sets the count back to 0 (the meeting of
// q4_0_mmvq_packed_kernel).
template <int M>
__global__ __launch_bounds__(512) void q4_0_gate_up_packed_kernel(
    const uint8_t *__restrict__ QG, const uint16_t *__restrict__ DG,
    const uint8_t *__restrict__ QU, const uint16_t *__restrict__ DU, int N, int nb, int P,
    int whole, const uint8_t *__restrict__ xq, float *__restrict__ g, float *__restrict__ u,
    float *__restrict__ h, uint8_t *__restrict__ hq, float *__restrict__ ws_sum,
    uint32_t *__restrict__ ws_count)
{
    constexpr int MS = PkShape<M>::MS;
    constexpr int SLOTS = MS * 4;
    constexpr int STRIDE = pk_wave_stride<M, 4>();
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int S = __builtin_amdgcn_readfirstlane(blockDim.x >> 6);
    const int nch = nb / PK_CB;
    int grp = blockIdx.x, c0 = 0, c1 = nch, j = -1;
    if ((int)blockIdx.x >= whole) {
        j = blockIdx.x - whole;
        const int r = j % P;
        grp = whole + j / P;
        c0 = (int)((int64_t)r * nch / P);
        c1 = (int)((int64_t)(r + 1) * nch / P);
    }
    const int n0 = grp * 2 * PK_TILE;
    const size_t tb = (size_t)PK_TILE * nb * 16; // nibble bytes of one full tile
    const size_t t0 = (size_t)n0 * nb * 16;
    const uint8_t *tile[4] = {QG + t0, QG + t0 + tb, QU + t0, QU + t0 + tb};
    const uint16_t *dtile[4] = {DG + (size_t)n0 * nb, DG + (size_t)(n0 + PK_TILE) * nb,
                                DU + (size_t)n0 * nb, DU + (size_t)(n0 + PK_TILE) * nb};
    float acc[4][MS][4];
    pk_accumulate<M, 4>(tile, dtile, PK_TILE, (size_t)8 * PK_TILE * 16, (size_t)2 * PK_TILE * 8,
                        nb, c0, c1 - c0, xq, smem + (size_t)wave * STRIDE, acc);
    pk_store_partials<4, MS>(acc, smem + (size_t)wave * STRIDE, lane);
    __syncthreads();
    // tile i's sum over this workgroup's waves at (slot, l)
    auto wave_sum = [&](int i, int slot, int l) {
        float sacc = 0.0f;
        for (int v = 0; v < S; ++v)
            sacc += pk_partial_sum<4, MS>(smem, STRIDE, v, i, slot, l);
        return sacc;
    };
    if (j < 0) {
        gate_up_epilogue<M>(
            [&](int half, int slot, int l, float &sg, float &su) {
                sg = wave_sum(half, slot, l);
                su = wave_sum(2 + half, slot, l);
            },
            N, n0, grp, g, u, h, hq);
        return;
    }
    float *rsum = ws_sum + (size_t)(j - j % P) * 4 * SLOTS * 32; // the group's P ranges
    for (int idx = threadIdx.x; idx < 4 * SLOTS * 32; idx += blockDim.x) {
        const int i = idx / (SLOTS * 32), slot = (idx >> 5) % SLOTS, l = idx & 31;
        __hip_atomic_store(rsum + (size_t)(j % P) * 4 * SLOTS * 32 + idx, wave_sum(i, slot, l),
                           __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    // the partial sums have been read: wave 0's first LDS word then tells the
    // workgroup whether it arrived last
    int *last = reinterpret_cast<int *>(smem);
    if (threadIdx.x == 0)
        *last = __hip_atomic_fetch_add(ws_count + j / P, 1u, __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT) == (uint32_t)(P - 1);
    __syncthreads();
    if (!*last)
        return;
    gate_up_epilogue<M>(
        [&](int half, int slot, int l, float &sg, float &su) {
            const float *p = rsum + (size_t)half * SLOTS * 32 + slot * 32 + l;
            pk_range_sum2(p, p + (size_t)2 * SLOTS * 32, (size_t)4 * SLOTS * 32, P, sg, su);
        },
        N, n0, grp, g, u, h, hq);
    if (threadIdx.x == 0)
        __hip_atomic_store(ws_count + j / P, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Waves per workgroup: about 1600 waves in flight for M >= 3 and 2560 for
// the lighter M <= 2 (measured on the ffn_up and down shapes: two and five
// waves per 16-row tile at M = 6, three and eight at M = 1), at least two, at
// most eight, never more than the tile has chunks or the LDS holds.
static int packed_waves(int64_t wgs, int64_t chunks, int M, int64_t wave_lds, int64_t limit)
{
    const int64_t target = M <= 2 ? 2560 : 1600;
    int64_t s = (target + wgs - 1) / wgs;
    if (s < 2)
        s = 2;
    if (s > 8)
        s = 8;
    if (s > chunks)
        s = chunks;
    while (s > 1 && s * wave_lds > limit)
        --s;
    return (int)(s < 1 ? 1 : s);
}

// K ranges a CU-count remainder tile is cut into: four, never more than
// the tile's C chunks.
static int packed_parts(int64_t C)
{
    return (int)(C < 4 ? C : 4);
}

// Workspace of the balanced launches: ws_count (one uint32 per cut tile or
// 32-column group, fewer than CUs of them) in the first
// pk_ws_count_bytes(cus) bytes, then ws_sum, PK_WS_TILE_FLOATS floats per
// cut tile or group (P * 4 * SLOTS * 32 at most: 4 ranges, the joint
// launch's 4 tiles, 12 slots at M = 17; the product uses a quarter).
constexpr int64_t PK_WS_TILE_FLOATS = 4 * 4 * 12 * 32;
static int64_t pk_ws_bytes(int64_t cus)
{
    return pk_ws_count_bytes(cus) + cus * PK_WS_TILE_FLOATS * (int64_t)sizeof(float);
}

// ws == NULL: every tile in one workgroup.  Else, for M >= 9, the tiles
// beyond the last multiple of the CU count are cut into P K ranges each.
// There the per-tile compute is large enough for the balance to pay (ffn_up
// M = 17: 18.6 against 21.4 us; down M = 9 / 12 / 17: 16.0 / 16.8 / 22.0
// against 18.5 / 19.9 / 27.2 us).  At M = 6 the ranges' meeting in the
// workspace cost more than the balance saved (ffn_up: 11.42 against
// 11.19 us uncut, 11.01 us for the cut launch with the meeting left out),
// and at M = 1 the cut launch won on ffn_up but lost on down (11.95 against
// 11.24 us).
// Waves per workgroup of the two-tile product (M >= 9), from a sweep of
// 2..6 waves at every M = 9..17 on ffn_up (the balanced launch) and down
// (4 K ranges): three on an unsplit launch (ffn_up M = 9 / 12 / 16: 12.6 /
// 13.1 / 14.5 us), four from three MFMAs per block pair on (M = 17: 16.6
// against 17.1 us with three) and on a split launch (down M = 12 / 17:
// 14.8 / 18.6 us; 15.9 / 19.6 with three).  Never more than a range has
// chunks or the LDS holds.
static int pair_waves(int M, int nsplit, int64_t chunks, int64_t wave_lds, int64_t limit)
{
    int64_t s = (M > 16 || nsplit > 1) ? 4 : 3;
    if (s > chunks)
        s = chunks;
    while (s > 1 && s * wave_lds > limit)
        --s;
    return (int)(s < 1 ? 1 : s);
}

constexpr int MAX_SPLIT = 8;

// The split count for a shape: enough K ranges that the launch has at least
// 1024 workgroups (four per CU), at most MAX_SPLIT and at most one range per
// chunk.  1 for the ffn_up shape (1088 tiles), 4 for down (320 tiles).
static int packed_default_splits(int64_t N, int64_t K)
{
    const int64_t tiles = (N + PK_TILE - 1) / PK_TILE;
    int64_t p = (1024 + tiles - 1) / tiles;
    const int64_t nch = K / QK / PK_CB;
    if (p > MAX_SPLIT)
        p = MAX_SPLIT;
    if (p > nch)
        p = nch;
    return (int)(p < 1 ? 1 : p);
}

// The split count for M rows.  Up to M = 10 a split launch keeps one tile
// per workgroup and the count is packed_default_splits.  From M = 11 two
// tiles share a workgroup, and the count (2..8, at most one range per
// chunk, every workgroup resident at once by the runtime's occupancy figure)
// is the one that spreads the workgroups most evenly over the CUs: the
// least ratio of the busiest CU's workgroups to the mean, the smaller count
// on a tie.  Down [5120 x 17408], 160 two-tile units, us for 2 / 3 / 4 / 5 /
// 6 / 8 ranges: M = 12 16.5 / 13.0 / 14.7 / 15.0 / 13.5 / 15.1, M = 17
// 20.5 / 16.3 / 18.5 / 20.2 / 17.8 / 20.3, following that ratio (1.6, 1.07,
// 1.2, 1.28, 1.07 at 256 CUs; 8 ranges exceed the resident count).  -1
// without a device.
template <int M>
static int64_t packed_splits_rows(int64_t N, int64_t K)
{
    const int64_t dflt = packed_default_splits(N, K);
    if constexpr (M >= 11) {
        const int64_t cus = device_cus();
        if (cus <= 0)
            return -1;
        if (N % (2 * PK_TILE) != 0)
            return dflt;
        const int64_t units = N / (2 * PK_TILE);
        const int64_t C = K / QK / PK_CB;
        const int64_t limit = device_lds_limit();
        const int64_t wave_lds = pk_wave_stride<M, 2>();
        const void *kernel = (const void *)q4_0_mmvq_packed_kernel<M, PK_ANY, 2>;
        if (!allow_dynamic_lds(kernel, limit))
            return -1;
        int64_t best = 0, best_w = 1, best_top = 0;
        for (int64_t n = 2; n <= MAX_SPLIT && n <= C; ++n) {
            const int64_t w = units * n;
            if (w < cus) // the launch would keep one tile per workgroup
                continue;
            const int s = pair_waves(M, (int)n, C / n, wave_lds, limit);
            int per_cu = 0;
            if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, WAVE * s,
                                                             (size_t)s * wave_lds) != hipSuccess ||
                per_cu <= 0)
                return -1;
            if (w > per_cu * cus)
                continue;
            // busiest CU against the mean: top / (w / cus), compared exactly
            const int64_t top = (w + cus - 1) / cus;
            if (best == 0 || top * best_w < best_top * w) {
                best = n;
                best_w = w;
                best_top = top;
            }
        }
        if (best > 0)
            return best;
    }
    return dflt;
}

// One launch of the product with NT 16-row tiles per workgroup (the unit
// the K ranges, the split and the cut apply to).
template <int M, int NT>
static bq8_status packed_launch_nt(const uint8_t *wp, int64_t N, int64_t K, const void *xq,
                                   int nsplit, float *y, void *ws, int64_t cus,
                                   hipStream_t stream, int cut_all = 0)
{
    const int nb = (int)(K / QK);
    const int64_t C = nb / PK_CB;
    const int64_t units = (N + PK_TILE * NT - 1) / (PK_TILE * NT);
    const int P = cut_all > 0 ? cut_all : packed_parts(C);
    const int64_t wave_lds = pk_wave_stride<M, NT>();
    const int64_t limit = device_lds_limit();
    const int ranges = cut_all > 0 ? cut_all : nsplit;
    int s = NT == 1 ? packed_waves(units * nsplit, C / nsplit, M, wave_lds, limit)
                    : pair_waves(M, ranges, C / ranges, wave_lds, limit);
    // split launches at M <= 2 take a third wave per workgroup: down with 4
    // K ranges, M = 1 / 2: 10.18 / 10.20 -> 9.92 / 9.92 us (at M = 6 and 9
    // the third wave lost: 11.15 -> 11.31, 13.37 -> 14.71 us)
    if (NT == 1 && nsplit > 1 && M <= 2 && s < 3 && C / nsplit >= 3 && 3 * wave_lds <= limit)
        s = 3;
    const int64_t lds = (int64_t)s * wave_lds;
    if (lds > limit)
        return BQ8_ERR_SHAPE;
    int64_t whole = units;
    if (cut_all > 0)
        whole = 0;
    else if (ws && nsplit == 1 && M >= 9)
        whole = units - units % cus;
    const int64_t grid = nsplit > 1 ? units * nsplit : whole + (units - whole) * P;
    const uint8_t *QS = wp;
    const uint16_t *D = reinterpret_cast<const uint16_t *>(wp + N * nb * 16);
    uint32_t *ws_count = static_cast<uint32_t *>(ws);
    float *ws_sum = ws ? reinterpret_cast<float *>(static_cast<uint8_t *>(ws) +
                                                   pk_ws_count_bytes(cus))
                       : nullptr;
    auto launch = [&](auto kernel) -> bq8_status {
        if (!allow_dynamic_lds((const void *)kernel, limit))
            return BQ8_ERR_HIP;
        (void)hipGetLastError();
        hipLaunchKernelGGL(kernel, dim3((unsigned)grid), dim3(WAVE * s), (size_t)lds, stream, QS,
                           D, (int)N, nb, nsplit, P, (int)whole, (const uint8_t *)xq, y, ws_sum,
                           ws_count);
        return launch_status();
    };
    if constexpr (NT == 1 && M <= 8) {
        if (N % PK_TILE == 0)
            return nsplit > 1 ? launch(q4_0_mmvq_packed_kernel<M, PK_FULL_SPLIT, 1>)
                              : launch(q4_0_mmvq_packed_kernel<M, PK_FULL_WHOLE, 1>);
    }
    return launch(q4_0_mmvq_packed_kernel<M, PK_ANY, NT>);
}

// From M = 9 (M = 11 on a split launch) a workgroup takes two tiles when
// N % 32 == 0 and the launch still has a workgroup for every CU: each staged
// activation chunk and each A operand then serve two tiles (the activation
// bytes per chunk outweigh the weight bytes from M = 8 up).  Against one
// tile per workgroup: ffn_up (balanced) M = 9 / 12 / 17 12.6 / 13.1 / 16.6
// against 13.7 / 14.1 / 18.5 us; down, 4 K ranges, M = 12 / 17 14.8 / 18.6
// against 15.4 / 20.3 us, while at M = 9 and 10 one tile stays ahead
// (13.9 against 14.4 us).
template <int M>
static bq8_status packed_launch(const uint8_t *wp, int64_t N, int64_t K, const void *xq, int nsplit,
                                float *y, void *ws, int64_t cus, hipStream_t stream)
{
    if constexpr (M >= 9) {
        const int64_t cu = cus > 0 ? cus : device_cus();
        if (N % (2 * PK_TILE) == 0 && cu > 0 && N / (2 * PK_TILE) * nsplit >= cu &&
            (nsplit == 1 || M >= 11))
            return packed_launch_nt<M, 2>(wp, N, K, xq, nsplit, y, ws, cu, stream);
        if constexpr (M >= 11) {
            // a balanced launch with fewer two-tile units than CUs: every
            // unit is cut into the split count's K ranges, which meet in the
            // workspace
            if (ws && nsplit == 1 && N % (2 * PK_TILE) == 0 && cu > 0) {
                const int64_t P = packed_splits_rows<M>(N, K);
                if (P >= 2 && N / (2 * PK_TILE) * P >= cu)
                    return packed_launch_nt<M, 2>(wp, N, K, xq, 1, y, ws, cu, stream, (int)P);
            }
        }
    }
    return packed_launch_nt<M, 1>(wp, N, K, xq, nsplit, y, ws, cus, stream);
}

// Waves per gate/up workgroup: about 1088 waves in flight for M <= 2, 1632
// for M = 3..8 and 2176 from M = 9 (two, three and four per 32-column
// workgroup on the 17408 x 5120 shape; a sweep of 2..8 waves there put
// M = 1 / 6 / 9 / 17 at 18.6 / 19.8 / 25.6 / 30.6 us), at least one, at most
// eight, never more than the row has chunks or the LDS holds.
static int gate_up_waves(int64_t groups, int nb, int M, int64_t wave_lds, int64_t limit)
{
    const int64_t target = M <= 2 ? 1088 : M <= 8 ? 1632 : 2176;
    int64_t s = (target + groups - 1) / groups;
    if (s > 8)
        s = 8;
    if (s > nb / PK_CB)
        s = nb / PK_CB;
    while (s > 1 && s * wave_lds > limit)
        --s;
    return (int)(s < 1 ? 1 : s);
}

template <int M>
static bq8_status gate_up_launch(const uint8_t *wg, const uint8_t *wu, int64_t N, int64_t K,
                                 const void *xq, float *g, float *u, float *h, void *hq, void *ws,
                                 int64_t cus, hipStream_t stream)
{
    const int nb = (int)(K / QK);
    const int64_t groups = N / (2 * PK_TILE);
    const int64_t limit = device_lds_limit();
    const int s = gate_up_waves(groups, nb, M, pk_wave_stride<M, 4>(), limit);
    const int64_t lds = (int64_t)s * pk_wave_stride<M, 4>();
    if (lds > limit)
        return BQ8_ERR_SHAPE;
    if (!allow_dynamic_lds((const void *)q4_0_gate_up_packed_kernel<M>, limit))
        return BQ8_ERR_HIP;
    const size_t dplane = (size_t)N * nb * 16;
    // with a workspace and at least as many groups as CUs, the groups past
    // the last multiple of the CU count are cut into P K ranges each (ffn
    // shape, M = 6 / 1 / 9 / 17: 22.4 / 21.5 / 28.1 / 34.5 us uncut, 20.6 /
    // 19.9 / 26.1 / 31.6 us cut).  With fewer groups than CUs every group
    // would be cut, and the meeting outweighs the balance (the 8-way shard,
    // 68 groups: 9.5 us uncut, 12.3 us cut).
    const int P = packed_parts(nb / PK_CB);
    const int64_t whole = ws && groups >= cus ? groups - groups % cus : groups;
    const int64_t grid = whole + (groups - whole) * P;
    uint32_t *ws_count = static_cast<uint32_t *>(ws);
    float *ws_sum = ws ? reinterpret_cast<float *>(static_cast<uint8_t *>(ws) +
                                                   pk_ws_count_bytes(cus))
                       : nullptr;
    (void)hipGetLastError();
    hipLaunchKernelGGL((q4_0_gate_up_packed_kernel<M>), dim3((unsigned)grid), dim3(WAVE * s),
                       (size_t)lds, stream, wg, reinterpret_cast<const uint16_t *>(wg + dplane), wu,
                       reinterpret_cast<const uint16_t *>(wu + dplane), (int)N, nb, P, (int)whole,
                       (const uint8_t *)xq, g, u, h, (uint8_t *)hq, ws_sum, ws_count);
    return launch_status();
}

static bool packed_shape_ok(int64_t N, int64_t K)
{
    return N >= 1 && N < (int64_t(1) << 31) && K >= 512 && K % 512 == 0 &&
           K <= (int64_t(1) << 26) && N * (K / QK) * Q4_0_BYTES < (int64_t(1) << 40);
}

static bq8_status packed_product(const void *wp, int64_t N, int64_t K, const void *xq, int64_t M,
                                 int nsplit, float *y, void *ws, int64_t ws_bytes, void *stream)
{
    if (!wp || !xq || !y)
        return BQ8_ERR_NULL;

    if (!packed_shape_ok(N, K) || M < 1 || M > 17 || M * K >= (int64_t(1) << 31) || nsplit < 1 ||
        nsplit > MAX_SPLIT || nsplit > K / QK / PK_CB ||
        (int64_t)nsplit * M * N >= (int64_t(1) << 40) ||
        (int64_t)nsplit * ((N + PK_TILE - 1) / PK_TILE) >= (int64_t(1) << 31))
        return BQ8_ERR_SHAPE;
    if (!aligned(wp, 16) || !aligned(xq, 16) || !aligned(y, 4) || !aligned(ws, 256))
        return BQ8_ERR_ALIGN;
    int64_t cus = 0;
    if (ws) {
        cus = device_cus();
        if (cus <= 0)
            return BQ8_ERR_HIP;
        if (ws_bytes < pk_ws_bytes(cus))
            return BQ8_ERR_SIZE;
    }
    const uint8_t *p = (const uint8_t *)wp;
    hipStream_t s = (hipStream_t)stream;
    switch (M) {
    case 1: return packed_launch<1>(p, N, K, xq, nsplit, y, ws, cus, s);
    case 2: return packed_launch<2>(p, N, K, xq, nsplit, y, ws, cus, s);
    case 3: return packed_launch<3>(p, N, K, xq, nsplit, y, ws, cus, s);
    case 4: return packed_launch<4>(p, N, K, xq, nsplit, y, ws, cus, s);
    case 5: return packed_launch<5>(p, N, K, xq, nsplit, y, ws, cus, s);
    case 6: return packed_launch<6>(p, N, K, xq, nsplit, y, ws, cus, s);
    case 7: return packed_launch<7>(p, N, K, xq, nsplit, y, ws, cus, s);
    case 8: return packed_launch<8>(p, N, K, xq, nsplit, y, ws, cus, s);
    case 9: return packed_launch<9>(p, N, K, xq, nsplit, y, ws, cus, s);
    case 10: return packed_launch<10>(p, N, K, xq, nsplit, y, ws, cus, s);
    case 11: return packed_launch<11>(p, N, K, xq, nsplit, y, ws, cus, s);
    case 12: return packed_launch<12>(p, N, K, xq, nsplit, y, ws, cus, s);
    case 13: return packed_launch<13>(p, N, K, xq, nsplit, y, ws, cus, s);
    case 14: return packed_launch<14>(p, N, K, xq, nsplit, y, ws, cus, s);
    case 15: return packed_launch<15>(p, N, K, xq, nsplit, y, ws, cus, s);
    case 16: return packed_launch<16>(p, N, K, xq, nsplit, y, ws, cus, s);
    default: return packed_launch<17>(p, N, K, xq, nsplit, y, ws, cus, s);
    }
}

} // namespace bq8

using namespace bq8;

BQ8_EXPORT int64_t q4_0_pack_bytes(int64_t N, int64_t K)
{
    if (!packed_shape_ok(N, K))
        return -1;
    return N * (K / QK) * Q4_0_BYTES;
}

BQ8_EXPORT bq8_status q4_0_pack(const void *w, int64_t N, int64_t K, void *wp, int64_t wp_bytes,
                                void *stream)
{
    if (!w || !wp)
        return BQ8_ERR_NULL;
    if (!packed_shape_ok(N, K))
        return BQ8_ERR_SHAPE;
    if (!aligned(w, 2) || !aligned(wp, 16))
        return BQ8_ERR_ALIGN;
    if (wp_bytes != q4_0_pack_bytes(N, K))
        return BQ8_ERR_SIZE;
    const int nb = (int)(K / QK);
    const int64_t items = N * nb;
    uint8_t *QS = (uint8_t *)wp;
    uint16_t *D = reinterpret_cast<uint16_t *>(QS + N * nb * 16);
    (void)hipGetLastError();
    hipLaunchKernelGGL(q4_0_pack_kernel, dim3((unsigned)((items + 255) / 256)), dim3(256), 0,
                       (hipStream_t)stream, (const uint8_t *)w, (int)N, nb, QS, D);
    return launch_status();
}

BQ8_EXPORT bq8_status q4_0_mmvq_packed(const void *wp, int64_t N, int64_t K, const void *xq,
                                       int64_t M, float *y, void *stream)
{
    return packed_product(wp, N, K, xq, M, 1, y, nullptr, 0, stream);
}

BQ8_EXPORT int64_t q4_0_mmvq_packed_ws_bytes(void)
{
    const int64_t cus = device_cus();
    return cus > 0 ? pk_ws_bytes(cus) : -1;
}

BQ8_EXPORT bq8_status q4_0_mmvq_packed_ws(const void *wp, int64_t N, int64_t K, const void *xq,
                                          int64_t M, float *y, void *ws, int64_t ws_bytes,
                                          void *stream)
{
    if (!ws)
        return BQ8_ERR_NULL;
    return packed_product(wp, N, K, xq, M, 1, y, ws, ws_bytes, stream);
}

BQ8_EXPORT int64_t q4_0_mmvq_packed_splits(int64_t N, int64_t K)
{
    if (!packed_shape_ok(N, K))
        return -1;
    return packed_default_splits(N, K);
}

BQ8_EXPORT int64_t q4_0_mmvq_packed_splits_rows(int64_t N, int64_t K, int64_t M)
{
    if (!packed_shape_ok(N, K) || M < 1 || M > 17)
        return -1;
    switch (M) {
    case 11: return packed_splits_rows<11>(N, K);
    case 12: return packed_splits_rows<12>(N, K);
    case 13: return packed_splits_rows<13>(N, K);
    case 14: return packed_splits_rows<14>(N, K);
    case 15: return packed_splits_rows<15>(N, K);
    case 16: return packed_splits_rows<16>(N, K);
    case 17: return packed_splits_rows<17>(N, K);
    default: return packed_default_splits(N, K);
    }
}

BQ8_EXPORT bq8_status q4_0_mmvq_packed_split(const void *wp, int64_t N, int64_t K,
                                             const void *xq, int64_t M, int64_t nsplit,
                                             float *ypart, void *stream)
{
    if (nsplit < 1 || nsplit > MAX_SPLIT)
        return BQ8_ERR_SHAPE;
    return packed_product(wp, N, K, xq, M, (int)nsplit, ypart, nullptr, 0, stream);
}

static bq8_status gate_up_product(const void *wg, const void *wu, int64_t N, int64_t K,
                                  const void *xq, int64_t M, float *g, float *u, float *h,
                                  void *hq, void *ws, int64_t ws_bytes, void *stream)
{
    if (!wg || !wu || !xq || !hq)
        return BQ8_ERR_NULL;
    if (!packed_shape_ok(N, K) || N % (2 * PK_TILE) != 0 || M < 1 || M > 17 ||
        M * K >= (int64_t(1) << 31) || M * N >= (int64_t(1) << 31))
        return BQ8_ERR_SHAPE;
    if (!aligned(wg, 16) || !aligned(wu, 16) || !aligned(xq, 16) || !aligned(hq, 4) ||
        (g && !aligned(g, 4)) || (u && !aligned(u, 4)) || (h && !aligned(h, 4)) ||
        !aligned(ws, 256))
        return BQ8_ERR_ALIGN;
    int64_t cus = 0;
    if (ws) {
        cus = device_cus();
        if (cus <= 0)
            return BQ8_ERR_HIP;
        if (ws_bytes < pk_ws_bytes(cus))
            return BQ8_ERR_SIZE;
    }
    const uint8_t *a = (const uint8_t *)wg, *b = (const uint8_t *)wu;
    hipStream_t s = (hipStream_t)stream;
    switch (M) {
    case 1: return gate_up_launch<1>(a, b, N, K, xq, g, u, h, hq, ws, cus, s);
    case 2: return gate_up_launch<2>(a, b, N, K, xq, g, u, h, hq, ws, cus, s);
    case 3: return gate_up_launch<3>(a, b, N, K, xq, g, u, h, hq, ws, cus, s);
    case 4: return gate_up_launch<4>(a, b, N, K, xq, g, u, h, hq, ws, cus, s);
    case 5: return gate_up_launch<5>(a, b, N, K, xq, g, u, h, hq, ws, cus, s);
    case 6: return gate_up_launch<6>(a, b, N, K, xq, g, u, h, hq, ws, cus, s);
    case 7: return gate_up_launch<7>(a, b, N, K, xq, g, u, h, hq, ws, cus, s);
    case 8: return gate_up_launch<8>(a, b, N, K, xq, g, u, h, hq, ws, cus, s);
    case 9: return gate_up_launch<9>(a, b, N, K, xq, g, u, h, hq, ws, cus, s);
    case 10: return gate_up_launch<10>(a, b, N, K, xq, g, u, h, hq, ws, cus, s);
    case 11: return gate_up_launch<11>(a, b, N, K, xq, g, u, h, hq, ws, cus, s);
    case 12: return gate_up_launch<12>(a, b, N, K, xq, g, u, h, hq, ws, cus, s);
    case 13: return gate_up_launch<13>(a, b, N, K, xq, g, u, h, hq, ws, cus, s);
    case 14: return gate_up_launch<14>(a, b, N, K, xq, g, u, h, hq, ws, cus, s);
    case 15: return gate_up_launch<15>(a, b, N, K, xq, g, u, h, hq, ws, cus, s);
    case 16: return gate_up_launch<16>(a, b, N, K, xq, g, u, h, hq, ws, cus, s);
    default: return gate_up_launch<17>(a, b, N, K, xq, g, u, h, hq, ws, cus, s);
    }
}

BQ8_EXPORT bq8_status q4_0_gate_up_silu_q8_1_packed(const void *wg, const void *wu, int64_t N,
                                                    int64_t K, const void *xq, int64_t M,
                                                    float *g, float *u, float *h, void *hq,
                                                    void *stream)
{
    return gate_up_product(wg, wu, N, K, xq, M, g, u, h, hq, nullptr, 0, stream);
}

BQ8_EXPORT bq8_status q4_0_gate_up_silu_q8_1_packed_ws(const void *wg, const void *wu, int64_t N,
                                                       int64_t K, const void *xq, int64_t M,
                                                       float *g, float *u, float *h, void *hq,
                                                       void *ws, int64_t ws_bytes, void *stream)
{
    if (!ws)
        return BQ8_ERR_NULL;
    return gate_up_product(wg, wu, N, K, xq, M, g, u, h, hq, ws, ws_bytes, stream);
}
