// Width-6 verifier FFN stream: a chain of layers, each a Q4_0 gate and up
// projection sharing one Q8_1 activation, SiLU(gate)*up requantized to Q8_1
// on the device, and a Q4_0 down projection whose output becomes the next
// layer's input through an RMS step and a Q8_1 quantize.
//
// "Qwen3.6 27B Q4_0 DFlash/SYCL closure": offline-packed width-6 gate/up and
// down projections carry the target verifier ("What materially worked");
// the down-to-next-RMS/Q8 boundary ("Closed or negative paths").
// "Qwen3.6 27B B70 follow-up: Q8 activation cache, FP8 artifacts, MTP
// blocker", "Q8_1 activation cache prototype": gate and up read the same
// quantized activation.
//
// The whole pass is enqueued from native code on the caller's stream, no
// host synchronization, no allocation: five launches per layer on standard
// weights, three on packed ones -- the RMS step, one joint launch for gate,
// up and the SiLU*up requant, and a down projection split along K into
// enough ranges to spread over every CU, whose partial sums the next RMS
// step adds (one last sum writes y).  Every shape and every layer's pointers are validated
// before the first launch, so a rejected call enqueues nothing.
#include "bq8_dev.h"
#include "bq8_host.h"

namespace bq8 {

static int64_t align256(int64_t v) { return (v + 255) & ~int64_t(255); }

// Clears the workspace's counters at the start of a pass (a kernel, not a
// memset, so that the pass can be captured in a HIP graph).
__global__ __launch_bounds__(256) void zero_words_kernel(uint32_t *__restrict__ p, int n)
{
    for (int i = threadIdx.x; i < n; i += blockDim.x)
        p[i] = 0u;
}

// Offsets of the stage buffers inside the caller's workspace; `parts`
// holds the packed path's split down-projection sums (up to eight partial
// [M][hidden] rows), internal to the pass.
struct StreamLayout {
    int64_t xq, g, u, hq, parts, total;
};

static bool stream_layout(int64_t M, int64_t hidden, int64_t ffn, StreamLayout *L)
{
    if (M < 1 || M > 17 || hidden < QK || hidden % QK != 0 || ffn < QK || ffn % QK != 0 ||
        hidden > 32768 || ffn > (int64_t(1) << 26) ||
        M * hidden >= (int64_t(1) << 31) || M * ffn >= (int64_t(1) << 31))
        return false;
    L->xq = 0;
    L->g = align256(M * (hidden / QK) * Q8_1_BYTES);
    L->u = L->g + align256(M * ffn * 4);
    L->hq = L->u + align256(M * ffn * 4);
    L->parts = L->hq + align256(M * (ffn / QK) * Q8_1_BYTES);
    L->total = L->parts + align256(8 * M * hidden * 4);
    return true;
}

} // namespace bq8

using namespace bq8;

BQ8_EXPORT bq8_status q4_0_ffn_stream_layout(int64_t M, int64_t hidden, int64_t ffn,
                                             int64_t *offsets)
{
    if (!offsets)
        return BQ8_ERR_NULL;
    StreamLayout L;
    if (!stream_layout(M, hidden, ffn, &L))
        return BQ8_ERR_SHAPE;
    offsets[0] = L.xq;
    offsets[1] = L.g;
    offsets[2] = L.u;
    offsets[3] = L.hq;
    // on a device, room for the joint launches' workspace after the stages
    const int64_t wsb = q4_0_mmvq_packed_ws_bytes();
    offsets[4] = L.total + (wsb > 0 ? align256(wsb) : 0);
    return BQ8_OK;
}

typedef bq8_status (*proj_fn)(const void *w, int64_t N, int64_t K, const void *xq, int64_t M,
                              float *y, void *stream);

static bq8_status ffn_stream(proj_fn proj, bool joint, int64_t align_k,
                             const void *const *w_gate,
                             const void *const *w_up, const void *const *w_down, int64_t layers,
                             int64_t M, int64_t hidden, int64_t ffn, const float *x0, float eps,
                             float *y, void *work, int64_t work_bytes, void *stream)
{
    if (!w_gate || !w_up || !w_down || !x0 || !y || !work)
        return BQ8_ERR_NULL;
    StreamLayout L;
    if (layers < 1 || layers > (int64_t(1) << 20) || !stream_layout(M, hidden, ffn, &L) ||
        !(eps > 0.0f) || ffn * (hidden / QK) * Q4_0_BYTES >= (int64_t(1) << 40) ||
        hidden % align_k != 0 || ffn % align_k != 0)
        return BQ8_ERR_SHAPE;
    for (int64_t l = 0; l < layers; ++l) {
        if (!w_gate[l] || !w_up[l] || !w_down[l])
            return BQ8_ERR_NULL;
        if (!aligned(w_gate[l], 16) || !aligned(w_up[l], 16) || !aligned(w_down[l], 16))
            return BQ8_ERR_ALIGN;
    }
    if (!aligned(x0, 4) || !aligned(y, 4) || !aligned(work, 256))
        return BQ8_ERR_ALIGN;
    if (work_bytes < L.total)
        return BQ8_ERR_SIZE;

    uint8_t *base = static_cast<uint8_t *>(work);
    void *xq = base + L.xq;
    float *g = reinterpret_cast<float *>(base + L.g);
    float *u = reinterpret_cast<float *>(base + L.u);
    void *hq = base + L.hq;
    // packed path: the down projection is split in P ranges of its K, summed
    // in range order by the next layer's RMS step (and by a last sum into y)
    float *parts = reinterpret_cast<float *>(base + L.parts);
    const int64_t P = joint ? q4_0_mmvq_packed_splits(hidden, ffn) : 1;
    if (P < 1)
        return BQ8_ERR_SHAPE;

    // packed path: if the work area also holds the workspace, the joint
    // launches balance their 32-column groups over the CUs; its counters
    // are cleared here once, and every completed launch leaves them clear
    void *ws = nullptr;
    int64_t wsb = 0;
    const int64_t cus = joint ? device_cus() : -1;
    if (cus > 0) {
        wsb = q4_0_mmvq_packed_ws_bytes();
        if (wsb > 0 && work_bytes >= L.total + align256(wsb))
            ws = base + L.total;
    }

    // Everything below was validated above; a nonzero status can only be a
    // launch failure, reported as is.
    if (ws) {
        const int words = (int)(pk_ws_count_bytes(cus) / 4);
        (void)hipGetLastError();
        hipLaunchKernelGGL(zero_words_kernel, dim3(1), dim3(256), 0, (hipStream_t)stream,
                           static_cast<uint32_t *>(ws), words);
        if (hipGetLastError() != hipSuccess)
            return BQ8_ERR_HIP;
    }
    bq8_status st = q8_1_quantize(x0, M, hidden, xq, stream);
    for (int64_t l = 0; l < layers && st == BQ8_OK; ++l) {
        if (l > 0 && joint)
            st = rms_norm_q8_1_sum(parts, P, M, hidden, eps, nullptr, nullptr, xq, stream);
        if (l > 0 && !joint)
            st = rms_norm_q8_1(y, M, hidden, eps, nullptr, xq, stream);
        if (st == BQ8_OK && joint && ws)
            st = q4_0_gate_up_silu_q8_1_packed_ws(w_gate[l], w_up[l], ffn, hidden, xq, M,
                                                  nullptr, nullptr, nullptr, hq, ws, wsb, stream);
        if (st == BQ8_OK && joint && !ws)
            st = q4_0_gate_up_silu_q8_1_packed(w_gate[l], w_up[l], ffn, hidden, xq, M, nullptr,
                                               nullptr, nullptr, hq, stream);
        if (st == BQ8_OK && !joint)
            st = proj(w_gate[l], ffn, hidden, xq, M, g, stream);
        if (st == BQ8_OK && !joint)
            st = proj(w_up[l], ffn, hidden, xq, M, u, stream);
        if (st == BQ8_OK && !joint)
            st = silu_mul_q8_1(g, u, M, ffn, nullptr, hq, stream);
        if (st == BQ8_OK && joint)
            st = q4_0_mmvq_packed_split(w_down[l], hidden, ffn, hq, M, P, parts, stream);
        if (st == BQ8_OK && !joint)
            st = proj(w_down[l], hidden, ffn, hq, M, y, stream);
    }
    if (st == BQ8_OK && joint)
        st = rms_norm_q8_1_sum(parts, P, M, hidden, eps, y, nullptr, nullptr, stream);
    return st;
}

static bq8_status proj_standard(const void *w, int64_t N, int64_t K, const void *xq, int64_t M,
                                float *y, void *stream)
{
    return q4_0_mmvq(w, N, K, xq, M, y, stream);
}

static bq8_status proj_packed(const void *w, int64_t N, int64_t K, const void *xq, int64_t M,
                              float *y, void *stream)
{
    return q4_0_mmvq_packed(w, N, K, xq, M, y, stream);
}

BQ8_EXPORT bq8_status q4_0_ffn_stream(const void *const *w_gate, const void *const *w_up,
                                      const void *const *w_down, int64_t layers, int64_t M,
                                      int64_t hidden, int64_t ffn, const float *x0, float eps,
                                      float *y, void *work, int64_t work_bytes, void *stream)
{
    return ffn_stream(proj_standard, false, QK, w_gate, w_up, w_down, layers, M, hidden, ffn, x0,
                      eps, y, work, work_bytes, stream);
}

BQ8_EXPORT bq8_status q4_0_ffn_stream_packed(const void *const *w_gate, const void *const *w_up,
                                             const void *const *w_down, int64_t layers,
                                             int64_t M, int64_t hidden, int64_t ffn,
                                             const float *x0, float eps, float *y, void *work,
                                             int64_t work_bytes, void *stream)
{
    return ffn_stream(proj_packed, true, 512, w_gate, w_up, w_down, layers, M, hidden, ffn, x0,
                      eps, y, work, work_bytes, stream);
}
