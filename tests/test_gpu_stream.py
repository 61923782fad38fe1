"""GPU parity of the verifier FFN stream (q4_0_ffn_stream).

1. The native pass equals the same steps made one C-ABI call at a time,
   bit for bit (same kernels, fixed reduction orders), on small shapes that
   take both the MFMA path (K % 256 == 0) and the dot4 path, at several M,
   and on seeded random widths, row counts and layer counts.
2. At the full stream shape (64 layers of gate/up [5120 -> 17408] and down
   [17408 -> 5120], M = 6), on both weight layouts, every stage of the last
   layer is checked against
   the oracle given the GPU's own input to that stage: the RMS step and the
   two SiLU*up and Q8_1 steps to |d| <= 1e-5 |ref| + 1e-6 with the quantized
   bytes bit-exact given the GPU's f32 values, and the three projections to
   the block-term tolerance.  The chained end-to-end value is parity
   unpinned: one requantization flip moves outputs by more than the
   tolerance.
"""
import ctypes
import sys

import numpy as np
import pytest

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu
if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

import oracle  # noqa: E402
import block_quantized_gemv_q8_amd as bq  # noqa: E402
from block_quantized_gemv_q8_amd import synth  # noqa: E402

DEV = "cuda:0"
REL, ABS = 1e-5, 1e-6
EPS = 1e-6


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


def composed(wg, wu, wd, x0, eps):
    """The stream's steps, one C-ABI call each."""
    xq = bq.q8_1_quantize(x0)
    M = x0.shape[0]
    y = None
    for l in range(len(wg)):
        if l > 0:
            xq = bq.rms_norm_q8_1(y, eps)
        g = bq.q4_0_mmvq(wg[l], xq, M)
        u = bq.q4_0_mmvq(wu[l], xq, M)
        hq = bq.silu_mul_q8_1(g, u)
        y = bq.q4_0_mmvq(wd[l], hq, M)
    return y, dict(xq=xq, g=g, u=u, hq=hq)


def _random_stream_shapes(seed, granule, n):
    """Seeded (M, hidden, ffn, layers) draws: widths multiples of granule."""
    rng = np.random.default_rng(seed)
    return [(int(rng.integers(1, 18)), granule * int(rng.integers(1, 4096 // granule + 1)),
             granule * int(rng.integers(1, 4096 // granule + 1)), int(rng.integers(1, 4)))
            for _ in range(n)]


@pytest.mark.parametrize("M,hidden,ffn,layers", [(6, 512, 1024, 3), (1, 256, 768, 2),
                                                 (9, 288, 352, 3), (17, 1280, 512, 2)]
                         + _random_stream_shapes(9700, 32, 6))
def test_stream_equals_composed_calls(M, hidden, ffn, layers):
    say(f"stream vs composed M={M} hidden={hidden} ffn={ffn} layers={layers}")
    wg = [synth.q4_0_weights_device(900 + 3 * l, ffn, hidden) for l in range(layers)]
    wu = [synth.q4_0_weights_device(901 + 3 * l, ffn, hidden) for l in range(layers)]
    wd = [synth.q4_0_weights_device(902 + 3 * l, hidden, ffn) for l in range(layers)]
    x0 = torch.from_numpy(synth.stream_x0(M, hidden, seed=77)).to(DEV)
    y, work = bq.q4_0_ffn_stream(wg, wu, wd, x0, EPS)
    st = bq.stream_stages(work, M, hidden, ffn)
    y_ref, st_ref = composed(wg, wu, wd, x0, EPS)
    assert torch.equal(y, y_ref)
    for k in ("xq", "g", "u", "hq"):
        assert torch.equal(st[k], st_ref[k]), k
    assert torch.isfinite(y).all()
    # a second pass on the same buffers gives the same bits
    y2, _ = bq.q4_0_ffn_stream(wg, wu, wd, x0, EPS, y=torch.empty_like(y), work=work)
    assert torch.equal(y2, y)


def _gemv_check(w_dev, xq, M, gpu_y, what):
    w = host(w_dev)
    N = w.shape[0]
    K = w.shape[1] // 18 * 32
    ref, bound = oracle.q4_0_gemv(w, N, K, xq, M)
    err = np.abs(gpu_y.astype(np.float64) - ref)
    tol = REL * bound + ABS
    assert (err <= tol).all(), f"{what}: {(err > tol).sum()} outside tolerance"
    return float((err / tol).max())


def test_stream_full_shape_last_layer_stages():
    cfg = synth.STREAM
    L, M, H, F = cfg["layers"], cfg["M"], cfg["hidden"], cfg["ffn"]
    say(f"full stream: generating {L} layers of weights on the device")
    wg, wu, wd = synth.stream_weights_device(L, H, F)
    x0 = torch.from_numpy(synth.stream_x0()).to(DEV)
    tables = tuple(bq.stream_weight_table(ws) for ws in (wg, wu, wd))
    say("full stream: pass over layers 0..62")
    y_prev, _ = bq.q4_0_ffn_stream(wg[:-1], wu[:-1], wd[:-1], x0, EPS)
    y_prev = y_prev.clone()
    say("full stream: pass over layers 0..63")
    y, work = bq.q4_0_ffn_stream(wg, wu, wd, x0, EPS, tables=tables)
    st = {k: host(v) for k, v in bq.stream_stages(work, M, H, F).items()}
    yh = host(y)
    assert np.isfinite(yh).all()

    # RMS step into the last layer, from the GPU's own y of layer 62
    xo = torch.empty((M, H), dtype=torch.float32, device=DEV)
    xq = host(bq.rms_norm_q8_1(y_prev, EPS, x=xo))
    xg = host(xo)
    ref = oracle.rms_norm(host(y_prev), EPS)
    assert (np.abs(xg.astype(np.float64) - ref) <= REL * np.abs(ref) + ABS).all()
    assert (oracle.q8_1_quantize(xg) == xq).all()
    assert (xq == st["xq"]).all()

    # gate and up projections from the stream's own Q8_1 input
    say("full stream: oracle gate/up/down of layer 63")
    _gemv_check(wg[-1], st["xq"], M, st["g"], "gate")
    _gemv_check(wu[-1], st["xq"], M, st["u"], "up")

    # SiLU(g)*u and its requantization
    h = torch.empty((M, F), dtype=torch.float32, device=DEV)
    g_d = torch.from_numpy(st["g"]).to(DEV)
    u_d = torch.from_numpy(st["u"]).to(DEV)
    hq = host(bq.silu_mul_q8_1(g_d, u_d, h=h))
    hg = host(h)
    ref = oracle.silu_mul(st["g"], st["u"])
    assert (np.abs(hg.astype(np.float64) - ref) <= REL * np.abs(ref) + ABS).all()
    assert (oracle.q8_1_quantize(hg) == hq).all()
    assert (hq == st["hq"]).all()

    # down projection from the stream's own requantized h
    _gemv_check(wd[-1], st["hq"], M, yh, "down")


def composed_packed(wg, wu, wd, x0, eps, hidden, ffn):
    """The packed stream's steps, one C-ABI call each (its joint launches are
    the CU-balanced ones, through a workspace, as in the stream)."""
    xq = bq.q8_1_quantize(x0)
    M = x0.shape[0]
    P = bq.q4_0_mmvq_packed_splits(hidden, ffn)
    ws = bq.q4_0_mmvq_packed_workspace()
    parts = None
    for l in range(len(wg)):
        if l > 0:
            xq = bq.rms_norm_q8_1_sum(parts, eps)
        hq = bq.q4_0_gate_up_silu_q8_1_packed(wg[l], wu[l], ffn, hidden, xq, M, ws=ws)
        parts = bq.q4_0_mmvq_packed_split(wd[l], hidden, ffn, hq, M, P)
    y = torch.empty((M, hidden), dtype=torch.float32, device=DEV)
    bq.rms_norm_q8_1_sum(parts, eps, y=y, want_xq=False)
    return y, dict(xq=xq, hq=hq)


@pytest.mark.parametrize("M,hidden,ffn,layers", [(6, 512, 1024, 3), (17, 1024, 1536, 2),
                                                 (1, 512, 512, 2), (6, 5120, 1024, 2)]
                         + _random_stream_shapes(9701, 512, 6))
def test_packed_stream_equals_composed_calls(M, hidden, ffn, layers):
    say(f"packed stream vs composed M={M} hidden={hidden} ffn={ffn} layers={layers} "
        f"down split {bq.q4_0_mmvq_packed_splits(hidden, ffn)}")
    wg = [bq.q4_0_pack(synth.q4_0_weights_device(950 + 3 * l, ffn, hidden)) for l in range(layers)]
    wu = [bq.q4_0_pack(synth.q4_0_weights_device(951 + 3 * l, ffn, hidden)) for l in range(layers)]
    wd = [bq.q4_0_pack(synth.q4_0_weights_device(952 + 3 * l, hidden, ffn)) for l in range(layers)]
    x0 = torch.from_numpy(synth.stream_x0(M, hidden, seed=78)).to(DEV)
    y, work = bq.q4_0_ffn_stream(wg, wu, wd, x0, EPS, packed=True, ffn=ffn)
    st = bq.stream_stages(work, M, hidden, ffn)
    y_ref, st_ref = composed_packed(wg, wu, wd, x0, EPS, hidden, ffn)
    assert torch.equal(y, y_ref)
    for k in ("xq", "hq"):
        assert torch.equal(st[k], st_ref[k]), k


def test_packed_stream_full_shape_last_layer_stages():
    """The packed pass the bench times: all 64 full-shape layers."""
    cfg = synth.STREAM
    L, M, H, F = cfg["layers"], cfg["M"], cfg["hidden"], cfg["ffn"]
    say(f"packed stream: {L} full-shape layers, generated and packed on the device")
    pg, pu, pd = [], [], []
    for l in range(L):
        # pack layer by layer; only the last layer's standard-layout weights
        # are kept (the oracle reads them)
        wl = [synth.q4_0_weights_device(synth.stream_layer_seed(l, k), n, kk)
              for k, n, kk in (("gate", F, H), ("up", F, H), ("down", H, F))]
        pg.append(bq.q4_0_pack(wl[0]))
        pu.append(bq.q4_0_pack(wl[1]))
        pd.append(bq.q4_0_pack(wl[2]))
        if l == L - 1:
            wg, wu, wd = [wl[0]], [wl[1]], [wl[2]]
        del wl
    x0 = torch.from_numpy(synth.stream_x0()).to(DEV)
    y_prev, _ = bq.q4_0_ffn_stream(pg[:-1], pu[:-1], pd[:-1], x0, EPS, packed=True, ffn=F)
    y_prev = y_prev.clone()
    y, work = bq.q4_0_ffn_stream(pg, pu, pd, x0, EPS, packed=True, ffn=F)
    st = {k: host(v) for k, v in bq.stream_stages(work, M, H, F).items()}
    xq = host(bq.rms_norm_q8_1(y_prev, EPS))
    assert (xq == st["xq"]).all()
    # the joint gate/up launch of the last layer, rerun on the stream's own xq
    # with its optional outputs: products against the oracle (standard layout
    # of the same weights), h against SiLU(g)*u, hq against Q8_1(h) and the
    # stream's hq
    g = torch.empty((M, F), dtype=torch.float32, device=DEV)
    u, h = torch.empty_like(g), torch.empty_like(g)
    hq = host(bq.q4_0_gate_up_silu_q8_1_packed(pg[-1], pu[-1], F, H,
                                               torch.from_numpy(st["xq"]).to(DEV), M,
                                               g=g, u=u, h=h,
                                               ws=bq.q4_0_mmvq_packed_workspace()))
    gg, ug, hg = host(g), host(u), host(h)
    _gemv_check(wg[-1], st["xq"], M, gg, "gate")
    _gemv_check(wu[-1], st["xq"], M, ug, "up")
    ref = oracle.silu_mul(gg, ug)
    assert (np.abs(hg.astype(np.float64) - ref) <= REL * np.abs(ref) + ABS).all()
    assert (oracle.q8_1_quantize(hg) == hq).all()
    assert (hq == st["hq"]).all()
    _gemv_check(wd[-1], st["hq"], M, host(y), "down")


def test_packed_stream_stage_only_work_area_runs_unbalanced():
    """A work area that holds the stages but not the workspace: the pass runs
    the plain joint launch, and equals the composed calls made that way."""
    # ffn a multiple of 512 (the packed down projection's K) with 16 more
    # 32-column groups than CUs, so that the balanced pass cuts 16 groups
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    M, hidden, ffn, layers = 6, 512, 512 * (cus // 16 + 1), 2
    say(f"packed stream, stage-only work area M={M} hidden={hidden} ffn={ffn}")
    wg = [bq.q4_0_pack(synth.q4_0_weights_device(960 + 3 * l, ffn, hidden)) for l in range(layers)]
    wu = [bq.q4_0_pack(synth.q4_0_weights_device(961 + 3 * l, ffn, hidden)) for l in range(layers)]
    wd = [bq.q4_0_pack(synth.q4_0_weights_device(962 + 3 * l, hidden, ffn)) for l in range(layers)]
    x0 = torch.from_numpy(synth.stream_x0(M, hidden, seed=79)).to(DEV)
    total = bq.q4_0_ffn_stream_layout(M, hidden, ffn)["total"]
    stages = total - (bq.q4_0_mmvq_packed_ws_bytes() + 255) // 256 * 256
    work = torch.empty((stages,), dtype=torch.uint8, device=DEV)
    y = torch.empty((M, hidden), dtype=torch.float32, device=DEV)
    L = bq.lib()
    st = L.q4_0_ffn_stream_packed(bq.stream_weight_table(wg), bq.stream_weight_table(wu),
                                  bq.stream_weight_table(wd), layers, M, hidden, ffn,
                                  x0.data_ptr(), ctypes.c_float(EPS), y.data_ptr(),
                                  work.data_ptr(), stages,
                                  torch.cuda.current_stream().cuda_stream)
    assert st == 0
    # composed with the plain joint launch
    xq = bq.q8_1_quantize(x0)
    P = bq.q4_0_mmvq_packed_splits(hidden, ffn)
    parts = None
    for l in range(layers):
        if l > 0:
            xq = bq.rms_norm_q8_1_sum(parts, EPS)
        hq = bq.q4_0_gate_up_silu_q8_1_packed(wg[l], wu[l], ffn, hidden, xq, M)
        parts = bq.q4_0_mmvq_packed_split(wd[l], hidden, ffn, hq, M, P)
    y_ref = torch.empty_like(y)
    bq.rms_norm_q8_1_sum(parts, EPS, y=y_ref, want_xq=False)
    assert torch.equal(y, y_ref)
    # and the balanced pass (full work area) differs only by rounding in the
    # cut groups, which can move an h code by one step
    y_bal, _ = bq.q4_0_ffn_stream(wg, wu, wd, x0, EPS, packed=True, ffn=ffn)
    assert (y_bal - y).abs().max() <= 1e-3 * y.abs().max()
