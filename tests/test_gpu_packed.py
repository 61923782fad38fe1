"""GPU parity of the offline-packed Q4_0 path (q4_0_pack, q4_0_mmvq_packed).

Bars: the packed bytes equal the oracle's packing bit for bit; products are
within |gpu - oracle| <= 1e-5 * sum_b |t_b| + 1e-6 of the oracle's product
read from the packed layout, for every M = 1..17, at shapes spanning several
16-row tiles with a ragged last tile, and at the full ffn_up and down_sweep
workloads.
"""
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


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


def assert_close(gpu, ref, bound, what):
    err = np.abs(gpu.astype(np.float64) - ref)
    tol = REL * bound + ABS
    bad = err > tol
    assert not bad.any(), (f"{what}: {bad.sum()} of {bad.size} outside tolerance; first at "
                           f"{tuple(np.argwhere(bad)[0])}")


SHAPES = [(1, 512), (5, 1024), (16, 512), (37, 1024), (200, 512), (1000, 1536), (16390, 512),
          (33, 5120)]


@pytest.mark.parametrize("N,K", SHAPES)
def test_pack_bitexact(N, K):
    say(f"q4_0_pack N={N} K={K}")
    w, _ = synth.random_q4_0_case(2000 + N + K, N, K, 1)
    wp = host(bq.q4_0_pack(dev(w)))
    assert (wp == oracle.q4_0_pack(w, N, K)).all()


@pytest.mark.parametrize("N,K", SHAPES)
def test_mmvq_packed_every_m(N, K):
    w, x = synth.random_q4_0_case(3000 + N + K, N, K, 17)
    xq = oracle.q8_1_quantize(x)
    wpo = oracle.q4_0_pack(w, N, K)
    ref, bound = oracle.q4_0p_gemv(wpo, N, K, xq, 17)
    wp = bq.q4_0_pack(dev(w))
    xqd = dev(xq)
    for m in range(1, 18):
        say(f"q4_0_mmvq_packed M={m} N={N} K={K}")
        y = host(bq.q4_0_mmvq_packed(wp, N, K, xqd[:m], m))
        assert_close(y, ref[:m], bound[:m], f"packed m{m} N{N} K{K}")


def test_mmvq_packed_ffn_up_full():
    w, x = synth.ffn_up()
    N, K, M = 17408, 5120, 6
    say("ffn_up full: packed M=6")
    xqd = bq.q8_1_quantize(dev(x))
    xq = host(xqd)
    ref, bound = oracle.q4_0_gemv(w, N, K, xq, M)
    wp = bq.q4_0_pack(dev(w))
    y = host(bq.q4_0_mmvq_packed(wp, N, K, xqd, M))
    assert_close(y, ref, bound, "ffn_up packed")
    # deterministic, and bitwise equal for equal weight rows in different tiles
    y2 = host(bq.q4_0_mmvq_packed(wp, N, K, xqd, M))
    assert (y2 == y).all()


def test_mmvq_packed_down_sweep_full():
    w, x = synth.down_sweep()
    N, K = 5120, 17408
    xqd = bq.q8_1_quantize(dev(x))
    xq = host(xqd)
    ref, bound = oracle.q4_0_gemv(w, N, K, xq, 17)
    wp = bq.q4_0_pack(dev(w))
    for m in synth.DOWN_SWEEP["Ms"]:
        say(f"down_sweep packed M={m}")
        y = host(bq.q4_0_mmvq_packed(wp, N, K, xqd[:m], m))
        assert_close(y, ref[:m], bound[:m], f"down packed m{m}")


def test_mmvq_packed_equal_rows_and_guard_bytes():
    N, K, M = 150, 1024, 6
    w, x = synth.random_q4_0_case(79, N, K, M)
    w[100] = w[5]                     # same weights in another tile
    w[149] = w[5]                     # and in the ragged last tile
    buf = torch.full((M * N + 64,), 12345.0, dtype=torch.float32, device=DEV)
    y = buf[:M * N].view(M, N)
    xqd = bq.q8_1_quantize(dev(x))
    bq.q4_0_mmvq_packed(bq.q4_0_pack(dev(w)), N, K, xqd, M, y)
    b = host(buf)
    assert (b[M * N:] == 12345.0).all()
    yy = b[:M * N].reshape(M, N)
    assert (yy[:, 100] == yy[:, 5]).all() and (yy[:, 149] == yy[:, 5]).all()


# Wide shapes with a ragged last tile (256 to 512 tiles, one to two per CU):
# every M class against the oracle, equal weight rows anywhere give bitwise
# equal outputs, nothing is written past y, and a split into one range is the
# whole product bit for bit.
WIDE_SHAPES = [(4097, 1024), (4111, 512), (8191, 2560), (6000, 5120), (4100, 1536)]


@pytest.mark.parametrize("N,K", WIDE_SHAPES)
def test_mmvq_packed_wide_ragged(N, K):
    w, x = synth.random_q4_0_case(3500 + N + K, N, K, 17)
    copies = [15, 16, 17, 33, 34, 35, N // 2, N - 2, N - 1]
    for r in copies:
        w[r] = w[0]                   # equal rows in other tiles, at tile edges
    xq = oracle.q8_1_quantize(x)
    ref, bound = oracle.q4_0_gemv(w, N, K, xq, 17)
    wp = bq.q4_0_pack(dev(w))
    xqd = dev(xq)
    for m in (1, 2, 3, 6, 8, 9, 16, 17):
        say(f"q4_0_mmvq_packed wide ragged M={m} N={N} K={K}")
        buf = torch.full((m * N + 64,), 12345.0, dtype=torch.float32, device=DEV)
        y = buf[:m * N].view(m, N)
        bq.q4_0_mmvq_packed(wp, N, K, xqd[:m], m, y)
        b = host(buf)
        assert (b[m * N:] == 12345.0).all()
        yy = b[:m * N].reshape(m, N)
        assert_close(yy, ref[:m], bound[:m], f"wide ragged m{m} N{N} K{K}")
        for r in copies:
            assert np.array_equal(yy[:, r].view(np.uint32), yy[:, 0].view(np.uint32)), r
        one = host(bq.q4_0_mmvq_packed_split(wp, N, K, xqd[:m], m, 1))
        assert np.array_equal(one[0].view(np.uint32), yy.view(np.uint32))


# From M = 9 a workgroup takes two 16-row tiles when N % 32 == 0 and there
# are at least as many such pairs (times the split count) as CUs.  These
# shapes take that path for the plain and the split launches: every M from 9
# to 17 against the oracle, equal weight rows in different pairs bitwise
# equal, and a single range bitwise the whole product.
def test_mmvq_packed_two_tile_workgroups():
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    N, K = 32 * (cus + 44), 1024
    w, x = synth.random_q4_0_case(3600, N, K, 17)
    copies = [16, 31, 32, 47, N // 2 + 1, N - 1]
    for r in copies:
        w[r] = w[3]
    xq = oracle.q8_1_quantize(x)
    ref, bound = oracle.q4_0_gemv(w, N, K, xq, 17)
    wp = bq.q4_0_pack(dev(w))
    xqd = dev(xq)
    for m in range(9, 18):
        say(f"q4_0_mmvq_packed two-tile workgroups M={m} N={N} K={K}")
        y = host(bq.q4_0_mmvq_packed(wp, N, K, xqd[:m], m))
        assert_close(y, ref[:m], bound[:m], f"two-tile m{m}")
        for r in copies:
            assert np.array_equal(y[:, r].view(np.uint32), y[:, 3].view(np.uint32)), r
        one = host(bq.q4_0_mmvq_packed_split(wp, N, K, xqd[:m], m, 1))
        assert np.array_equal(one[0].view(np.uint32), y.view(np.uint32))
        parts = host(bq.q4_0_mmvq_packed_split(wp, N, K, xqd[:m], m, 3))
        assert_close(part_sum(parts), ref[:m], bound[:m], f"two-tile split 3 m{m}")


def part_sum(parts):
    """Sum of partial rows in part order, in binary32 (the documented order)."""
    y = parts[0].copy()
    for p in range(1, parts.shape[0]):
        y += parts[p]
    return y


@pytest.mark.parametrize("N,K,splits", [(37, 1024, (1, 2, 3, 4)), (200, 2560, (2, 5, 8)),
                                        (33, 5120, (3, 7)), (16, 512, (2,))])
def test_mmvq_packed_split_ranges(N, K, splits):
    w, x = synth.random_q4_0_case(4000 + N + K, N, K, 17)
    xq = oracle.q8_1_quantize(x)
    wp = bq.q4_0_pack(dev(w))
    xqd = dev(xq)
    for m in (1, 6, 17):
        ref, bound = oracle.q4_0_gemv(w, N, K, xq[:m], m)
        whole = host(bq.q4_0_mmvq_packed(wp, N, K, xqd[:m], m))
        for p in splits:
            say(f"q4_0_mmvq_packed_split M={m} N={N} K={K} nsplit={p}")
            parts = host(bq.q4_0_mmvq_packed_split(wp, N, K, xqd[:m], m, p))
            assert parts.shape == (p, m, N)
            assert_close(part_sum(parts), ref, bound, f"split {p} m{m}")
            if p == 1:
                assert np.array_equal(parts[0].view(np.uint32), whole.view(np.uint32))


def test_mmvq_packed_split_ranges_are_the_documented_chunks():
    """Part p holds exactly the blocks of chunks floor(p*C/P) .. floor((p+1)*C/P)-1:
    weights that are zero outside one range give zero in every other part."""
    N, K, M, P = 48, 2560, 6, 3           # C = 10 chunks: ranges 0-2, 3-5, 6-9
    w, x = synth.random_q4_0_case(4100, N, K, M)
    xq = oracle.q8_1_quantize(x)
    nb = K // 32
    blocks = w.reshape(N, nb, 18).copy()
    blocks[:, :, 0:2] = 0                 # d = 0 everywhere ...
    keep = slice(6 * 8, 10 * 8)           # ... except in chunks 6..9 (range 2)
    src = w.reshape(N, nb, 18)
    blocks[:, keep, 0:2] = src[:, keep, 0:2]
    wz = blocks.reshape(N, nb * 18)
    parts = host(bq.q4_0_mmvq_packed_split(bq.q4_0_pack(dev(wz)), N, K, dev(xq), M, P))
    assert not parts[0].any() and not parts[1].any()
    ref, bound = oracle.q4_0_gemv(wz, N, K, xq, M)
    assert_close(parts[2], ref, bound, "range 2")


def test_mmvq_packed_split_down_full():
    w, x = synth.down_sweep()
    N, K = 5120, 17408
    P = bq.q4_0_mmvq_packed_splits(N, K)
    assert P == 4
    xqd = bq.q8_1_quantize(dev(x))
    xq = host(xqd)
    ref, bound = oracle.q4_0_gemv(w, N, K, xq, 17)
    wp = bq.q4_0_pack(dev(w))
    for m in (1, 6, 17):
        say(f"down split {P} M={m}")
        parts = host(bq.q4_0_mmvq_packed_split(wp, N, K, xqd[:m], m, P))
        assert_close(part_sum(parts), ref[:m], bound[:m], f"down split m{m}")


def test_mmvq_packed_split_rows_count_down_full():
    """The per-M split count at the down shape: the shape's count up to
    M = 10, then a count whose two-tile workgroups are all resident; its
    split launch meets the oracle bar at M = 11, 12 and 17."""
    w, x = synth.down_sweep()
    N, K = 5120, 17408
    counts = {m: bq.q4_0_mmvq_packed_splits_rows(N, K, m) for m in range(1, 18)}
    say(f"split counts {counts}")
    for m in range(1, 11):
        assert counts[m] == bq.q4_0_mmvq_packed_splits(N, K)
    for m in range(11, 18):
        assert 2 <= counts[m] <= 8
    import torch

    if torch.cuda.get_device_properties(0).multi_processor_count == 256:
        # 160 two-tile units: 3 ranges put 480 workgroups 1 or 2 to a CU
        assert all(counts[m] == 3 for m in range(11, 18)), counts
    xqd = bq.q8_1_quantize(dev(x))
    xq = host(xqd)
    ref, bound = oracle.q4_0_gemv(w, N, K, xq, 17)
    wp = bq.q4_0_pack(dev(w))
    for m in (11, 12, 17):
        P = counts[m]
        say(f"down split {P} M={m}")
        parts = host(bq.q4_0_mmvq_packed_split(wp, N, K, xqd[:m], m, P))
        assert_close(part_sum(parts), ref[:m], bound[:m], f"down split {P} m{m}")


@pytest.mark.parametrize("P,M,K", [(4, 6, 5120), (1, 6, 5120), (3, 17, 1056), (8, 2, 32768),
                                   (2, 1, 32)])
def test_rms_norm_q8_1_sum(P, M, K):
    say(f"rms_norm_q8_1_sum P={P} M={M} K={K}")
    rng = np.random.default_rng(4200 + P + M + K)
    parts = (rng.standard_normal((P, M, K)) * 10).astype(np.float32)
    y = torch.empty((M, K), dtype=torch.float32, device=DEV)
    x = torch.empty_like(y)
    xq = host(bq.rms_norm_q8_1_sum(dev(parts), 1e-6, y=y, x=x))
    yg, xg = host(y), host(x)
    assert np.array_equal(yg.view(np.uint32), part_sum(parts).view(np.uint32))
    ref = oracle.rms_norm(yg, 1e-6)
    assert (np.abs(xg.astype(np.float64) - ref) <= REL * np.abs(ref) + ABS).all()
    assert (xq == oracle.q8_1_quantize(xg)).all()
    # the same step on the summed rows through rms_norm_q8_1: bitwise equal
    assert (host(bq.rms_norm_q8_1(y, 1e-6)) == xq).all()
    # y only
    y2 = torch.empty_like(y)
    assert bq.rms_norm_q8_1_sum(dev(parts), 1e-6, y=y2, want_xq=False) is None
    assert torch.equal(y2, y)


# The balanced launch (q4_0_mmvq_packed_ws): for M >= 9 the tiles past the
# last multiple of the CU count are cut into min(4, K/256) ranges of K whose
# sums meet in the workspace (M <= 8: no tile is cut; from M = 11 with fewer
# 32-row tile pairs than CUs, as at the down shape, every pair is cut).  Outputs of the other tiles are bitwise the plain
# launch's; the cut tiles' are within the oracle's tolerance; results repeat
# bit for bit.  Shapes: fewer tiles than CUs (every tile cut), a remainder
# with a ragged last tile, the full ffn_up and down shapes, every M = 1..17
# (the bench times the M = 12 launch at the down shape).  One workspace
# serves every shape and M in turn, and its counters are back at zero after
# each call.
WS_SMALL = [(1, 512), (37, 1024), (150, 1024), (4097, 1024), (6000, 5120)]
WS_FULL = [(17408, 5120), (5120, 17408)]


def _cus():
    return torch.cuda.get_device_properties(0).multi_processor_count


def _ws_count_bytes():
    return (_cus() * 4 + 255) // 256 * 256


def _whole_rows(N, K, M):
    if M <= 8:
        return N
    if M >= 11 and N % 32 == 0 and N // 32 < _cus():
        # fewer tile pairs than CUs: every pair is cut into the per-M split count
        P = bq.q4_0_mmvq_packed_splits_rows(N, K, M)
        if P >= 2 and N // 32 * P >= _cus():
            return 0
    tiles = (N + 15) // 16
    return min(N, 16 * (tiles - tiles % _cus()))


def test_mmvq_packed_ws_small():
    ws = bq.q4_0_mmvq_packed_workspace()
    assert ws.numel() == bq.q4_0_mmvq_packed_ws_bytes()
    for N, K in WS_SMALL:
        w, x = synth.random_q4_0_case(5100 + N + K, N, K, 17)
        xq = oracle.q8_1_quantize(x)
        ref, bound = oracle.q4_0_gemv(w, N, K, xq, 17)
        wp, xqd = bq.q4_0_pack(dev(w)), dev(xq)
        for m in range(1, 18):
            r0 = _whole_rows(N, K, m)
            say(f"q4_0_mmvq_packed_ws N={N} K={K} M={m} (rows {r0}.. cut into K ranges)")
            plain = host(bq.q4_0_mmvq_packed(wp, N, K, xqd[:m], m))
            yw = host(bq.q4_0_mmvq_packed(wp, N, K, xqd[:m], m, ws=ws))
            assert_close(yw, ref[:m], bound[:m], f"ws N{N} K{K} m{m}")
            assert np.array_equal(yw[:, :r0].view(np.uint32), plain[:, :r0].view(np.uint32))
            again = host(bq.q4_0_mmvq_packed(wp, N, K, xqd[:m], m, ws=ws))
            assert np.array_equal(again.view(np.uint32), yw.view(np.uint32))
            assert not host(ws[:_ws_count_bytes()]).any()


@pytest.mark.parametrize("N,K", WS_FULL)
def test_mmvq_packed_ws_full(N, K):
    ws = bq.q4_0_mmvq_packed_workspace()
    wd = synth.q4_0_weights_device(5200 + N, N, K)
    r0 = min(_whole_rows(N, K, m) for m in range(9, 18))
    w_cut = host(wd[r0:])                       # the cut tiles' rows, for the oracle
    wp = bq.q4_0_pack(wd)
    xqd = bq.q8_1_quantize(torch.randn((17, K), device=DEV))
    xq = host(xqd)
    ref, bound = oracle.q4_0_gemv(w_cut, N - r0, K, xq, 17)
    for m in range(1, 18):
        say(f"q4_0_mmvq_packed_ws full N={N} K={K} M={m} (rows {r0}.. cut)")
        plain = host(bq.q4_0_mmvq_packed(wp, N, K, xqd[:m], m))
        yw = host(bq.q4_0_mmvq_packed(wp, N, K, xqd[:m], m, ws=ws))
        whole = _whole_rows(N, K, m)
        assert np.array_equal(yw[:, :whole].view(np.uint32), plain[:, :whole].view(np.uint32))
        assert_close(yw[:, r0:], ref[:m], bound[:m], f"ws full cut rows m{m}")
        again = host(bq.q4_0_mmvq_packed(wp, N, K, xqd[:m], m, ws=ws))
        assert np.array_equal(again.view(np.uint32), yw.view(np.uint32))
        assert not host(ws[:_ws_count_bytes()]).any()


def test_mmvq_packed_ws_rejects_small_or_misaligned_workspace():
    N, K, M = 37, 1024, 6
    w, x = synth.random_q4_0_case(5300, N, K, M)
    wp, xqd = bq.q4_0_pack(dev(w)), bq.q8_1_quantize(dev(x))
    ws = bq.q4_0_mmvq_packed_workspace()
    y = torch.full((M, N), 7.0, device=DEV)
    with pytest.raises(bq.Bq8Error) as e:
        bq.q4_0_mmvq_packed(wp, N, K, xqd, M, y, ws=ws[:ws.numel() - 1])
    assert e.value.status == 4
    with pytest.raises(bq.Bq8Error) as e:
        bq.q4_0_mmvq_packed(wp, N, K, xqd, M, y, ws=ws[16:])
    assert e.value.status == 3
    assert (host(y) == 7.0).all()


def test_mmvq_packed_ws_two_streams_own_workspaces():
    """Two streams, each with its own workspace, run cut launches (M = 17,
    tiles past the last multiple of the CU count) at the same time: every
    result equals the single-stream result bit for bit."""
    N, K, M = 16 * (_cus() + 37), 2048, 17
    w, x = synth.random_q4_0_case(5400, N, K, M)
    wp, xqd = bq.q4_0_pack(dev(w)), bq.q8_1_quantize(dev(x))
    want = host(bq.q4_0_mmvq_packed(wp, N, K, xqd, M, ws=bq.q4_0_mmvq_packed_workspace()))
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    spaces = [bq.q4_0_mmvq_packed_workspace() for _ in streams]
    outs = [[torch.empty((M, N), device=DEV) for _ in range(6)] for _ in streams]
    torch.cuda.synchronize()
    say(f"q4_0_mmvq_packed_ws on two streams N={N} K={K} M={M}")
    for k in range(6):
        for s, ws, o in zip(streams, spaces, outs):
            with torch.cuda.stream(s):
                bq.q4_0_mmvq_packed(wp, N, K, xqd, M, o[k], ws=ws)
    torch.cuda.synchronize()
    for o in outs:
        for y in o:
            assert np.array_equal(host(y).view(np.uint32), want.view(np.uint32))
    for ws in spaces:
        assert not host(ws[:_ws_count_bytes()]).any()
