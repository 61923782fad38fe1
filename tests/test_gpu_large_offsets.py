"""Weights past 2 GiB: the kernels' byte offsets outgrow 32 bits.

A Q4_0 weight of 270336 x 16384 (2.49 GB in the GGUF layout, its packed
nibble plane alone 2.2 GB) and a Q6_K head of 524288 x 5120 (expanded pack
2.87 GB, compact pack 2.2 GB), generated on the device.  Checked against the
oracle on sampled rows on both sides of the 2 GiB boundary and at the end of
the matrix: the GGUF-layout and packed products (M = 6 and 17, the balanced
and split launches included), and the head through a dominant row planted
past 2 GiB, a planted tie across the boundary (the lower id wins) and
candidate logits of rows past it, on both packs.
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
GIB2 = 1 << 31


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


def assert_close(gpu, ref, bound, what):
    err = np.abs(gpu.astype(np.float64) - ref)
    tol = REL * bound + ABS
    bad = err > tol
    if bad.any():
        i = np.argwhere(bad)[0]
        raise AssertionError(f"{what}: {bad.sum()} of {bad.size} outside tolerance; first at "
                             f"{tuple(i)}: gpu={gpu[tuple(i)]!r} ref={ref[tuple(i)]!r}")


def test_q4_0_products_past_2_gib():
    N, K = 270336, 16384
    row_bytes = K // 32 * 18
    first_high = GIB2 // row_bytes + 1  # first GGUF row that starts past 2 GiB
    assert N * K // 32 * 16 > GIB2  # the packed nibble plane too
    say(f"Q4_0 [{N} x {K}]: {N * row_bytes:,} bytes, generated on the device")
    wd = synth.q4_0_weights_device(61, N, K)
    x = synth.normal_rows(np.random.default_rng(62), 17, K)
    xqd = bq.q8_1_quantize(torch.from_numpy(x).to(DEV))
    xq = host(xqd)
    assert (xq == oracle.q8_1_quantize(x)).all()
    rng = np.random.default_rng(63)
    rows = np.unique(np.concatenate([
        [0, 1, 15, 16, first_high - 2, first_high - 1, first_high, first_high + 1],
        np.arange(N - 48, N),
        rng.integers(first_high, N, 40)]))
    w_rows = host(wd[torch.from_numpy(rows).to(DEV)])
    ref, bound = oracle.q4_0_gemv(w_rows, len(rows), K, xq, 17)
    sel = torch.from_numpy(rows).to(DEV)
    for m in (6, 17):
        say(f"q4_0_mmvq_m{m} (GGUF layout)")
        y = getattr(bq, f"q4_0_mmvq_m{m}")(wd, xqd)
        assert_close(host(y[:, sel]), ref[:m], bound[:m], f"GGUF m{m}")
    say("q4_0_pack")
    wp = bq.q4_0_pack(wd)
    del wd
    torch.cuda.empty_cache()
    ws = bq.q4_0_mmvq_packed_workspace()
    for m in (6, 17):
        for balanced in (False, True):
            say(f"q4_0_mmvq_packed M={m}{' (balanced)' if balanced else ''}")
            y = bq.q4_0_mmvq_packed(wp, N, K, xqd, m, ws=ws if balanced else None)
            assert_close(host(y[:, sel]), ref[:m], bound[:m], f"packed m{m} ws={balanced}")
        say(f"q4_0_mmvq_packed_split M={m}, 4 K ranges")
        yp = bq.q4_0_mmvq_packed_split(wp, N, K, xqd, m, 4)
        ysum = yp[0] + yp[1] + yp[2] + yp[3]
        assert_close(host(ysum[:, sel]), ref[:m], bound[:m], f"split m{m}")
    del wp
    torch.cuda.empty_cache()


def _dominant_raw_row(xrows, K):
    v = (xrows / np.linalg.norm(xrows, axis=1, keepdims=True)).sum(axis=0)
    q = np.clip(np.round(31 * v / np.abs(v).max()), -32, 31).astype(np.int8)[None, :]
    sc = np.full((1, K // 16), 63, np.int8)
    d = np.full((1, K // 256), np.float16(1e-3).view(np.uint16), np.uint16)
    return oracle.q6k_encode(q, sc, d, 1, K)[0]


def test_lm_head_past_2_gib():
    N, K = 524288, 5120
    assert N * K > GIB2  # the expanded quant plane
    first_high = GIB2 // K + 1  # first row whose expanded quants start past 2 GiB
    say(f"Q6_K [{N} x {K}] raw, generated on the device")
    rawd = synth.q6k_raw_weights_device(64, N, K)
    x = synth.normal_rows(np.random.default_rng(65), 6, K)
    xd = torch.from_numpy(x).to(DEV)
    packs = {False: bq.q6k_pack_expand(rawd, N, K), True: bq.q6k_pack_compact(rawd, N, K)}
    assert packs[False].numel() == bq.q6k_pack_bytes(N, K) > GIB2 + GIB2 // 4

    def repack():
        bq.q6k_pack_expand(rawd, N, K, packs[False])
        bq.q6k_pack_compact(rawd, N, K, packs[True])

    # candidate logits of rows past the boundary against the oracle
    cand = np.array([first_high, first_high + 63, N - 65, N - 64, N - 2, N - 1], np.int32)
    sub = oracle.q6k_pack_expand(host(rawd[torch.from_numpy(cand.astype(np.int64)).to(DEV)]),
                                 len(cand), K)
    ref, bound = oracle.q6k_pack_logits(sub, len(cand), K, oracle.q8_1_quantize(x[1:6]), 5)
    cd = torch.from_numpy(np.tile(cand, (5, 1))).to(DEV)
    got = {}
    for compact in (False, True):
        say(f"candidate logits ({'compact' if compact else 'expanded'} pack)")
        _, _, scores = bq.q6k_lmhead_candidate_max(packs[compact], N, K, xd, 1, 5, cand_ids=cd,
                                                   compact=compact)
        got[compact] = host(scores)
        assert_close(got[compact], ref, bound, f"candidate logits compact={compact}")
    assert (got[False].view(np.uint32) == got[True].view(np.uint32)).all()

    row = _dominant_raw_row(x[1:6], K)
    hi = N - 3
    for lo in (None, 100):
        planted = [hi] if lo is None else [lo, hi]
        say(f"dominant row planted at {planted}")
        orig = {r: rawd[r].clone() for r in planted}
        try:
            for r in planted:
                rawd[r] = torch.from_numpy(row).to(DEV)
            repack()
            for compact in (False, True):
                ids = host(bq.q6k_lmhead_top1(packs[compact], N, K, xd, 1, 5, compact=compact))
                assert list(ids) == [planted[0]] * 5, (planted, compact, list(ids))
        finally:
            for r in planted:
                rawd[r] = orig[r]
            repack()
            torch.cuda.synchronize()
    del packs, rawd
    torch.cuda.empty_cache()
