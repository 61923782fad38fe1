"""GPU parity on seeded random shapes: the shape combinations the fixed lists
of the other tests do not name (ragged row counts against every M class, K
from one chunk to many, the cut and split launches at small grids, vocabulary
sizes that end mid-tile, any row window of the head).

Every draw comes from one seeded generator, so a failure names a shape that
reruns the same way.  The bars are those of the fixed-shape tests: Q8_1 bytes
and the head's ids bit for bit (ids up to a near tie inside the float bound,
tests/idcheck.py), float outputs within 1e-5 * sum_b |t_b| + 1e-6 of the
oracle.
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
from idcheck import check_ids  # noqa: E402
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


def _draws():
    rng = np.random.default_rng(9000)
    q8 = [(int(rng.integers(1, 18)), 32 * int(rng.integers(1, 200))) for _ in range(20)]
    gguf = [(int(rng.integers(1, 3001)), 32 * int(rng.integers(1, 129)), int(rng.integers(1, 18)))
            for _ in range(30)]
    packed = []
    for _ in range(30):
        K = 512 * int(rng.integers(1, 9))
        packed.append((int(rng.integers(1, 3001)), K, int(rng.integers(1, 18)),
                       int(rng.integers(1, min(8, K // 256) + 1))))
    joint = [(32 * int(rng.integers(1, 101)), 512 * int(rng.integers(1, 7)),
              int(rng.integers(1, 18))) for _ in range(20)]
    head = []
    for _ in range(24):
        rows = int(rng.integers(1, 9))
        M = rows + int(rng.integers(0, 3))
        head.append((int(rng.integers(1, 5001)), 256 * int(rng.integers(1, 9)), M,
                     int(rng.integers(0, M - rows + 1)), rows, int(rng.integers(0, 9))))
    glue = [(int(rng.integers(1, 18)), 32 * int(rng.integers(1, 400)), int(rng.integers(1, 5)))
            for _ in range(16)]
    return q8, gguf, packed, joint, head, glue


Q8, GGUF, PACKED, JOINT, HEAD, GLUE = _draws()


def _name(t):
    return "-".join(str(v) for v in t)


@pytest.mark.parametrize("M,K", Q8, ids=[_name(t) for t in Q8])
def test_random_q8_1_quantize(M, K):
    rng = np.random.default_rng(9100 + M * 7919 + K)
    x = synth.normal_rows(rng, M, K)
    x *= np.exp(rng.uniform(-12, 12, (M, K // 32, 1))).astype(np.float32).repeat(32, 2).reshape(M, K)
    say(f"q8_1_quantize M={M} K={K}")
    assert (host(bq.q8_1_quantize(dev(x))) == oracle.q8_1_quantize(x)).all()


@pytest.mark.parametrize("N,K,M", GGUF, ids=[_name(t) for t in GGUF])
def test_random_gguf_product(N, K, M):
    w, x = synth.random_q4_0_case(9200 + N + K + M, N, K, M)
    xq = oracle.q8_1_quantize(x)
    ref, bound = oracle.q4_0_gemv(w, N, K, xq, M)
    say(f"q4_0_mmvq M={M} N={N} K={K}")
    y = host(bq.q4_0_mmvq(dev(w), dev(xq), M))
    assert_close(y, ref, bound, f"gguf M{M} N{N} K{K}")


@pytest.fixture(scope="module")
def workspace():
    return bq.q4_0_mmvq_packed_workspace()


@pytest.mark.parametrize("N,K,M,nsplit", PACKED, ids=[_name(t) for t in PACKED])
def test_random_packed_products(N, K, M, nsplit, workspace):
    w, x = synth.random_q4_0_case(9300 + N + K + M, N, K, M)
    xq = oracle.q8_1_quantize(x)
    ref, bound = oracle.q4_0_gemv(w, N, K, xq, M)
    wp, xqd = bq.q4_0_pack(dev(w)), dev(xq)
    say(f"q4_0_mmvq_packed M={M} N={N} K={K}")
    y = host(bq.q4_0_mmvq_packed(wp, N, K, xqd, M))
    assert_close(y, ref, bound, f"packed M{M} N{N} K{K}")
    say(f"q4_0_mmvq_packed_ws M={M} N={N} K={K}")
    yw = host(bq.q4_0_mmvq_packed(wp, N, K, xqd, M, ws=workspace))
    assert_close(yw, ref, bound, f"packed_ws M{M} N{N} K{K}")
    yw2 = host(bq.q4_0_mmvq_packed(wp, N, K, xqd, M, ws=workspace))
    assert np.array_equal(yw.view(np.uint32), yw2.view(np.uint32)), "balanced launch not reproducible"
    say(f"q4_0_mmvq_packed_split M={M} N={N} K={K} nsplit={nsplit}")
    parts = bq.q4_0_mmvq_packed_split(wp, N, K, xqd, M, nsplit)
    ysum = parts[0].clone()
    for p in range(1, nsplit):
        ysum += parts[p]
    assert_close(host(ysum), ref, bound, f"split M{M} N{N} K{K} nsplit{nsplit}")
    if nsplit == 1:
        assert np.array_equal(host(parts[0]).view(np.uint32), y.view(np.uint32))


@pytest.mark.parametrize("N,K,M", JOINT, ids=[_name(t) for t in JOINT])
def test_random_joint_gate_up(N, K, M, workspace):
    rng = np.random.default_rng(9400 + N + K + M)
    wg = synth.q4_0_weights(rng, N, K)
    wu = synth.q4_0_weights(rng, N, K)
    x = synth.normal_rows(rng, M, K)
    xq = oracle.q8_1_quantize(x)
    pg, pu, xqd = bq.q4_0_pack(dev(wg)), bq.q4_0_pack(dev(wu)), dev(xq)
    ref_g, bound_g = oracle.q4_0_gemv(wg, N, K, xq, M)
    ref_u, bound_u = oracle.q4_0_gemv(wu, N, K, xq, M)
    for ws in (None, workspace):
        say(f"q4_0_gate_up_silu_q8_1_packed{'_ws' if ws is not None else ''} M={M} N={N} K={K}")
        g = torch.empty((M, N), dtype=torch.float32, device=DEV)
        u, h = torch.empty_like(g), torch.empty_like(g)
        hq = host(bq.q4_0_gate_up_silu_q8_1_packed(pg, pu, N, K, xqd, M, g=g, u=u, h=h, ws=ws))
        gg, ug, hg = host(g), host(u), host(h)
        assert_close(gg, ref_g, bound_g, f"gate M{M} N{N} K{K}")
        assert_close(ug, ref_u, bound_u, f"up M{M} N{N} K{K}")
        ref_h = oracle.silu_mul(gg, ug)
        assert (np.abs(hg.astype(np.float64) - ref_h) <= REL * np.abs(ref_h) + ABS).all()
        assert (hq == oracle.q8_1_quantize(hg)).all(), "hq differs from Q8_1 of the GPU's h"


@pytest.mark.parametrize("N,K,M,row0,rows,ncand", HEAD, ids=[_name(t) for t in HEAD])
def test_random_lm_head(N, K, M, row0, rows, ncand):
    rng = np.random.default_rng(9500 + N + K + M)
    raw = synth.q6k_raw_weights(rng, N, K)
    x = synth.normal_rows(rng, M, K)
    pack = oracle.q6k_pack_expand(raw, N, K)
    oid, logits, bound, _ = oracle.q6k_lmhead_top1(pack, N, K, x, row0, rows)
    rawd, xd = dev(raw), dev(x)
    packs = {False: bq.q6k_pack_expand(rawd, N, K), True: bq.q6k_pack_compact(rawd, N, K)}
    # candidates: in range mostly, one past the vocabulary when there is room
    cand = rng.integers(0, N, (rows, ncand)).astype(np.int32)
    if ncand:
        cand[0, -1] = N
    got = {}
    for compact in (False, True):
        kind = "compact" if compact else "expanded"
        say(f"q6k head ({kind}) N={N} K={K} M={M} row0={row0} rows={rows} ncand={ncand}")
        ids = host(bq.q6k_lmhead_top1(packs[compact], N, K, xd, row0, rows, compact=compact))
        check_ids(ids, oid, logits, bound, f"ids {kind}")
        cids, vals, scores = bq.q6k_lmhead_candidate_max(
            packs[compact], N, K, xd, row0, rows, cand_ids=dev(cand) if ncand else None,
            compact=compact)
        cids, vals, scores = host(cids), host(vals), host(scores)
        assert (cids == ids).all(), "candidate-max ids differ from top-1 ids"
        assert_close(vals, logits[np.arange(rows), ids], bound[np.arange(rows), ids],
                     f"top values {kind}")
        if ncand:
            inr = cand < N
            ref = logits[np.arange(rows)[:, None], np.where(inr, cand, 0)]
            bnd = bound[np.arange(rows)[:, None], np.where(inr, cand, 0)]
            assert np.isnan(scores[~inr]).all(), "out-of-range candidates must read NaN"
            assert_close(np.where(inr, scores, 0), np.where(inr, ref, 0), np.where(inr, bnd, 0),
                         f"candidate scores {kind}")
        got[compact] = (ids, vals, scores)
    for a, b in zip(got[False], got[True]):
        assert np.array_equal(a.view(np.uint32), b.view(np.uint32)), "compact differs from expanded"


@pytest.mark.parametrize("M,K,P", GLUE, ids=[_name(t) for t in GLUE])
def test_random_glue(M, K, P):
    rng = np.random.default_rng(9600 + M + K + P)
    parts = (rng.standard_normal((P, M, K)) * 20).astype(np.float32)
    say(f"rms_norm_q8_1_sum P={P} M={M} K={K}")
    y = torch.empty((M, K), dtype=torch.float32, device=DEV)
    xo = torch.empty_like(y)
    xq = host(bq.rms_norm_q8_1_sum(dev(parts), 1e-6, y=y, x=xo))
    ysum = parts[0].copy()
    for p in range(1, P):
        ysum = (ysum + parts[p]).astype(np.float32)
    assert np.array_equal(host(y).view(np.uint32), ysum.view(np.uint32)), "part-order sum"
    xg = host(xo)
    ref = oracle.rms_norm(ysum, 1e-6)
    assert (np.abs(xg.astype(np.float64) - ref) <= REL * np.abs(ref) + ABS).all()
    assert (xq == oracle.q8_1_quantize(xg)).all()
    say(f"silu_mul_q8_1 M={M} N={K}")
    g = (rng.standard_normal((M, K)) * 4).astype(np.float32)
    u = (rng.standard_normal((M, K)) * 2).astype(np.float32)
    h = torch.empty((M, K), dtype=torch.float32, device=DEV)
    hq = host(bq.silu_mul_q8_1(dev(g), dev(u), h=h))
    hg = host(h)
    ref_h = oracle.silu_mul(g, u)
    assert (np.abs(hg.astype(np.float64) - ref_h) <= REL * np.abs(ref_h) + ABS).all()
    assert (hq == oracle.q8_1_quantize(hg)).all()
