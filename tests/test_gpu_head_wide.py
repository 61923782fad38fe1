"""GPU parity of the fused Q6_K head on wide vocabularies: at least 3600
tiles of 64 rows (230,400 rows), where the head runs one wave per whole tile
with no superblock split, as at the full 248,320-row head.  Short K keeps
the oracle quick.

Cases: ragged last tiles of 1, 15, 17 and 63 rows; every activation-row
count 1..8 at several first rows; planted duplicate dominant rows at
16-row, tile and vocabulary edges, where the lower id must win; candidates,
including out-of-range ids and ids at the edges; all-zero activations.
Bars as the other head tests: ids equal to the oracle's or within the
block-term tolerance of its maximum; top values and candidate scores within
1e-5 * sum|terms| + 1e-6 of the oracle's logits.  The compact pack gives
the expanded pack's ids, top values and candidate scores bit for bit.
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
WIDE = 3600 * 64  # the narrowest vocabulary the head runs without a superblock split


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


def edge_candidates(oid, N, rows):
    out = np.empty((rows, 8), np.int32)
    for r in range(rows):
        out[r] = [int(oid[r]), 0, N - 1, 15, 16, WIDE, -1, N]
    return out


def run_both(raw, N, K, x, row0, rows, cand):
    """The head on the expanded and the compact pack of raw: (ids, vals,
    scores) of each, after checking the compact pack against the oracle's."""
    pack = dev(oracle.q6k_pack_expand(raw, N, K))
    cpack_ref = oracle.q6k_pack_compact(raw, N, K)
    cpack = bq.q6k_pack_compact(dev(raw), N, K)
    assert (host(cpack) == cpack_ref).all()
    out = []
    for p, compact in ((pack, False), (cpack, True)):
        res = bq.q6k_lmhead_candidate_max(p, N, K, dev(x), row0, rows,
                                          None if cand is None else dev(cand), compact=compact)
        out.append(tuple(host(t) for t in res))
    return out


@pytest.mark.parametrize("N,K,row0,rows", [
    (WIDE + 1, 256, 1, 5),     # last tile 1 row: groups 1..3 past the end
    (WIDE + 15, 512, 0, 8),    # last tile 15 rows: group 0 ragged
    (WIDE + 17, 256, 2, 1),    # last tile 17 rows: group 1 holds one row
    (WIDE + 63, 768, 1, 5),    # last tile 63 rows: group 3 ragged
    (WIDE + 63, 256, 0, 6),
    (WIDE, 256, 1, 2), (WIDE, 256, 0, 3), (WIDE + 40, 256, 3, 4), (WIDE + 1, 256, 0, 7),
])
def test_wide_vocabulary_every_row_count(N, K, row0, rows):
    rng = np.random.default_rng(900 + N % 97 + K + 10 * rows + row0)
    raw = synth.q6k_raw_weights(rng, N, K)
    x = synth.normal_rows(rng, row0 + rows + 1, K)
    say(f"wide head N={N} K={K} row0={row0} rows={rows}")
    oid, logits, bound, _ = oracle.q6k_lmhead_top1(oracle.q6k_pack_expand(raw, N, K), N, K, x,
                                                   row0, rows)
    cand = edge_candidates(oid, N, rows)
    (ids, vals, scores), (cids, cvals, cscores) = run_both(raw, N, K, x, row0, rows, cand)
    check_ids(ids, oid, logits, bound, what=f"wide N={N} rows={rows}")
    for r in range(rows):
        g = ids[r]
        assert abs(float(vals[r]) - logits[r, g]) <= REL * bound[r, g] + ABS
        for c, cid in enumerate(cand[r]):
            s = scores[r, c]
            if not 0 <= cid < N:
                assert np.isnan(s), (r, cid, s)
                continue
            assert abs(float(s) - logits[r, cid]) <= REL * bound[r, cid] + ABS, (r, cid)
            if cid == g:
                assert np.float32(s).view(np.uint32) == np.float32(vals[r]).view(np.uint32)
    assert (cids == ids).all()
    assert (cvals.view(np.uint32) == vals.view(np.uint32)).all()
    assert (cscores.view(np.uint32) == scores.view(np.uint32)).all()


def _dominant_raw_row(xrows, K):
    """A raw Q6_K row whose logit exceeds every random row's for all given
    activation rows: quants follow the sign pattern of sum_r x_r/|x_r|, with
    the largest subscale and d = 1e-3 (encoded by the oracle's codec)."""
    v = (xrows / np.linalg.norm(xrows, axis=1, keepdims=True)).sum(axis=0)
    q = np.clip(np.round(31 * v / np.abs(v).max()), -32, 31).astype(np.int8)[None, :]
    sc = np.full((1, K // 16), 63, np.int8)
    d = np.full((1, K // 256), np.float16(1e-3).view(np.uint16), np.uint16)
    return oracle.q6k_encode(q, sc, d, 1, K)[0]


@pytest.mark.parametrize("lo,hi", [(15, 16), (47, 48), (63, 64), (WIDE - 1, WIDE),
                                   (WIDE, WIDE + 16), (0, WIDE + 16)])
def test_wide_vocabulary_planted_ties(lo, hi):
    N, K = WIDE + 17, 256
    rng = np.random.default_rng(950)
    raw = synth.q6k_raw_weights(rng, N, K)
    x = synth.normal_rows(rng, 6, K)
    raw[lo] = raw[hi] = _dominant_raw_row(x[1:6], K)
    say(f"wide head tie ({lo},{hi})")
    oid, _, _, _ = oracle.q6k_lmhead_top1(oracle.q6k_pack_expand(raw, N, K), N, K, x, 1, 5)
    assert list(oid) == [lo] * 5
    (ids, vals, _), (cids, cvals, _) = run_both(raw, N, K, x, 1, 5, None)
    assert list(ids) == [lo] * 5
    assert (cids == ids).all()
    assert (cvals.view(np.uint32) == vals.view(np.uint32)).all()


def test_wide_vocabulary_zero_activations():
    N, K = WIDE + 15, 256
    rng = np.random.default_rng(960)
    raw = synth.q6k_raw_weights(rng, N, K)
    x = np.zeros((6, K), np.float32)
    (ids, vals, _), (cids, cvals, _) = run_both(raw, N, K, x, 0, 6, None)
    assert list(ids) == [0] * 6 and list(cids) == [0] * 6
    assert (vals.view(np.uint32) == 0).all() and (cvals.view(np.uint32) == 0).all()
