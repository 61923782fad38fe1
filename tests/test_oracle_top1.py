"""Pins for the oracle's greedy top-1 and the fused LM-head boundary.

"Q6_K M=6 fused DFlash top-1 production record", section "Exactness and
safety contracts": the reducer follows a lowest-token-ID finite-tie contract,
checked with full-vocabulary zero ties and crossing ties 1/256, 255/256 and
0/248319.  Only rows 1..5 of the six-row draft block are projected
("Outcome").
"""
import os

import numpy as np
import pytest

from block_quantized_gemv_q8_amd import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _tie_pairs():
    out = []
    with open(os.path.join(GOLDEN, "lm_head_tie_pairs.txt")) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if line:
                out.append(tuple(int(v) for v in line.split()))
    return out


def test_matches_numpy_argmax_first_occurrence(orc):
    rng = np.random.default_rng(31)
    logits = rng.standard_normal((7, 5000))
    logits[3, 100] = logits[3, 4000] = logits[3].max() + 1.0
    logits[4] = np.round(logits[4] * 2)          # many exact ties
    assert (orc.top1(logits) == np.argmax(logits, axis=1)).all()


@pytest.mark.parametrize("pair", _tie_pairs())
def test_planted_tie_pairs(orc, pair):
    lo, hi = pair
    N = 248320
    rng = np.random.default_rng(lo * 7 + hi)
    logits = rng.standard_normal((2, N))
    logits[:, lo] = logits[:, hi] = 10.0
    assert list(orc.top1(logits)) == [lo, lo]
    # and in reverse placement order the lower id still wins
    logits[:, [lo, hi]] = logits[:, [hi, lo]]
    assert list(orc.top1(logits)) == [lo, lo]


def test_zero_vocabulary_and_signed_zero(orc):
    assert list(orc.top1(np.zeros((5, 248320)))) == [0] * 5
    assert orc.top1(np.array([[-0.0, 0.0, -0.0]]))[0] == 0
    assert orc.top1(np.array([[-1.0, -0.0, 0.0]]))[0] == 1
    assert orc.top1(np.array([[np.nan, -3.0, -2.0]]))[0] == 2


def test_bruteforce_tiny_vocabularies(orc):
    # every assignment of values {0,1,2} to 6 ids: the answer is the first max
    import itertools

    for vals in itertools.product([0.0, 1.0, 2.0], repeat=6):
        v = np.array([vals])
        expect = min(i for i, x in enumerate(vals) if x == max(vals))
        assert orc.top1(v)[0] == expect


def test_fused_boundary_small(orc):
    rng = np.random.default_rng(33)
    N, K, M, row0, rows = 700, 512, 6, 1, 5
    raw = synth.q6k_raw_weights(rng, N, K)
    pack = orc.q6k_pack_expand(raw, N, K)
    x = synth.normal_rows(rng, M, K)
    ids, logits, bound, xq = orc.q6k_lmhead_top1(pack, N, K, x, row0, rows)
    # the boundary quantizes exactly rows 1..5 and nothing of row 0
    assert (xq == orc.q8_1_quantize(x[row0:row0 + rows])).all()
    ref, _ = orc.q6k_pack_logits(pack, N, K, xq, rows)
    assert (logits == ref).all()
    assert (ids == np.argmax(ref, axis=1)).all()
    # changing row 0 changes nothing
    x2 = x.copy()
    x2[0] = 1e3
    ids2, _, _, _ = orc.q6k_lmhead_top1(pack, N, K, x2, row0, rows)
    assert (ids2 == ids).all()


def test_fused_boundary_planted_duplicates(orc):
    # duplicate a weight row: the two logits are identical, lowest id wins
    rng = np.random.default_rng(34)
    N, K = 600, 256
    raw = synth.q6k_raw_weights(rng, N, K)
    x = synth.normal_rows(rng, 6, K)
    pack = orc.q6k_pack_expand(raw, N, K)
    ids, logits, _, _ = orc.q6k_lmhead_top1(pack, N, K, x, 1, 5)
    for r, best in enumerate(ids):
        raw2 = raw.copy()
        dup = (best + 97) % N
        raw2[dup] = raw2[best]
        pack2 = orc.q6k_pack_expand(raw2, N, K)
        ids2, l2, _, _ = orc.q6k_lmhead_top1(pack2, N, K, x, 1, 5)
        assert l2[r, dup] == l2[r, best]
        assert ids2[r] == min(best, dup)
    # all-zero activations: every logit is zero, the answer is id 0
    ids0, l0, _, _ = orc.q6k_lmhead_top1(pack, N, K, np.zeros((6, K), np.float32), 1, 5)
    assert not l0.any() and list(ids0) == [0] * 5
