"""GPU parity of the fused Q6_K head's variants: all six rows of the target
side, the candidate-max outputs (q6k_lmhead_candidate_max), and the compact
pack (q6k_pack_compact, q6k_lmhead_*_compact).

Bars: ids as the top-1 tests (equal to the oracle's, or within the
block-term tolerance of its maximum when two logits are that close), and
bitwise equal to q6k_lmhead_top1's on the same inputs; top values and
candidate scores within |gpu - oracle| <= 1e-5 * sum|terms| + 1e-6 of the
oracle's logits; a candidate equal to the top id scores bitwise the top
value; candidates outside [0, N) score NaN.  The compact pack equals the
oracle's byte for byte, and the head on it returns the expanded pack's ids,
top values and candidate scores bit for bit.
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


def check_candidate_max(pack_d, N, K, x, row0, rows, cand, logits, bound, oid, compact=False):
    ids, vals, scores = bq.q6k_lmhead_candidate_max(pack_d, N, K, dev(x), row0, rows,
                                                    None if cand is None else dev(cand),
                                                    compact=compact)
    ids, vals, scores = host(ids), host(vals), host(scores)
    check_ids(ids, oid, logits, bound)
    plain = host(bq.q6k_lmhead_top1(pack_d, N, K, dev(x), row0, rows, compact=compact))
    assert (plain == ids).all()
    for r in range(rows):
        g = ids[r]
        assert abs(float(vals[r]) - logits[r, g]) <= REL * bound[r, g] + ABS
        if cand is None:
            continue
        for c, cid in enumerate(cand[r]):
            s = scores[r, c]
            if not 0 <= cid < N:
                assert np.isnan(s), f"row {r} candidate {cid}: {s}"
                continue
            assert abs(float(s) - logits[r, cid]) <= REL * bound[r, cid] + ABS, (r, cid)
            if cid == g:
                assert np.float32(s).view(np.uint32) == np.float32(vals[r]).view(np.uint32)
    return ids, vals, scores


def candidates(rng, oid, N, rows, ncand):
    """Per row: the oracle's top id, id 0, id N - 1, out-of-range ids and
    random ids, cut to ncand."""
    out = np.empty((rows, ncand), np.int32)
    for r in range(rows):
        pool = [int(oid[r]), 0, N - 1, -1, N, *rng.integers(0, N, 4).tolist()]
        out[r] = pool[:ncand]
    return out


@pytest.mark.parametrize("N,K,row0,rows,ncand", [(300, 512, 1, 5, 5), (64, 256, 0, 1, 1),
                                                 (1000, 1280, 0, 8, 8), (1, 256, 2, 3, 3),
                                                 (4097, 768, 0, 6, 8), (700, 512, 1, 5, 0)])
def test_candidate_max_small(N, K, row0, rows, ncand):
    rng = np.random.default_rng(500 + N + rows + ncand)
    raw = synth.q6k_raw_weights(rng, N, K)
    x = synth.normal_rows(rng, row0 + rows + 1, K)
    pack = oracle.q6k_pack_expand(raw, N, K)
    say(f"q6k_lmhead_candidate_max N={N} K={K} row0={row0} rows={rows} ncand={ncand}")
    oid, logits, bound, _ = oracle.q6k_lmhead_top1(pack, N, K, x, row0, rows)
    cand = candidates(rng, oid, N, rows, ncand) if ncand else None
    check_candidate_max(dev(pack), N, K, x, row0, rows, cand, logits, bound, oid)


def test_candidate_max_zero_activations():
    N, K = 700, 512
    rng = np.random.default_rng(520)
    raw = synth.q6k_raw_weights(rng, N, K)
    pack = dev(oracle.q6k_pack_expand(raw, N, K))
    x = np.zeros((6, K), np.float32)
    cand = np.array([[0, 5, 699]] * 6, np.int32)
    ids, vals, scores = [host(t) for t in bq.q6k_lmhead_candidate_max(pack, N, K, dev(x), 0, 6,
                                                                      dev(cand))]
    assert list(ids) == [0] * 6
    assert (vals.view(np.uint32) == 0).all()          # +0, also where a -0 won
    assert (scores == 0).all()


@pytest.fixture(scope="module")
def lm_head_full():
    N, K = synth.LM_HEAD["N"], synth.LM_HEAD["K"]
    say("lm_head: generating raw Q6_K [248320 x 5120]")
    raw, x = synth.lm_head()
    packd = bq.q6k_pack_expand(dev(raw), N, K)
    pack = oracle.q6k_pack_expand(raw, N, K)
    return dict(N=N, K=K, x=x, packd=packd, pack=pack)


def test_candidate_max_lm_head_rows_1_to_5(lm_head_full):
    f = lm_head_full
    N, K = f["N"], f["K"]
    say("lm_head: candidate-max rows 1..5")
    oid, logits, bound, _ = oracle.q6k_lmhead_top1(f["pack"], N, K, f["x"], 1, 5)
    cand = candidates(np.random.default_rng(530), oid, N, 5, 6)
    check_candidate_max(f["packd"], N, K, f["x"], 1, 5, cand, logits, bound, oid)


def test_target_side_all_six_rows(lm_head_full):
    f = lm_head_full
    N, K = f["N"], f["K"]
    say("lm_head: target side, rows 0..5")
    oid, logits, bound, _ = oracle.q6k_lmhead_top1(f["pack"], N, K, f["x"], 0, 6)
    ids = host(bq.q6k_lmhead_top1(f["packd"], N, K, dev(f["x"]), 0, 6))
    check_ids(ids, oid, logits, bound)
    cand = candidates(np.random.default_rng(531), oid, N, 6, 2)
    check_candidate_max(f["packd"], N, K, f["x"], 0, 6, cand, logits, bound, oid)


# ------------------------------------------------------------ compact pack
def same_bits(a, b):
    return np.array_equal(np.asarray(a).view(np.uint32), np.asarray(b).view(np.uint32))


@pytest.mark.parametrize("N,K", [(1, 256), (70, 512), (130, 768), (4097, 1280)])
def test_pack_compact_bitexact(N, K):
    rng = np.random.default_rng(600 + N)
    raw = synth.q6k_raw_weights(rng, N, K)
    say(f"q6k_pack_compact N={N} K={K}")
    cp = host(bq.q6k_pack_compact(dev(raw), N, K))
    assert (cp == oracle.q6k_pack_compact(raw, N, K)).all()


@pytest.mark.parametrize("N,K,row0,rows,ncand", [(300, 512, 1, 5, 5), (64, 256, 0, 1, 1),
                                                 (1000, 1280, 0, 8, 8), (4097, 768, 0, 6, 3)])
def test_compact_head_equals_expanded(N, K, row0, rows, ncand):
    rng = np.random.default_rng(610 + N + rows)
    raw = synth.q6k_raw_weights(rng, N, K)
    x = synth.normal_rows(rng, row0 + rows + 1, K)
    rawd = dev(raw)
    ep = bq.q6k_pack_expand(rawd, N, K)
    cpk = bq.q6k_pack_compact(rawd, N, K)
    say(f"compact head N={N} K={K} rows={rows} ncand={ncand}")
    oid, logits, bound, _ = oracle.q6k_compact_lmhead_top1(oracle.q6k_pack_compact(raw, N, K), N,
                                                           K, x, row0, rows)
    cand = candidates(rng, oid, N, rows, ncand)
    a = check_candidate_max(cpk, N, K, x, row0, rows, cand, logits, bound, oid, compact=True)
    b = check_candidate_max(ep, N, K, x, row0, rows, cand, logits, bound, oid)
    assert (a[0] == b[0]).all()
    assert same_bits(a[1], b[1])
    assert same_bits(np.nan_to_num(a[2], nan=-1.0), np.nan_to_num(b[2], nan=-1.0))


def test_compact_lm_head_full(lm_head_full):
    f = lm_head_full
    N, K = f["N"], f["K"]
    raw = synth.lm_head()[0]
    say("lm_head: q6k_pack_compact")
    cpk = bq.q6k_pack_compact(dev(raw), N, K)
    assert cpk.numel() == 1_042_944_000
    assert (host(cpk) == oracle.q6k_pack_compact(raw, N, K)).all()
    xd = dev(f["x"])
    for row0, rows in [(1, 5), (0, 6)]:
        say(f"lm_head compact vs expanded rows {row0}..{row0 + rows - 1}")
        cand = torch.tensor([[12305, 198, r] for r in range(rows)], dtype=torch.int32,
                            device=DEV)
        a = [host(t) for t in bq.q6k_lmhead_candidate_max(cpk, N, K, xd, row0, rows, cand,
                                                           compact=True)]
        b = [host(t) for t in bq.q6k_lmhead_candidate_max(f["packd"], N, K, xd, row0, rows,
                                                           cand)]
        assert (a[0] == b[0]).all()
        assert same_bits(a[1], b[1]) and same_bits(a[2], b[2])
    oid, logits, bound, _ = oracle.q6k_lmhead_top1(f["pack"], N, K, f["x"], 1, 5)
    check_ids(host(bq.q6k_lmhead_top1(cpk, N, K, xd, 1, 5, compact=True)), oid, logits, bound)
