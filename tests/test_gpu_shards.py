"""GPU parity at one GPU's share of the path under 8-way sharding, at the
shapes bench.py times:

  * the gate/up column shard (N = 17408/8 = 2176, K = 5120, M = 6) through
    the packed product and the joint gate/up launch;
  * the down row shard (N = 5120, K = 17408/8 = 2176) on the GGUF block
    layout -- the packed layout takes K in multiples of 512 only, and rejects
    this K with a shape error;
  * the LM head's vocabulary shard (248320/8 = 31040 rows, rows 1..5 of six)
    through the expanded and the compact pack.

Bars as everywhere: products within |gpu - oracle| <= 1e-5 * sum_b |t_b| +
1e-6; a greedy id equal to the oracle's, or within that tolerance of the
oracle's logit where two rows nearly tie; the joint launch's Q8_1 output
bitwise equal to the standalone SiLU*up requant of its own g and u.

Also the head at two wider vocabularies that split each tile's K into four
ranges (one at more tiles than workgroups), and the read-only HBM probe that
bench.py reports as the streaming ceiling:
it reads every 32-bit word of its buffer exactly once, so the XOR of its
outputs is the XOR of the buffer's words, for every launch shape.
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
SHARDS = 8


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


def assert_close(gpu, ref, bound, what):
    err = np.abs(gpu.astype(np.float64) - ref)
    bad = err > REL * bound + ABS
    assert not bad.any(), (f"{what}: {bad.sum()} of {bad.size} outside tolerance; first at "
                           f"{tuple(np.argwhere(bad)[0])}")


def test_gate_up_column_shard():
    N, K, M = synth.FFN_UP["N"] // SHARDS, synth.FFN_UP["K"], 6
    say(f"gate/up column shard N={N} K={K} M={M}")
    wg, x = synth.random_q4_0_case(8100, N, K, M)
    wu, _ = synth.random_q4_0_case(8101, N, K, 1)
    xq = oracle.q8_1_quantize(x)
    pg, pu, xqd = bq.q4_0_pack(dev(wg)), bq.q4_0_pack(dev(wu)), dev(xq)
    ref_g, bound_g = oracle.q4_0_gemv(wg, N, K, xq, M)
    ref_u, bound_u = oracle.q4_0_gemv(wu, N, K, xq, M)
    assert_close(host(bq.q4_0_mmvq_packed(pg, N, K, xqd, M)), ref_g, bound_g, "packed shard")
    g = torch.empty((M, N), dtype=torch.float32, device=DEV)
    u = torch.empty_like(g)
    hq = host(bq.q4_0_gate_up_silu_q8_1_packed(pg, pu, N, K, xqd, M, g=g, u=u))
    assert_close(host(g), ref_g, bound_g, "joint gate shard")
    assert_close(host(u), ref_u, bound_u, "joint up shard")
    assert (host(bq.silu_mul_q8_1(g, u)) == hq).all()


def test_down_row_shard():
    N, K, M = synth.DOWN_SWEEP["N"], synth.DOWN_SWEEP["K"] // SHARDS, 6
    say(f"down row shard N={N} K={K} M={M} (GGUF layout)")
    w, x = synth.random_q4_0_case(8200, N, K, M, x_std=0.5)
    xq = oracle.q8_1_quantize(x)
    wd = dev(w)
    ref, bound = oracle.q4_0_gemv(w, N, K, xq, M)
    assert_close(host(bq.q4_0_mmvq_m6(wd, dev(xq))), ref, bound, "down shard")
    with pytest.raises(bq.Bq8Error):
        bq.q4_0_pack(wd)              # K = 2176 is not a multiple of 512


def test_lm_head_vocab_shard():
    N, K = synth.LM_HEAD["N"] // SHARDS, synth.LM_HEAD["K"]
    say(f"lm head vocabulary shard N={N} K={K} rows 1..5")
    rng = np.random.default_rng(8300)
    raw = synth.q6k_raw_weights(rng, N, K)
    x = synth.normal_rows(rng, 6, K)
    oid, logits, bound, _ = oracle.q6k_lmhead_top1(oracle.q6k_pack_expand(raw, N, K), N, K, x, 1, 5)
    rawd, xd = dev(raw), dev(x)
    ids_e = host(bq.q6k_lmhead_top1(bq.q6k_pack_expand(rawd, N, K), N, K, xd, 1, 5))
    ids_c = host(bq.q6k_lmhead_top1(bq.q6k_pack_compact(rawd, N, K), N, K, xd, 1, 5,
                                    compact=True))
    say(f"shard ids gpu {list(ids_e)} oracle {list(oid)}")
    assert (ids_c == ids_e).all()
    check_ids(ids_e, oid, logits, bound, f"vocabulary rows {N}")


@pytest.mark.parametrize("nbytes", [16, 1024 * 1024 + 48, synth.FFN_UP["N"] * 160 * 18])
def test_hbm_read_probe_reads_every_word_once(nbytes):
    rng = np.random.default_rng(8400 + nbytes % 997)
    buf = rng.integers(0, 256, nbytes, dtype=np.uint8)
    want = np.bitwise_xor.reduce(buf.view(np.uint32))
    bd = dev(buf)
    for wgs, unroll in ((1, 1), (7, 2), (1024, 4), (4096, 8)):
        say(f"hbm_read_probe bytes={nbytes} workgroups={wgs} unroll={unroll}")
        out = host(bq.hbm_read_probe(bd, wgs, unroll))
        assert out.shape == (4 * wgs,)
        assert np.bitwise_xor.reduce(out.view(np.uint32)) == want


# Widths that split each tile's K into four ranges: 70001 rows (1094 tiles,
# one per workgroup, a ragged last tile) and 200000 rows (3125 tiles, more
# than the 1024 workgroups, so each workgroup walks several tiles).
@pytest.mark.parametrize("N", [70001, 200000])
def test_lm_head_split_widths(N):
    K = synth.LM_HEAD["K"]
    say(f"lm head N={N} K={K} rows 1..5 (four superblock ranges per tile)")
    rng = np.random.default_rng(8500 + N % 1000)
    raw = synth.q6k_raw_weights(rng, N, K)
    x = synth.normal_rows(rng, 6, K)
    raw[N - 1] = raw[3]               # equal rows: the lower id must win a tie
    oid, logits, bound, _ = oracle.q6k_lmhead_top1(oracle.q6k_pack_expand(raw, N, K), N, K, x, 1, 5)
    rawd, xd = dev(raw), dev(x)
    ids_e = host(bq.q6k_lmhead_top1(bq.q6k_pack_expand(rawd, N, K), N, K, xd, 1, 5))
    ids_c = host(bq.q6k_lmhead_top1(bq.q6k_pack_compact(rawd, N, K), N, K, xd, 1, 5,
                                    compact=True))
    say(f"ids gpu {list(ids_e)} oracle {list(oid)}")
    assert (ids_c == ids_e).all()
    assert (ids_e != N - 1).all()
    check_ids(ids_e, oid, logits, bound, f"vocabulary rows {N}")
