"""Pins for the oracle's Q6_K codec, expanded pack and LM-head logits.

"Q6_K M=6 fused DFlash top-1 production record": the output tensor is
expanded once into signed int8 quants, int8 subscales and fp16 superblock
scales ("Why this was slow"); the pack for [5120, 248320] is 1,360,793,600
bytes ("Memory and startup").
"""
import os
from fractions import Fraction

import numpy as np
import pytest

from block_quantized_gemv_q8_amd import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden_rows(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if line:
                rows.append([int(v) for v in line.split()])
    return rows


def test_pack_bytes_match_pages(orc):
    (N, K, nbytes), = _golden_rows("q6k_pack_bytes.txt")
    assert orc.q6k_pack_bytes(N, K) == nbytes
    # one byte per quant, one per 16-value subscale, two per 256-value scale
    assert nbytes == N * K + N * K // 16 + 2 * N * K // 256


def test_raw_roundtrip(orc):
    rng = np.random.default_rng(21)
    N, K = 5, 512
    raw = synth.q6k_raw_weights(rng, N, K)
    q, sc, d = orc.q6k_decode(raw, N, K)
    assert q.min() >= -32 and q.max() <= 31
    assert (orc.q6k_encode(q, sc, d, N, K) == raw).all()
    q2 = rng.integers(-32, 32, (N, K), dtype=np.int8)
    sc2 = rng.integers(-128, 128, (N, K // 16), dtype=np.int8)
    d2 = rng.integers(0, 65536, (N, K // 256), dtype=np.uint16)
    a, b, c = orc.q6k_decode(orc.q6k_encode(q2, sc2, d2, N, K), N, K)
    assert (a == q2).all() and (b == sc2).all() and (c == d2).all()


def test_uniform_random_bytes_give_uniform_codes(orc):
    # the generator draws ql/qh as random bytes; every 6-bit code must be
    # reachable and roughly equally likely
    rng = np.random.default_rng(22)
    raw = synth.q6k_raw_weights(rng, 64, 1024)
    q, _, _ = orc.q6k_decode(raw, 64, 1024)
    counts = np.bincount((q.astype(np.int64) + 32).reshape(-1), minlength=64)
    assert counts.min() > 0.8 * counts.mean() and counts.max() < 1.2 * counts.mean()


def test_decode_worked_example(orc):
    # hand-built superblock: ql[0] = 0x5A, ql[32] = 0xC3, qh[0] = 0b11100100,
    # second half ql[64] = 0x0F, qh[32] = 0b00000011; all else zero.
    blk = np.zeros(210, np.uint8)
    blk[0], blk[32], blk[128] = 0x5A, 0xC3, 0b11100100
    blk[64], blk[160] = 0x0F, 0b00000011
    blk[192:208] = np.arange(16, dtype=np.int8).view(np.uint8)
    blk[208:210] = np.array([np.float16(0.5).view(np.uint16)], "<u2").view(np.uint8)
    q, sc, d = orc.q6k_decode(blk, 1, 256)
    code = q[0].astype(np.int64) + 32
    assert code[0] == 0xA | (0b00 << 4)       # low nibble of ql[0], qh bits 0-1
    assert code[32] == 0x3 | (0b01 << 4)      # low nibble of ql[32], qh bits 2-3
    assert code[64] == 0x5 | (0b10 << 4)      # high nibble of ql[0], qh bits 4-5
    assert code[96] == 0xC | (0b11 << 4)      # high nibble of ql[32], qh bits 6-7
    assert code[128] == 0xF | (0b11 << 4)     # second half: ql[64], qh[32]
    others = np.delete(code, [0, 32, 64, 96, 128])
    assert (others == 0).all()
    assert (sc[0] == np.arange(16)).all() and d[0, 0] == np.float16(0.5).view(np.uint16)


def test_pack_planes(orc):
    """The pack's layout, checked value by value from the decoded raw blocks:
    tiles of 64 rows (the last one ragged), each tile storing 16-value pieces
    of all its rows piece after piece (Q), the 16 subscales of each
    superblock row after row (SC), and the superblock scales (D)."""
    rng = np.random.default_rng(23)
    N, K = 70, 768            # one full tile and a ragged tile of 6 rows; 3 superblocks
    raw = synth.q6k_raw_weights(rng, N, K)
    pack = orc.q6k_pack_expand(raw, N, K)
    q, sc, d = orc.q6k_decode(raw, N, K)
    assert pack.size == orc.q6k_pack_bytes(N, K)
    Qp = pack[:N * K].view(np.int8)
    SCp = pack[N * K:N * K + N * K // 16].view(np.int8)
    Dp = pack[N * K + N * K // 16:].view("<u2")
    for t0, rows_t in [(0, 64), (64, 6)]:
        tq = Qp[t0 * K:(t0 + rows_t) * K].reshape(K // 16, rows_t, 16)
        assert (tq.transpose(1, 0, 2).reshape(rows_t, K) == q[t0:t0 + rows_t]).all()
        ts = SCp[t0 * K // 16:(t0 + rows_t) * K // 16].reshape(K // 256, rows_t, 16)
        assert (ts.transpose(1, 0, 2).reshape(rows_t, K // 16) == sc[t0:t0 + rows_t]).all()
        td = Dp[t0 * K // 256:(t0 + rows_t) * K // 256].reshape(K // 256, rows_t)
        assert (td.T == d[t0:t0 + rows_t]).all()
    # a tile's piece c of its 64 rows is one contiguous kilobyte
    c, r = 5, 17
    assert (Qp[(c * 64 + r) * 16:(c * 64 + r) * 16 + 16] == q[r, 16 * c:16 * c + 16]).all()


def _xq(orc, rows, K, seed):
    rng = np.random.default_rng(seed)
    return orc.q8_1_quantize(synth.normal_rows(rng, rows, K))


@pytest.mark.parametrize("qv,scv,qx", [(31, 63, 127), (-32, -64, 5), (7, 1, -127)])
def test_constant_closed_form(orc, qv, scv, qx):
    N, K, rows = 3, 512, 2
    dw = np.float16(3.1e-4)
    dx = np.float16(0.0173)
    raw = orc.q6k_encode(np.full((N, K), qv, np.int8), np.full((N, K // 16), scv, np.int8),
                         np.full((N, K // 256), dw.view(np.uint16), np.uint16), N, K)
    pack = orc.q6k_pack_expand(raw, N, K)
    nblk = rows * K // 32
    xq = np.empty((nblk, 36), np.uint8)
    xq[:, 0:2] = np.array([dx.view(np.uint16)], "<u2").view(np.uint8)
    xq[:, 2:4] = 0
    xq[:, 4:] = np.int8(qx).view(np.uint8)
    logits, bound = orc.q6k_pack_logits(pack, N, K, xq.reshape(-1), rows)
    expect = float(dw) * scv * qv * float(dx) * qx * K
    assert (logits == expect).all() and (bound == abs(expect)).all()


def test_exact_rational_bruteforce(orc):
    rng = np.random.default_rng(24)
    N, K, rows = 3, 512, 2       # two superblocks, 16 subscales each (one ragged tile)
    raw = synth.q6k_raw_weights(rng, N, K)
    pack = orc.q6k_pack_expand(raw, N, K)
    xq = _xq(orc, rows, K, 25)
    logits, bound = orc.q6k_pack_logits(pack, N, K, xq, rows)
    q, sc, d = orc.q6k_decode(raw, N, K)
    dv = d.view(np.float16).astype(np.float64)
    xb = xq.reshape(rows, K // 32, 36)
    dx = xb[:, :, 0:2].copy().view("<u2")[..., 0].view(np.float16).astype(np.float64)
    qx = xb[:, :, 4:].view(np.int8).astype(np.int64).reshape(rows, K)
    for r in range(rows):
        for n in range(N):
            exact, mag = Fraction(0), Fraction(0)
            for b in range(K // 32):
                t = Fraction(0)
                for j in range(32):
                    k = 32 * b + j
                    t += (Fraction(float(dv[n, k // 256])) * int(sc[n, k // 16]) * int(q[n, k])
                          * Fraction(float(dx[r, b])) * int(qx[r, k]))
                exact += t
                mag += abs(t)
            assert abs(Fraction(float(logits[r, n])) - exact) <= mag * Fraction(K // 32, 2 ** 52)
            assert bound[r, n] == float(mag)


def test_numpy_dequantize_matmul(orc):
    rng = np.random.default_rng(26)
    N, K, rows = 300, 1024, 5    # four full 64-row tiles and a ragged one of 44 rows
    raw = synth.q6k_raw_weights(rng, N, K)
    pack = orc.q6k_pack_expand(raw, N, K)
    xq = _xq(orc, rows, K, 27)
    logits, bound = orc.q6k_pack_logits(pack, N, K, xq, rows)
    q, sc, d = orc.q6k_decode(raw, N, K)
    W = (q.astype(np.float64) * np.repeat(sc.astype(np.float64), 16, axis=1)
         * np.repeat(d.view(np.float16).astype(np.float64), 256, axis=1))
    xb = xq.reshape(rows, K // 32, 36)
    dx = xb[:, :, 0:2].copy().view("<u2")[..., 0].view(np.float16).astype(np.float64)
    X = (xb[:, :, 4:].view(np.int8).astype(np.float64) * dx[:, :, None]).reshape(rows, K)
    ref = X @ W.T
    assert (np.abs(logits - ref) <= 1e-12 * bound).all()
