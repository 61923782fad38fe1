"""Pins for the oracle's Q4_0 codec and its Q4_0 x Q8_1 GEMV.

The GEMV is the plain definition y[m][n] = sum_k W[n][k] X[m][k] over the
dequantized stored values (Q4_0 MMVQ of "Qwen3.6 27B Q4_0 DFlash/SYCL
closure", "What materially worked").  Pins: the constant-quant closed form
d_w*d_x*(q_w-8)*q_x*K, exact rational brute force, an independent numpy
dequantize-then-matmul, and the tolerance bound's definition.
"""
from fractions import Fraction

import numpy as np
import pytest

from block_quantized_gemv_q8_amd import synth


def _q8_1_bytes(d_bits, s_bits, q):
    """Lay out Q8_1 blocks by hand (d, s, q[32]) for controlled activations."""
    d_bits = np.asarray(d_bits, np.uint16).reshape(-1)
    s_bits = np.asarray(s_bits, np.uint16).reshape(-1)
    q = np.asarray(q, np.int8).reshape(-1, 32)
    out = np.empty((q.shape[0], 36), np.uint8)
    out[:, 0:2] = d_bits.astype("<u2").view(np.uint8).reshape(-1, 2)
    out[:, 2:4] = s_bits.astype("<u2").view(np.uint8).reshape(-1, 2)
    out[:, 4:] = q.view(np.uint8)
    return out.reshape(-1)


def test_codec_roundtrip(orc):
    rng = np.random.default_rng(3)
    N, K = 7, 320
    w = synth.q4_0_weights(rng, N, K)
    d, q = orc.q4_0_decode(w, N, K)
    assert q.max() <= 15
    assert (orc.q4_0_encode(d, q, N, K) == w).all()
    d2 = rng.integers(0, 65536, N * K // 32, dtype=np.uint16)
    q2 = rng.integers(0, 16, (N, K), dtype=np.uint8)
    w2 = orc.q4_0_encode(d2, q2, N, K)
    a, b = orc.q4_0_decode(w2, N, K)
    assert (a == d2).all() and (b == q2).all()


def test_nibble_order_worked_example(orc):
    # one block: d = 1.0, qs[0] = 0x21, qs[15] = 0xF0, others 0x88
    blk = np.full(18, 0x88, np.uint8)
    blk[0:2] = np.array([np.float16(1.0).view(np.uint16)], "<u2").view(np.uint8)
    blk[2] = 0x21
    blk[17] = 0xF0
    d, q = orc.q4_0_decode(blk, 1, 32)
    assert q[0, 0] == 1 and q[0, 16] == 2      # low nibble first half, high second
    assert q[0, 15] == 0 and q[0, 31] == 15
    assert (q[0, 1:15] == 8).all() and (q[0, 17:31] == 8).all()


@pytest.mark.parametrize("qw,qx", [(0, 127), (15, -127), (3, 5), (8, 100), (12, -1)])
def test_constant_closed_form(orc, qw, qx):
    N, K, M = 5, 512, 3
    dw = np.float16(0.0137)
    dx = np.float16(0.0219)
    d_bits = np.full(N * K // 32, dw.view(np.uint16), np.uint16)
    w = orc.q4_0_encode(d_bits, np.full((N, K), qw, np.uint8), N, K)
    nblk = M * K // 32
    xq = _q8_1_bytes(np.full(nblk, dx.view(np.uint16)), np.zeros(nblk), np.full((nblk, 32), qx))
    y, bound = orc.q4_0_gemv(w, N, K, xq, M)
    expect = float(dw) * float(dx) * (qw - 8) * qx * K
    assert (y == expect).all()
    assert (bound == abs(expect)).all()


def _exact_gemv(w, N, K, xq, M):
    """Exact rational y and block-term bound, decoding with numpy bit ops."""
    nb = K // 32
    wb = w.reshape(N, nb, 18)
    dw = wb[:, :, 0:2].copy().view("<u2")[..., 0].view(np.float16).astype(np.float64)
    lo = (wb[:, :, 2:] & 0x0F).astype(np.int64)
    hi = (wb[:, :, 2:] >> 4).astype(np.int64)
    qw = np.concatenate([lo, hi], axis=2) - 8                     # [N][nb][32]
    xb = xq.reshape(M, nb, 36)
    dx = xb[:, :, 0:2].copy().view("<u2")[..., 0].view(np.float16).astype(np.float64)
    qx = xb[:, :, 4:].view(np.int8).astype(np.int64)             # [M][nb][32]
    y = [[Fraction(0)] * N for _ in range(M)]
    bound = [[Fraction(0)] * N for _ in range(M)]
    for m in range(M):
        for n in range(N):
            for b in range(nb):
                t = Fraction(float(dw[n, b])) * Fraction(float(dx[m, b])) * int(
                    (qw[n, b] * qx[m, b]).sum())
                y[m][n] += t
                bound[m][n] += abs(t)
    return y, bound


def test_exact_rational_bruteforce(orc):
    rng = np.random.default_rng(11)
    N, K, M = 4, 160, 3           # non-square, M > 1: a transposed index fails
    w = synth.q4_0_weights(rng, N, K)
    x = synth.normal_rows(rng, M, K)
    xq = orc.q8_1_quantize(x)
    y, bound = orc.q4_0_gemv(w, N, K, xq, M)
    ey, eb = _exact_gemv(w, N, K, xq, M)
    for m in range(M):
        for n in range(N):
            # binary64 summation of K/32 exact block terms
            err = abs(Fraction(float(y[m, n])) - ey[m][n])
            assert err <= eb[m][n] * Fraction(K // 32, 2 ** 52)
            assert bound[m, n] == float(eb[m][n])


def test_numpy_dequantize_matmul_tiny(orc):
    w, x = synth.tiny()
    N, K, M = 256, 256, 1
    xq = orc.q8_1_quantize(x)
    y, bound = orc.q4_0_gemv(w, N, K, xq, M)
    nb = K // 32
    wb = w.reshape(N, nb, 18)
    dw = wb[:, :, 0:2].copy().view("<u2")[..., 0].view(np.float16).astype(np.float64)
    nib = np.concatenate([wb[:, :, 2:] & 15, wb[:, :, 2:] >> 4], axis=2).astype(np.float64)
    W = ((nib - 8) * dw[:, :, None]).reshape(N, K)
    xb = xq.reshape(M, nb, 36)
    dx = xb[:, :, 0:2].copy().view("<u2")[..., 0].view(np.float16).astype(np.float64)
    X = (xb[:, :, 4:].view(np.int8).astype(np.float64) * dx[:, :, None]).reshape(M, K)
    ref = X @ W.T
    assert (np.abs(y - ref) <= 1e-12 * bound).all()
    # and the quantized result is close to the unquantized f32 product
    approx = x.astype(np.float64) @ W.T
    assert np.abs(y - approx).max() < 0.05 * np.abs(approx).max()


def test_rows_are_independent(orc):
    # permuting weight rows permutes outputs; duplicated rows give equal values
    rng = np.random.default_rng(5)
    N, K, M = 9, 96, 2
    w = synth.q4_0_weights(rng, N, K)
    xq = orc.q8_1_quantize(synth.normal_rows(rng, M, K))
    y, _ = orc.q4_0_gemv(w, N, K, xq, M)
    perm = rng.permutation(N)
    yp, _ = orc.q4_0_gemv(w[perm], N, K, xq, M)
    assert (yp == y[:, perm]).all()
    w2 = w.copy()
    w2[4] = w2[1]
    y2, _ = orc.q4_0_gemv(w2, N, K, xq, M)
    assert (y2[:, 4] == y2[:, 1]).all()
