"""Pins for the oracle's Q8_1 activation quantizer.

The pages call the activation format "exact Q8_1" ("Qwen3.6 27B B70
follow-up", section "Q8_1 activation cache prototype") without spelling out
its arithmetic; the reading pinned here: per 32 values d = max|x|/127 in
binary32, q = x/d rounded to nearest with halves away from zero, stored
d = fp16(d), s = fp16(d * sum q).  The pins are closed forms, exact half-way
constructions, and invariants any correct quantizer of that reading meets.
"""
import numpy as np
import pytest


def _f16(bits):
    return np.asarray(bits, np.uint16).view(np.float16).astype(np.float64)


def test_zero_block(orc):
    xq = orc.q8_1_quantize(np.zeros((2, 64), np.float32))
    assert not xq.any()


@pytest.mark.parametrize("c", [1.0, -3.5, 1e-3, 250.0, 6.1e-5])
def test_constant_block(orc, c):
    x = np.full((1, 32), c, np.float32)
    d, s, q = orc.q8_1_fields(orc.q8_1_quantize(x))
    sign = 1 if c > 0 else -1
    assert (q == sign * 127).all()
    d32 = np.float32(abs(c)) / np.float32(127)
    assert d[0] == np.float16(d32).view(np.uint16)
    # s = d * sum(q) with sum(q) = +-32*127 = +-4064
    assert s[0] == np.float16(np.float32(d32) * np.float32(sign * 4064)).view(np.uint16)


@pytest.mark.parametrize("sign", [1, -1])
def test_half_way_rounds_away_from_zero(orc, sign):
    # d = 2^-7 exactly when amax = 127/128; then x = (k + 1/2) / 128 gives
    # x/d = k + 1/2 exactly in binary32: a tie for every k.
    k = np.arange(31, dtype=np.float64)
    x = np.empty(32, np.float64)
    x[0] = 127.0 / 128.0
    x[1:] = (k + 0.5) / 128.0
    x = (sign * x).astype(np.float32)[None, :]
    d, s, q = orc.q8_1_fields(orc.q8_1_quantize(x))
    assert _f16(d)[0] == 2.0 ** -7
    expect = np.concatenate([[127], k + 1]).astype(np.int64) * sign
    assert (q[0].astype(np.int64) == expect).all()
    # a half-to-even quantizer would give k for even k: make sure it differs
    assert (np.round(k + 0.5) != k + 1).any()


def _blocks(seed, M=8, K=4096):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((M, K), dtype=np.float32)
    x[:, rng.choice(K, K // 100, replace=False)] *= 20
    x[0, :32] = 0.0                          # zero block
    x[1, :32] = 7.25                         # constant block
    x[2, :32] *= 1e-30                       # tiny but normal amax
    return x


def test_nearest_and_range_invariants(orc):
    x = _blocks(7)
    M, K = x.shape
    d, s, q = orc.q8_1_fields(orc.q8_1_quantize(x))
    xb = x.reshape(-1, 32).astype(np.float64)
    amax = np.abs(xb).max(axis=1)
    d32 = (amax.astype(np.float32) / np.float32(127)).astype(np.float64)
    nz = amax > 0
    qf = q.astype(np.float64)
    # every nonzero block uses the full code range at its largest element
    assert (np.abs(q[nz]).max(axis=1) == 127).all()
    assert (np.abs(q) <= 127).all()
    # nearest rounding: |x/d - q| <= 1/2 (binary32 quotient may sit on a tie)
    t = xb[nz] / d32[nz, None]
    assert (np.abs(t - qf[nz]) <= 0.5 + 1e-5).all()
    # the stored d is the fp16 rounding of amax/127
    assert (d == d32.astype(np.float32).astype(np.float16).view(np.uint16)).all()
    # s is d * sum(q), rounded once to fp16: within half an fp16 ulp-ish
    ssum = qf.sum(axis=1)
    target = d32 * ssum
    sv = _f16(s)
    assert (np.abs(sv - target) <= np.abs(target) * 2.0 ** -11 + 2.0 ** -25).all()
    # zero block is all zero
    assert d[0] == 0 and s[0] == 0 and not q[0].any()


def test_sign_symmetry(orc):
    x = _blocks(8)
    a = orc.q8_1_fields(orc.q8_1_quantize(x))
    b = orc.q8_1_fields(orc.q8_1_quantize(-x))
    assert (a[0] == b[0]).all()
    assert (a[2] == -b[2]).all()
    sa, sb = _f16(a[1]), _f16(b[1])
    assert (sa == -sb).all()


def test_scale_invariance_power_of_two(orc):
    # multiplying by 2^e leaves quants unchanged and scales d and s by 2^e
    # (while everything stays in the binary16 normal range)
    x = _blocks(9)[3:]
    a = orc.q8_1_fields(orc.q8_1_quantize(x))
    b = orc.q8_1_fields(orc.q8_1_quantize(x * np.float32(4.0)))
    assert (a[2] == b[2]).all()
    da, db = _f16(a[0]), _f16(b[0])
    ok = (da > 2.0 ** -14) & (db < 60000)
    assert (db[ok] == 4 * da[ok]).all()


def test_subnormal_amax_stays_in_range(orc):
    # amax so small that amax/127 is subnormal or zero in binary32
    x = np.zeros((3, 32), np.float32)
    x[0, 0] = np.float32(1e-45)         # d underflows to 0 -> zero block
    x[1, :] = np.float32(3e-43)
    x[1, 5] = np.float32(-1.7e-43)
    x[2, :4] = np.array([1e-40, -2e-41, 5e-42, 0], np.float32)
    d, s, q = orc.q8_1_fields(orc.q8_1_quantize(x))
    assert (np.abs(q) <= 127).all()
    assert not q[0].any() and d[0] == 0 and s[0] == 0
    assert q[2, 0] == 127


def test_layout_row_major_blocks(orc):
    # block (m, b) occupies bytes [(m*nb + b)*36, +36) with d, s, q[32]
    x = np.zeros((2, 64), np.float32)
    x[1, 33] = 127.0  # row 1, block 1, element 1
    xq = orc.q8_1_quantize(x).reshape(-1)
    blk = xq[3 * 36:4 * 36]
    assert blk[0:2].view(np.uint16)[0] == np.float16(1.0).view(np.uint16)
    assert blk[2:4].view(np.uint16)[0] == np.float16(127.0).view(np.uint16)
    assert blk[4 + 1] == 127 and blk[4:].sum() == 127
    assert not xq[:3 * 36].any()
