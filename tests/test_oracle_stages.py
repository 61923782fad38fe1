"""Pins for the oracle's verifier-layer stages between projections.

Reading (the pages are silent on the block's glue): h = SiLU(gate) * up, and
the next layer's input is the weightless row RMS normalization of the down
projection's output ("Qwen3.6 27B Q4_0 DFlash/SYCL closure": width-6 gate/up
and down projections; the down-to-next-RMS/Q8 boundary).
"""
import math

import numpy as np


def test_silu_closed_forms(orc):
    g = np.array([0.0, 1.0, -1.0, 30.0, -30.0, 100.0, -100.0, 2.5], np.float32)
    u = np.array([5.0, 1.0, 1.0, 2.0, 2.0, -1.0, 1.0, 0.0], np.float32)
    h = orc.silu_mul(g, u)
    assert h[0] == 0.0 and h[7] == 0.0
    assert math.isclose(h[1], 1.0 / (1.0 + math.exp(-1.0)), rel_tol=1e-15)
    # SiLU(g) - SiLU(-g) = g
    assert math.isclose(h[1] - h[2], 1.0, rel_tol=1e-15)
    assert math.isclose(h[3], 60.0, rel_tol=1e-12)
    assert abs(h[4]) < 1e-11 and h[4] <= 0.0
    assert h[5] == -100.0
    assert abs(h[6]) < 1e-40


def test_silu_symmetry_random(orc):
    rng = np.random.default_rng(41)
    g = rng.standard_normal(10000).astype(np.float32) * 4
    one = np.ones_like(g)
    a = orc.silu_mul(g, one)
    b = orc.silu_mul(-g, one)
    assert np.allclose(a - b, g.astype(np.float64), rtol=1e-14, atol=1e-14)
    # linear in the up operand
    u = rng.standard_normal(10000).astype(np.float32)
    assert np.allclose(orc.silu_mul(g, u), a * u.astype(np.float64), rtol=1e-15, atol=0)


def test_rms_norm_closed_forms(orc):
    eps = 1e-6
    y = np.full((2, 64), 3.0, np.float32)
    y[1] = -0.5
    out = orc.rms_norm(y, eps)
    assert np.allclose(out[0], 3.0 / math.sqrt(9.0 + eps), rtol=1e-15)
    assert np.allclose(out[1], -0.5 / math.sqrt(0.25 + eps), rtol=1e-15)
    z = orc.rms_norm(np.zeros((1, 32), np.float32), eps)
    assert not z.any()


def test_rms_norm_unit_mean_square(orc):
    rng = np.random.default_rng(42)
    y = (rng.standard_normal((6, 5120)) * 37.0).astype(np.float32)
    eps = 1e-6
    out = orc.rms_norm(y, eps)
    ms_in = (y.astype(np.float64) ** 2).mean(axis=1)
    ms_out = (out ** 2).mean(axis=1)
    assert np.allclose(ms_out, ms_in / (ms_in + eps), rtol=1e-12)
    # the direction of each row is unchanged
    assert (np.sign(out) == np.sign(y)).all()
