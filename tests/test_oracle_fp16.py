"""Pins for the oracle's IEEE binary16 codec against numpy's independent one."""
import numpy as np


def _same_bits_or_both_nan(a32, b32):
    a = np.asarray(a32, np.float32)
    b = np.asarray(b32, np.float32)
    both_nan = np.isnan(a) & np.isnan(b)
    return both_nan | (a.view(np.uint32) == b.view(np.uint32))


def test_decode_exhaustive(orc):
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ours = orc.f16_bits_to_f32(bits)
    ref = bits.view(np.float16).astype(np.float32)
    assert _same_bits_or_both_nan(ours, ref).all()


def test_roundtrip_every_finite_pattern(orc):
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    vals = bits.view(np.float16).astype(np.float32)
    finite = np.isfinite(vals)
    back = orc.f32_to_f16_bits(vals[finite])
    assert (back == bits[finite]).all()
    # infinities keep their sign, NaN stays NaN
    inf_bits = orc.f32_to_f16_bits(np.array([np.inf, -np.inf], np.float32))
    assert list(inf_bits) == [0x7C00, 0xFC00]
    nan = orc.f32_to_f16_bits(np.array([np.nan], np.float32)).view(np.float16)
    assert np.isnan(nan).all()


def _midpoints():
    """Exact f32 midpoints between consecutive finite binary16 values (the
    round-to-nearest-even ties) plus their f32 neighbours."""
    bits = np.arange(0, 0x7BFF, dtype=np.uint16)
    lo = bits.view(np.float16).astype(np.float64)
    hi = (bits + 1).view(np.float16).astype(np.float64)
    mid = ((lo + hi) / 2).astype(np.float32)  # exact: needs at most 12 bits
    assert ((mid.astype(np.float64)) == (lo + hi) / 2).all()
    up = np.nextafter(mid, np.float32(np.inf))
    dn = np.nextafter(mid, np.float32(0))
    return np.concatenate([mid, up, dn, -mid, -up, -dn])


def test_encode_ties_and_neighbours_match_numpy(orc):
    x = _midpoints()
    ours = orc.f32_to_f16_bits(x)
    ref = x.astype(np.float16).view(np.uint16)
    assert (ours == ref).all()


def test_encode_overflow_and_subnormal_edges(orc):
    edges = np.array([65504.0, 65519.0, 65519.996, 65520.0, 65536.0, 1e9, 3.4e38,
                      2.0 ** -24, 2.0 ** -25, np.nextafter(np.float32(2.0 ** -25), np.float32(1)),
                      2.0 ** -26, 2.0 ** -14, np.nextafter(np.float32(2.0 ** -14), np.float32(0)),
                      1e-45, 0.0, -0.0], np.float32)
    x = np.concatenate([edges, -edges])
    ours = orc.f32_to_f16_bits(x)
    ref = x.astype(np.float16).view(np.uint16)
    assert (ours == ref).all()


def test_encode_random_matches_numpy(orc):
    rng = np.random.default_rng(1234)
    n = 2_000_000
    # log-uniform magnitudes across the whole binary16 range and beyond
    mag = np.exp2(rng.uniform(-30, 18, n)).astype(np.float32)
    sign = np.where(rng.random(n) < 0.5, -1, 1).astype(np.float32)
    x = mag * sign
    raw = rng.integers(0, 2 ** 32, 500_000, dtype=np.uint64).astype(np.uint32).view(np.float32)
    x = np.concatenate([x, raw[np.isfinite(raw)]])
    ours = orc.f32_to_f16_bits(x)
    ref = x.astype(np.float16).view(np.uint16)
    assert (ours == ref).all()
