"""Pins for the oracle's offline-packed Q4_0 layout.

"Qwen3.6 27B Q4_0 DFlash/SYCL closure", "What materially worked": the
verifier's width-6 gate/up and down projections ran on offline-packed
weights.  The pages do not give the format; the oracle's reading keeps the
18 bytes per 32 weights and regroups them (bq8_oracle.c documents it).  The
pins: the packing is a bijection on the bytes, its layout is the one stated
(checked element by element), and the product read from the packed layout
equals, bit for bit, the already pinned product of the standard layout.
"""
import numpy as np
import pytest

from block_quantized_gemv_q8_amd import synth


def _elements(w, N, K):
    """Element codes [N][K] and scale bits [N][K/32] of standard Q4_0 bytes,
    straight from the block format: element j < 16 is the low nibble of
    qs[j], element j >= 16 the high nibble of qs[j-16]."""
    nb = K // 32
    blk = np.asarray(w, np.uint8).reshape(N, nb, 18)
    qs = blk[:, :, 2:]
    e = np.concatenate([qs & 0x0F, qs >> 4], axis=2).reshape(N, K)
    d = blk[:, :, 0:2].copy().view("<u2").reshape(N, nb)
    return e, d


@pytest.mark.parametrize("N,K", [(16, 512), (37, 1024), (100, 512)])
def test_pack_roundtrip_and_size(orc, N, K):
    rng = np.random.default_rng(N * K)
    w = synth.q4_0_weights(rng, N, K)
    wp = orc.q4_0_pack(w, N, K)
    assert wp.size == w.size                      # same 18 bytes per 32 weights
    assert (orc.q4_0_unpack(wp, N, K) == w).all()


def test_pack_layout_element_by_element(orc):
    N, K = 21, 1024                               # one full tile of 16 rows and a ragged one of 5
    rng = np.random.default_rng(31)
    w = synth.q4_0_weights(rng, N, K)
    wp = orc.q4_0_pack(w, N, K)
    e, d = _elements(w, N, K)
    nb = K // 32
    QS, D = wp[:N * nb * 16], wp[N * nb * 16:].view("<u2")
    for n in range(N):
        n0 = n // 16 * 16
        r, rows_t = n - n0, min(16, N - n0)
        for b in range(nb):
            u, v = b // 4, (b % 4) // 2
            for j in range(32):
                h, jj = j // 16, j % 16
                g = 2 * (b % 2) + h
                byte = QS[n0 * nb * 16 + u * 4 * rows_t * 16 + (g * rows_t + r) * 16 + 8 * v + jj % 8]
                nib = (byte >> 4) if jj >= 8 else (byte & 0x0F)
                assert nib == e[n, 32 * b + j]
            at = n0 * nb + ((b // 16) * 2 + b % 2) * rows_t * 8 + r * 8 + (b % 16) // 2
            assert D[at] == d[n, b]
    # a tile's 16 rows of one (4-block group, lane group) are 256 contiguous bytes
    assert QS[:256].size == 256


@pytest.mark.parametrize("N,K,M", [(48, 512, 6), (37, 1536, 17), (16, 512, 1)])
def test_packed_product_equals_standard_product(orc, N, K, M):
    rng = np.random.default_rng(N + K + M)
    w, x = synth.random_q4_0_case(int(rng.integers(1 << 30)), N, K, M)
    xq = orc.q8_1_quantize(x)
    y, bound = orc.q4_0_gemv(w, N, K, xq, M)
    yp, boundp = orc.q4_0p_gemv(orc.q4_0_pack(w, N, K), N, K, xq, M)
    assert (yp == y).all() and (boundp == bound).all()
