"""Pins of the oracle's compact Q6_K pack (the raw Q6_K bits re-tiled).

The layout is this library's own (include/bq8.h), so what is pinned is what
it must guarantee: it holds exactly the raw bytes (its size is the raw size
and unpacking restores the raw superblocks bit for bit, ragged tiles
included); each 64-row tile stores 16-byte piece p of all its rows
contiguously, rows in order, for the ql and qh planes (the purpose of the
layout); its subscale and scale planes are the expanded pack's, byte for
byte (the expanded planes are pinned value by value against the decoded raw
blocks); and the weights it encodes are the raw format's, so top-1 through
it equals top-1 through the raw weights' expanded pack, logits bitwise.
"""
import numpy as np
import pytest

from block_quantized_gemv_q8_amd import synth

SHAPES = [(1, 256), (70, 512), (130, 768), (64, 256), (65, 1024)]


def test_size_is_the_raw_size(orc):
    assert orc.q6k_compact_bytes(248320, 5120) == 1_042_944_000     # 210 B per 256 weights
    assert orc.q6k_compact_bytes(1, 256) == 210
    assert orc.q6k_compact_bytes(248320, 5120) * 256 == 210 * 248320 * 5120


@pytest.mark.parametrize("N,K", SHAPES)
def test_roundtrip_restores_raw(orc, N, K):
    rng = np.random.default_rng(900 + N + K)
    raw = synth.q6k_raw_weights(rng, N, K)
    cp = orc.q6k_pack_compact(raw, N, K)
    assert cp.size == raw.size
    assert (orc.q6k_compact_unpack(cp, N, K) == raw).all()
    # a permutation of the raw bytes: the same multiset of byte values
    assert (np.bincount(cp, minlength=256) == np.bincount(raw.ravel(), minlength=256)).all()


def test_pieces_are_contiguous_per_tile(orc):
    """Mark every raw byte with its (row, superblock, byte) and read the planes back."""
    N, K = 130, 512                      # tiles of 64, 64, 2 rows; two superblocks a row
    ns = K // 256
    raw = np.zeros((N, ns * 210), np.uint8)
    cps = []
    for field in range(3):               # encode row, superblock and byte index in turn
        for n in range(N):
            for s in range(ns):
                for i in range(210):
                    raw[n, s * 210 + i] = (n, s, i)[field] % 256
        cps.append(orc.q6k_pack_compact(raw, N, K))
    row_of, sb_of, byte_of = cps
    ql_plane = N * K // 2
    for n0, rows_t in [(0, 64), (64, 64), (128, 2)]:
        base = n0 * K // 2
        for p in range(8 * ns):          # 16-byte pieces of the ql plane
            for r in range(rows_t):
                o = base + (p * rows_t + r) * 16
                assert (row_of[o:o + 16] == n0 + r).all()
                assert (sb_of[o:o + 16] == p // 8).all()
                assert (byte_of[o:o + 16] == np.arange(16) + 16 * (p % 8)).all()
        base = ql_plane + n0 * K // 4
        for p in range(4 * ns):          # qh plane
            for r in range(rows_t):
                o = base + (p * rows_t + r) * 16
                assert (row_of[o:o + 16] == n0 + r).all()
                assert (sb_of[o:o + 16] == p // 4).all()
                assert (byte_of[o:o + 16] == 128 + np.arange(16) + 16 * (p % 4)).all()


@pytest.mark.parametrize("N,K", SHAPES)
def test_subscale_and_scale_planes_are_the_expanded_packs(orc, N, K):
    rng = np.random.default_rng(970 + N + K)
    raw = synth.q6k_raw_weights(rng, N, K)
    cp = orc.q6k_pack_compact(raw, N, K)
    ep = orc.q6k_pack_expand(raw, N, K)
    c_sc = N * K // 2 + N * K // 4       # after the ql and qh planes
    e_sc = N * K                         # after the int8 quants
    n_sc, n_d = N * K // 16, N * K // 128
    assert (cp[c_sc:c_sc + n_sc] == ep[e_sc:e_sc + n_sc]).all()
    assert (cp[c_sc + n_sc:] == ep[e_sc + n_sc:]).all()
    assert cp.size - (c_sc + n_sc) == n_d == ep.size - (e_sc + n_sc)


@pytest.mark.parametrize("N,K,rows", [(300, 512, 5), (65, 768, 6), (1, 256, 3)])
def test_compact_top1_equals_raw_top1(orc, N, K, rows):
    rng = np.random.default_rng(950 + N)
    raw = synth.q6k_raw_weights(rng, N, K)
    x = synth.normal_rows(rng, rows + 1, K)
    a = orc.q6k_lmhead_top1(orc.q6k_pack_expand(raw, N, K), N, K, x, 1, rows)
    b = orc.q6k_compact_lmhead_top1(orc.q6k_pack_compact(raw, N, K), N, K, x, 1, rows)
    assert (a[0] == b[0]).all()
    assert (a[1].view(np.uint64) == b[1].view(np.uint64)).all()
