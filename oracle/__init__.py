"""Python face of the scalar CPU oracle (``bq8_oracle.c``).

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the
benchmark's CPU-baseline leg are the only callers.  Nothing in the GPU
package imports this module, and this module imports nothing from it.

Every function takes and returns numpy arrays; byte-level formats (Q8_1,
Q4_0, raw Q6_K, expanded Q6_K pack) travel as ``uint8`` arrays and fp16
fields as raw ``uint16`` bits.  The arithmetic, layouts and readings are
documented in ``bq8_oracle.c``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "bq8_oracle.c")
_LIB = os.path.join(_HERE, "libbq8_oracle.so")

QK = 32
QK_K = 256
Q4_0_BYTES = 18
Q8_1_BYTES = 36
Q6_K_BYTES = 210

CFLAGS = ["-O2", "-ffp-contract=off", "-fno-fast-math", "-fopenmp", "-Wall", "-Wextra",
          "-shared", "-fPIC"]


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (binary64 accumulation, no contraction)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        subprocess.run(["gcc", *CFLAGS, "-o", tmp, _SRC, "-lm"], check=True)
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        _lib = ctypes.CDLL(_LIB)
        _declare(_lib)
    return _lib


_P = ctypes.c_void_p
_I64 = ctypes.c_int64


def _declare(L):
    L.orc_f16_to_f32.restype = ctypes.c_float
    L.orc_f16_to_f32.argtypes = [ctypes.c_uint16]
    L.orc_f32_to_f16.restype = ctypes.c_uint16
    L.orc_f32_to_f16.argtypes = [ctypes.c_float]
    L.orc_f32_to_f16_array.argtypes = [_P, _P, _I64]
    L.orc_f16_to_f32_array.argtypes = [_P, _P, _I64]
    L.orc_q8_1_quantize.argtypes = [_P, _I64, _I64, _P]
    L.orc_q8_1_fields.argtypes = [_P, _I64, _P, _P, _P]
    L.orc_q4_0_decode.argtypes = [_P, _I64, _I64, _P, _P]
    L.orc_q4_0_encode.argtypes = [_P, _P, _I64, _I64, _P]
    L.orc_q4_0_q8_1_gemv.argtypes = [_P, _I64, _I64, _P, _I64, _P, _P]
    L.orc_q4_0_pack_bytes.restype = _I64
    L.orc_q4_0_pack_bytes.argtypes = [_I64, _I64]
    L.orc_q4_0_pack.argtypes = [_P, _I64, _I64, _P]
    L.orc_q4_0_unpack.argtypes = [_P, _I64, _I64, _P]
    L.orc_q4_0p_q8_1_gemv.argtypes = [_P, _I64, _I64, _P, _I64, _P, _P]
    L.orc_q6k_decode.argtypes = [_P, _I64, _I64, _P, _P, _P]
    L.orc_q6k_encode.argtypes = [_P, _P, _P, _I64, _I64, _P]
    L.orc_q6k_pack_bytes.restype = _I64
    L.orc_q6k_pack_bytes.argtypes = [_I64, _I64]
    L.orc_q6k_pack_expand.argtypes = [_P, _I64, _I64, _P]
    L.orc_q6k_pack_logits.argtypes = [_P, _I64, _I64, _P, _I64, _P, _P]
    L.orc_q6k_compact_bytes.restype = _I64
    L.orc_q6k_compact_bytes.argtypes = [_I64, _I64]
    L.orc_q6k_pack_compact.argtypes = [_P, _I64, _I64, _P]
    L.orc_q6k_compact_unpack.argtypes = [_P, _I64, _I64, _P]
    L.orc_top1.argtypes = [_P, _I64, _I64, _P]
    L.orc_q6k_lmhead_top1.argtypes = [_P, _I64, _I64, _P, _I64, _I64, _I64, _P, _P, _P, _P]
    L.orc_silu_mul.argtypes = [_P, _P, _I64, _P]
    L.orc_rms_norm.argtypes = [_P, _I64, _I64, ctypes.c_double, _P]
    L.orc_num_threads.restype = ctypes.c_int
    L.orc_set_num_threads.argtypes = [ctypes.c_int]


def _ptr(a: np.ndarray) -> int:
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data


def _c(a, dtype) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=dtype)


# --------------------------------------------------------------------- fp16
def f32_to_f16_bits(x) -> np.ndarray:
    x = _c(x, np.float32)
    out = np.empty(x.shape, np.uint16)
    lib().orc_f32_to_f16_array(_ptr(x), _ptr(out), x.size)
    return out


def f16_bits_to_f32(h) -> np.ndarray:
    h = _c(h, np.uint16)
    out = np.empty(h.shape, np.float32)
    lib().orc_f16_to_f32_array(_ptr(h), _ptr(out), h.size)
    return out


# --------------------------------------------------------------------- Q8_1
def q8_1_quantize(x) -> np.ndarray:
    """f32 [M][K] -> Q8_1 bytes [M][K/32*36]."""
    x = _c(x, np.float32)
    M, K = x.shape
    assert K % QK == 0
    out = np.empty((M, K // QK * Q8_1_BYTES), np.uint8)
    lib().orc_q8_1_quantize(_ptr(x), M, K, _ptr(out))
    return out


def q8_1_fields(xq):
    """Q8_1 bytes -> (d bits [nblk], s bits [nblk], q int8 [nblk][32])."""
    xq = _c(xq, np.uint8)
    nblk = xq.size // Q8_1_BYTES
    d = np.empty(nblk, np.uint16)
    s = np.empty(nblk, np.uint16)
    q = np.empty((nblk, QK), np.int8)
    lib().orc_q8_1_fields(_ptr(xq), nblk, _ptr(d), _ptr(s), _ptr(q))
    return d, s, q


# --------------------------------------------------------------------- Q4_0
def q4_0_decode(w, N: int, K: int):
    """Q4_0 bytes -> (d bits [N*K/32], nibbles uint8 [N][K])."""
    w = _c(w, np.uint8)
    assert w.size == N * K // QK * Q4_0_BYTES
    d = np.empty(N * K // QK, np.uint16)
    q = np.empty((N, K), np.uint8)
    lib().orc_q4_0_decode(_ptr(w), N, K, _ptr(d), _ptr(q))
    return d, q


def q4_0_encode(d_bits, q, N: int, K: int) -> np.ndarray:
    d_bits = _c(d_bits, np.uint16)
    q = _c(q, np.uint8)
    w = np.empty((N, K // QK * Q4_0_BYTES), np.uint8)
    lib().orc_q4_0_encode(_ptr(d_bits), _ptr(q), N, K, _ptr(w))
    return w


def q4_0_gemv(w, N: int, K: int, xq, M: int):
    """(y [M][N] float64, bound [M][N] float64) for Q4_0 w times Q8_1 xq."""
    w = _c(w, np.uint8)
    xq = _c(xq, np.uint8)
    assert w.size == N * K // QK * Q4_0_BYTES
    assert xq.size == M * K // QK * Q8_1_BYTES
    y = np.empty((M, N), np.float64)
    bound = np.empty((M, N), np.float64)
    lib().orc_q4_0_q8_1_gemv(_ptr(w), N, K, _ptr(xq), M, _ptr(y), _ptr(bound))
    return y, bound


# ------------------------------------------------------------ packed Q4_0
def q4_0_pack(w, N: int, K: int) -> np.ndarray:
    """Q4_0 [N][K/32] blocks -> the offline-packed layout (K % 512 == 0)."""
    assert K % 512 == 0
    w = _c(w, np.uint8)
    assert w.size == N * K // QK * Q4_0_BYTES
    out = np.empty(int(lib().orc_q4_0_pack_bytes(N, K)), np.uint8)
    lib().orc_q4_0_pack(_ptr(w), N, K, _ptr(out))
    return out


def q4_0_unpack(wp, N: int, K: int) -> np.ndarray:
    """The inverse of q4_0_pack: Q4_0 bytes [N][K/32*18]."""
    wp = _c(wp, np.uint8)
    out = np.empty((N, K // QK * Q4_0_BYTES), np.uint8)
    lib().orc_q4_0_unpack(_ptr(wp), N, K, _ptr(out))
    return out


def q4_0p_gemv(wp, N: int, K: int, xq, M: int):
    """(y, bound) as q4_0_gemv, reading the packed layout."""
    wp = _c(wp, np.uint8)
    xq = _c(xq, np.uint8)
    assert wp.size == N * K // QK * Q4_0_BYTES
    assert xq.size == M * K // QK * Q8_1_BYTES
    y = np.empty((M, N), np.float64)
    bound = np.empty((M, N), np.float64)
    lib().orc_q4_0p_q8_1_gemv(_ptr(wp), N, K, _ptr(xq), M, _ptr(y), _ptr(bound))
    return y, bound


# --------------------------------------------------------------------- Q6_K
def q6k_decode(raw, N: int, K: int):
    """raw Q6_K -> (q int8 [N][K], sc int8 [N][K/16], d bits [N][K/256])."""
    raw = _c(raw, np.uint8)
    assert raw.size == N * K // QK_K * Q6_K_BYTES
    q = np.empty((N, K), np.int8)
    sc = np.empty((N, K // 16), np.int8)
    d = np.empty((N, K // QK_K), np.uint16)
    lib().orc_q6k_decode(_ptr(raw), N, K, _ptr(q), _ptr(sc), _ptr(d))
    return q, sc, d


def q6k_encode(q, sc, d_bits, N: int, K: int) -> np.ndarray:
    q = _c(q, np.int8)
    sc = _c(sc, np.int8)
    d_bits = _c(d_bits, np.uint16)
    raw = np.empty((N, K // QK_K * Q6_K_BYTES), np.uint8)
    lib().orc_q6k_encode(_ptr(q), _ptr(sc), _ptr(d_bits), N, K, _ptr(raw))
    return raw


def q6k_pack_bytes(N: int, K: int) -> int:
    return int(lib().orc_q6k_pack_bytes(N, K))


def q6k_pack_expand(raw, N: int, K: int) -> np.ndarray:
    raw = _c(raw, np.uint8)
    assert raw.size == N * K // QK_K * Q6_K_BYTES
    pack = np.empty(q6k_pack_bytes(N, K), np.uint8)
    lib().orc_q6k_pack_expand(_ptr(raw), N, K, _ptr(pack))
    return pack


def q6k_pack_logits(pack, N: int, K: int, xq, rows: int):
    pack = _c(pack, np.uint8)
    xq = _c(xq, np.uint8)
    assert pack.size == q6k_pack_bytes(N, K)
    assert xq.size == rows * K // QK * Q8_1_BYTES
    logits = np.empty((rows, N), np.float64)
    bound = np.empty((rows, N), np.float64)
    lib().orc_q6k_pack_logits(_ptr(pack), N, K, _ptr(xq), rows, _ptr(logits), _ptr(bound))
    return logits, bound


def q6k_compact_bytes(N: int, K: int) -> int:
    return int(lib().orc_q6k_compact_bytes(N, K))


def q6k_pack_compact(raw, N: int, K: int) -> np.ndarray:
    """raw Q6_K [N][K/256 * 210] -> the compact pack (the same bytes, re-tiled)."""
    raw = _c(raw, np.uint8)
    assert raw.size == q6k_compact_bytes(N, K)
    pack = np.empty(q6k_compact_bytes(N, K), np.uint8)
    lib().orc_q6k_pack_compact(_ptr(raw), N, K, _ptr(pack))
    return pack


def q6k_compact_unpack(pack, N: int, K: int) -> np.ndarray:
    pack = _c(pack, np.uint8)
    assert pack.size == q6k_compact_bytes(N, K)
    raw = np.empty((N, K // QK_K * Q6_K_BYTES), np.uint8)
    lib().orc_q6k_compact_unpack(_ptr(pack), N, K, _ptr(raw))
    return raw


def q6k_compact_lmhead_top1(cpack, N: int, K: int, x, row0: int, rows: int):
    """q6k_lmhead_top1 of the weights a compact pack encodes: unpack to raw
    Q6_K, expand, then the same quantize + logits + top-1."""
    return q6k_lmhead_top1(q6k_pack_expand(q6k_compact_unpack(cpack, N, K), N, K), N, K, x,
                           row0, rows)


def top1(logits) -> np.ndarray:
    logits = _c(logits, np.float64)
    rows, N = logits.shape
    ids = np.empty(rows, np.int32)
    lib().orc_top1(_ptr(logits), rows, N, _ptr(ids))
    return ids


def q6k_lmhead_top1(pack, N: int, K: int, x, row0: int, rows: int):
    """-> (ids int32 [rows], logits [rows][N], bound [rows][N], xq)."""
    pack = _c(pack, np.uint8)
    x = _c(x, np.float32)
    M = x.shape[0]
    assert x.shape[1] == K and 0 <= row0 and row0 + rows <= M
    xq = np.empty((rows, K // QK * Q8_1_BYTES), np.uint8)
    logits = np.empty((rows, N), np.float64)
    bound = np.empty((rows, N), np.float64)
    ids = np.empty(rows, np.int32)
    lib().orc_q6k_lmhead_top1(_ptr(pack), N, K, _ptr(x), M, row0, rows, _ptr(xq),
                              _ptr(logits), _ptr(bound), _ptr(ids))
    return ids, logits, bound, xq


# ------------------------------------------------------------ layer stages
def silu_mul(g, u) -> np.ndarray:
    g = _c(g, np.float32)
    u = _c(u, np.float32)
    assert g.shape == u.shape
    h = np.empty(g.shape, np.float64)
    lib().orc_silu_mul(_ptr(g), _ptr(u), g.size, _ptr(h))
    return h


def rms_norm(y, eps: float) -> np.ndarray:
    y = _c(y, np.float32)
    M, K = y.shape
    out = np.empty((M, K), np.float64)
    lib().orc_rms_norm(_ptr(y), M, K, float(eps), _ptr(out))
    return out


def num_threads() -> int:
    return int(lib().orc_num_threads())


def set_num_threads(n: int) -> None:
    """Threads for the loops over output rows (results do not change)."""
    lib().orc_set_num_threads(int(n))


# ------------------------------------------------------------ comparators
def within_tol(gpu, ref, bound, rel=1e-5, abs_=1e-6):
    """Boolean mask of |gpu - ref| <= rel * bound + abs_ (the parity rule for
    float outputs: bound is the sum of |32-block contributions|)."""
    return np.abs(np.asarray(gpu, np.float64) - ref) <= rel * bound + abs_
