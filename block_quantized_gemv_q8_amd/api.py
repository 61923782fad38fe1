"""Thin Python binding of libbq8 (include/bq8.h): argument marshalling only.

Each function takes torch tensors on the current HIP device, checks their
dtype and shape, and calls the C entry point of the same name with raw device
pointers and the current stream (``torch.cuda.current_stream()``).  Every
step of the computation runs in the library's HIP kernels; there is no other
code path.  Output tensors may be passed in (preallocated) or are allocated
here with ``torch.empty``.  A nonzero status from the library raises
``Bq8Error``.  If libbq8.so has not been built the first call raises.
"""
from __future__ import annotations

import ctypes
import os

import torch  # loads the HIP runtime libbq8 links against (same soname)

from . import synth

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libbq8.so")

QK = 32
QK_K = 256
Q4_0_BYTES = 18
Q8_1_BYTES = 36
Q6_K_BYTES = 210
MAX_M = 17

_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_ST = ctypes.c_int32


class Bq8Error(RuntimeError):
    def __init__(self, fn: str, status: int, message: str):
        super().__init__(f"{fn}: status {status}: {message}")
        self.status = status


_lib = None


def lib() -> ctypes.CDLL:
    """Load libbq8.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"libbq8.so not found at {LIB_PATH}; build it with "
                "`python -m block_quantized_gemv_q8_amd.build` (hipcc, gfx950)")
        L = ctypes.CDLL(LIB_PATH)
        L.bq8_status_string.restype = ctypes.c_char_p
        L.bq8_status_string.argtypes = [_ST]
        L.bq8_abi_version.restype = ctypes.c_int32
        L.bq8_abi_version.argtypes = []
        L.q8_1_quantize.restype = _ST
        L.q8_1_quantize.argtypes = [_P, _I64, _I64, _P, _P]
        for m in range(1, MAX_M + 1):
            f = getattr(L, f"q4_0_mmvq_m{m}")
            f.restype = _ST
            f.argtypes = [_P, _I64, _I64, _P, _P, _P]
        L.q4_0_mmvq.restype = _ST
        L.q4_0_mmvq.argtypes = [_P, _I64, _I64, _P, _I64, _P, _P]
        L.q6k_pack_bytes.restype = _I64
        L.q6k_pack_bytes.argtypes = [_I64, _I64]
        L.q6k_pack_expand.restype = _ST
        L.q6k_pack_expand.argtypes = [_P, _I64, _I64, _P, _I64, _P]
        L.q6k_lmhead_top1_scratch_bytes.restype = _I64
        L.q6k_lmhead_top1_scratch_bytes.argtypes = [_I64, _I64, _I64]
        L.q6k_lmhead_top1.restype = _ST
        L.q6k_lmhead_top1.argtypes = [_P, _I64, _I64, _P, _I64, _I64, _I64, _P, _P, _I64, _P]
        L.q6k_lmhead_top1_noalloc.restype = _ST
        L.q6k_lmhead_top1_noalloc.argtypes = [_P, _I64, _I64, _P, _I64, _I64, _I64, _P, _P]
        L.q6k_lmhead_candidate_max.restype = _ST
        L.q6k_lmhead_candidate_max.argtypes = [_P, _I64, _I64, _P, _I64, _I64, _I64, _P, _I64,
                                               _P, _P, _P, _P, _I64, _P]
        L.q6k_compact_bytes.restype = _I64
        L.q6k_compact_bytes.argtypes = [_I64, _I64]
        L.q6k_pack_compact.restype = _ST
        L.q6k_pack_compact.argtypes = [_P, _I64, _I64, _P, _I64, _P]
        L.q6k_lmhead_top1_compact.restype = _ST
        L.q6k_lmhead_top1_compact.argtypes = [_P, _I64, _I64, _P, _I64, _I64, _I64, _P, _P, _I64,
                                              _P]
        L.q6k_lmhead_candidate_max_compact.restype = _ST
        L.q6k_lmhead_candidate_max_compact.argtypes = [_P, _I64, _I64, _P, _I64, _I64, _I64, _P,
                                                       _I64, _P, _P, _P, _P, _I64, _P]
        L.silu_mul_q8_1.restype = _ST
        L.silu_mul_q8_1.argtypes = [_P, _P, _I64, _I64, _P, _P, _P]
        L.rms_norm_q8_1.restype = _ST
        L.rms_norm_q8_1.argtypes = [_P, _I64, _I64, ctypes.c_float, _P, _P, _P]
        L.q4_0_pack_bytes.restype = _I64
        L.q4_0_pack_bytes.argtypes = [_I64, _I64]
        L.q4_0_pack.restype = _ST
        L.q4_0_pack.argtypes = [_P, _I64, _I64, _P, _I64, _P]
        L.q4_0_mmvq_packed.restype = _ST
        L.q4_0_mmvq_packed.argtypes = [_P, _I64, _I64, _P, _I64, _P, _P]
        L.q4_0_mmvq_packed_ws_bytes.restype = _I64
        L.q4_0_mmvq_packed_ws_bytes.argtypes = []
        L.q4_0_mmvq_packed_ws.restype = _ST
        L.q4_0_mmvq_packed_ws.argtypes = [_P, _I64, _I64, _P, _I64, _P, _P, _I64, _P]
        L.q4_0_mmvq_packed_split.restype = _ST
        L.q4_0_mmvq_packed_split.argtypes = [_P, _I64, _I64, _P, _I64, _I64, _P, _P]
        L.q4_0_mmvq_packed_splits.restype = _I64
        L.q4_0_mmvq_packed_splits.argtypes = [_I64, _I64]
        L.q4_0_mmvq_packed_splits_rows.restype = _I64
        L.q4_0_mmvq_packed_splits_rows.argtypes = [_I64, _I64, _I64]
        L.rms_norm_q8_1_sum.restype = _ST
        L.rms_norm_q8_1_sum.argtypes = [_P, _I64, _I64, _I64, ctypes.c_float, _P, _P, _P, _P]
        L.q4_0_gate_up_silu_q8_1_packed.restype = _ST
        L.q4_0_gate_up_silu_q8_1_packed.argtypes = [_P, _P, _I64, _I64, _P, _I64, _P, _P, _P,
                                                    _P, _P]
        L.q4_0_gate_up_silu_q8_1_packed_ws.restype = _ST
        L.q4_0_gate_up_silu_q8_1_packed_ws.argtypes = [_P, _P, _I64, _I64, _P, _I64, _P, _P, _P,
                                                       _P, _P, _I64, _P]
        L.bq8_hbm_read_probe.restype = _ST
        L.bq8_hbm_read_probe.argtypes = [_P, _I64, _I64, _I64, _P, _P]
        L.q4_0_ffn_stream_layout.restype = _ST
        L.q4_0_ffn_stream_layout.argtypes = [_I64, _I64, _I64, ctypes.POINTER(_I64)]
        for f in (L.q4_0_ffn_stream, L.q4_0_ffn_stream_packed):
            f.restype = _ST
            f.argtypes = [_P, _P, _P, _I64, _I64, _I64, _I64, _P, ctypes.c_float, _P, _P, _I64, _P]
        _lib = L
    return _lib


def _check(fn: str, status: int):
    if status != 0:
        msg = lib().bq8_status_string(status).decode()
        raise Bq8Error(fn, status, msg)


try:  # the raw handle of the current stream without building a Stream object
    _raw_stream = torch._C._cuda_getCurrentRawStream
except AttributeError:  # pragma: no cover - older torch
    def _raw_stream(device):
        return torch.cuda.current_stream(device).cuda_stream


def _stream():
    return _raw_stream(torch.cuda.current_device())


def _dev(t: torch.Tensor, name: str, dtype=None) -> int:
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a device tensor")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t.data_ptr()


def _out(t, shape, dtype, device, name):
    if t is None:
        return torch.empty(shape, dtype=dtype, device=device)
    if tuple(t.shape) != tuple(shape) or t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype} {tuple(shape)}, got {t.dtype} {tuple(t.shape)}")
    return t


def status_string(status: int) -> str:
    return lib().bq8_status_string(status).decode()


def abi_version() -> int:
    return int(lib().bq8_abi_version())


# ----------------------------------------------------------------- Q8_1
def q8_1_quantize(x: torch.Tensor, xq: torch.Tensor | None = None) -> torch.Tensor:
    """f32 [M][K] -> Q8_1 uint8 [M][K/32*36]."""
    M, K = x.shape
    xq = _out(xq, (M, K // QK * Q8_1_BYTES), torch.uint8, x.device, "xq")
    _check("q8_1_quantize", lib().q8_1_quantize(_dev(x, "x", torch.float32), M, K,
                                                _dev(xq, "xq", torch.uint8), _stream()))
    return xq


# ----------------------------------------------------------------- Q4_0
def _q4_0_shape(w: torch.Tensor):
    N, row_bytes = w.shape
    if row_bytes % Q4_0_BYTES:
        raise ValueError("w rows must hold whole 18-byte Q4_0 blocks")
    return N, row_bytes // Q4_0_BYTES * QK


def q4_0_mmvq(w: torch.Tensor, xq: torch.Tensor, M: int, y: torch.Tensor | None = None):
    """Q4_0 w uint8 [N][K/32*18] times M Q8_1 rows -> f32 y [M][N]."""
    N, K = _q4_0_shape(w)
    if xq.numel() < M * (K // QK) * Q8_1_BYTES:
        raise ValueError("xq holds fewer than M quantized rows of length K")
    y = _out(y, (M, N), torch.float32, w.device, "y")
    _check("q4_0_mmvq", lib().q4_0_mmvq(_dev(w, "w", torch.uint8), N, K,
                                        _dev(xq, "xq", torch.uint8), M,
                                        _dev(y, "y", torch.float32), _stream()))
    return y


def _make_mmvq(m: int):
    name = f"q4_0_mmvq_m{m}"

    def fn(w: torch.Tensor, xq: torch.Tensor, y: torch.Tensor | None = None):
        N, K = _q4_0_shape(w)
        if xq.numel() < m * (K // QK) * Q8_1_BYTES:
            raise ValueError("xq holds fewer than M quantized rows of length K")
        y = _out(y, (m, N), torch.float32, w.device, "y")
        _check(name, getattr(lib(), name)(_dev(w, "w", torch.uint8), N, K,
                                          _dev(xq, "xq", torch.uint8),
                                          _dev(y, "y", torch.float32), _stream()))
        return y

    fn.__name__ = name
    fn.__doc__ = f"Q4_0 x Q8_1 at M={m}: y [{m}][N] = W x^T (C entry point {name})."
    return fn


for _m in range(1, MAX_M + 1):
    globals()[f"q4_0_mmvq_m{_m}"] = _make_mmvq(_m)
del _m


# ----------------------------------------------------------------- Q6_K
def q6k_pack_bytes(N: int, K: int) -> int:
    return int(lib().q6k_pack_bytes(N, K))


def q6k_pack_expand(raw: torch.Tensor, N: int, K: int, pack: torch.Tensor | None = None):
    """raw Q6_K uint8 [N][K/256*210] -> expanded pack uint8 [q6k_pack_bytes]."""
    nbytes = q6k_pack_bytes(N, K)
    if nbytes < 0:
        raise ValueError("invalid Q6_K shape")
    if raw.numel() != N * (K // QK_K) * Q6_K_BYTES:
        raise ValueError("raw does not hold N x K/256 superblocks")
    pack = _out(pack, (nbytes,), torch.uint8, raw.device, "pack")
    _check("q6k_pack_expand", lib().q6k_pack_expand(_dev(raw, "raw", torch.uint8), N, K,
                                                    _dev(pack, "pack", torch.uint8),
                                                    pack.numel(), _stream()))
    return pack


def q6k_lmhead_top1_scratch_bytes(N: int, K: int, rows: int) -> int:
    return int(lib().q6k_lmhead_top1_scratch_bytes(N, K, rows))


def q6k_lmhead_top1(pack: torch.Tensor, N: int, K: int, x: torch.Tensor, row0: int, rows: int,
                    ids: torch.Tensor | None = None, scratch: torch.Tensor | None = None,
                    compact: bool = False):
    """Greedy ids int32 [rows] of rows row0.. of f32 x [M][K] through the pack
    (the expanded pack, or the compact one with compact=True)."""
    M = x.shape[0]
    if x.shape[1] != K:
        raise ValueError("x must be [M][K]")
    ids = _out(ids, (rows,), torch.int32, x.device, "ids")
    need = q6k_lmhead_top1_scratch_bytes(N, K, rows)
    if scratch is None:
        scratch = torch.empty(max(need, 16), dtype=torch.uint8, device=x.device)
    name = "q6k_lmhead_top1_compact" if compact else "q6k_lmhead_top1"
    _check(name, getattr(lib(), name)(
        _dev(pack, "pack", torch.uint8), N, K, _dev(x, "x", torch.float32), M, row0, rows,
        _dev(ids, "ids", torch.int32), _dev(scratch, "scratch", torch.uint8), scratch.numel(),
        _stream()))
    return ids


def q6k_lmhead_top1_noalloc(pack: torch.Tensor, N: int, K: int, x: torch.Tensor, row0: int,
                            rows: int, ids: torch.Tensor | None = None):
    """q6k_lmhead_top1 on the expanded pack with the library's own per-GPU
    scratch: nothing is allocated on the device but ids when not given."""
    M = x.shape[0]
    if x.shape[1] != K:
        raise ValueError("x must be [M][K]")
    ids = _out(ids, (rows,), torch.int32, x.device, "ids")
    _check("q6k_lmhead_top1_noalloc", lib().q6k_lmhead_top1_noalloc(
        _dev(pack, "pack", torch.uint8), N, K, _dev(x, "x", torch.float32), M, row0, rows,
        _dev(ids, "ids", torch.int32), _stream()))
    return ids


def q6k_compact_bytes(N: int, K: int) -> int:
    return int(lib().q6k_compact_bytes(N, K))


def q6k_pack_compact(raw: torch.Tensor, N: int, K: int, pack: torch.Tensor | None = None):
    """raw Q6_K uint8 [N][K/256*210] -> the compact pack, uint8 [bytes]."""
    nbytes = q6k_compact_bytes(N, K)
    if nbytes < 0:
        raise Bq8Error("q6k_pack_compact", 2, status_string(2))
    pack = _out(pack, (nbytes,), torch.uint8, raw.device, "pack")
    _check("q6k_pack_compact", lib().q6k_pack_compact(
        _dev(raw, "raw", torch.uint8), N, K, _dev(pack, "pack", torch.uint8), pack.numel(),
        _stream()))
    return pack


def q6k_lmhead_candidate_max(pack: torch.Tensor, N: int, K: int, x: torch.Tensor, row0: int,
                             rows: int, cand_ids: torch.Tensor | None = None,
                             scratch: torch.Tensor | None = None, compact: bool = False,
                             ids: torch.Tensor | None = None, vals: torch.Tensor | None = None,
                             scores: torch.Tensor | None = None):
    """(ids int32 [rows], top_vals f32 [rows], cand_scores f32 [rows][ncand]) of
    rows row0.. of x through the pack; cand_ids int32 [rows][ncand] (or None).
    ids, vals, scores may be given (preallocated outputs)."""
    M = x.shape[0]
    if x.shape[1] != K:
        raise ValueError("x must be [M][K]")
    ncand = 0 if cand_ids is None else cand_ids.shape[1]
    if cand_ids is not None and cand_ids.shape[0] != rows:
        raise ValueError("cand_ids must be [rows][ncand]")
    ids = _out(ids, (rows,), torch.int32, x.device, "ids")
    vals = _out(vals, (rows,), torch.float32, x.device, "vals")
    scores = _out(scores, (rows, ncand), torch.float32, x.device, "scores")
    need = q6k_lmhead_top1_scratch_bytes(N, K, rows)
    if scratch is None:
        scratch = torch.empty(max(need, 16), dtype=torch.uint8, device=x.device)
    cp = _dev(cand_ids, "cand_ids", torch.int32) if ncand else None
    sp = _dev(scores, "cand_scores", torch.float32) if ncand else None
    name = "q6k_lmhead_candidate_max_compact" if compact else "q6k_lmhead_candidate_max"
    _check(name, getattr(lib(), name)(
        _dev(pack, "pack", torch.uint8), N, K, _dev(x, "x", torch.float32), M, row0, rows, cp,
        ncand, _dev(ids, "ids", torch.int32), _dev(vals, "top_vals", torch.float32), sp,
        _dev(scratch, "scratch", torch.uint8), scratch.numel(), _stream()))
    return ids, vals, scores


# --------------------------------------------------------- layer glue
def silu_mul_q8_1(g: torch.Tensor, u: torch.Tensor, hq: torch.Tensor | None = None,
                  h: torch.Tensor | None = None):
    """hq = Q8_1(SiLU(g) * u); if h is given it receives the f32 product."""
    M, N = g.shape
    if tuple(u.shape) != (M, N):
        raise ValueError("g and u must have the same shape")
    hq = _out(hq, (M, N // QK * Q8_1_BYTES), torch.uint8, g.device, "hq")
    hp = None if h is None else _dev(_out(h, (M, N), torch.float32, g.device, "h"), "h")
    _check("silu_mul_q8_1", lib().silu_mul_q8_1(_dev(g, "g", torch.float32),
                                                _dev(u, "u", torch.float32), M, N, hp,
                                                _dev(hq, "hq", torch.uint8), _stream()))
    return hq


def rms_norm_q8_1(y: torch.Tensor, eps: float, xq: torch.Tensor | None = None,
                  x: torch.Tensor | None = None):
    """xq = Q8_1(y / sqrt(mean(y^2) + eps)) per row; x receives the f32 rows."""
    M, K = y.shape
    xq = _out(xq, (M, K // QK * Q8_1_BYTES), torch.uint8, y.device, "xq")
    xp = None if x is None else _dev(_out(x, (M, K), torch.float32, y.device, "x"), "x")
    _check("rms_norm_q8_1", lib().rms_norm_q8_1(_dev(y, "y", torch.float32), M, K, float(eps),
                                                xp, _dev(xq, "xq", torch.uint8), _stream()))
    return xq


def rms_norm_q8_1_sum(yparts: torch.Tensor, eps: float, xq: torch.Tensor | None = None,
                      y: torch.Tensor | None = None, x: torch.Tensor | None = None,
                      want_xq: bool = True):
    """The RMS step on the part-order sum of yparts (f32 [P][M][K]): returns
    xq (Q8_1 [M][K/32]) unless want_xq is False; y and x, if given, receive
    the summed and the normalized rows."""
    P, M, K = yparts.shape
    if want_xq:
        xq = _out(xq, (M, K // QK * Q8_1_BYTES), torch.uint8, yparts.device, "xq")
    xqp = _dev(xq, "xq", torch.uint8) if want_xq else None
    yp = None if y is None else _dev(_out(y, (M, K), torch.float32, yparts.device, "y"), "y")
    xp = None if x is None else _dev(_out(x, (M, K), torch.float32, yparts.device, "x"), "x")
    _check("rms_norm_q8_1_sum", lib().rms_norm_q8_1_sum(
        _dev(yparts, "yparts", torch.float32), P, M, K, float(eps), yp, xp, xqp, _stream()))
    return xq if want_xq else None


# ------------------------------------------------------------ packed Q4_0
def q4_0_pack_bytes(N: int, K: int) -> int:
    return int(lib().q4_0_pack_bytes(N, K))


def q4_0_pack(w: torch.Tensor, wp: torch.Tensor | None = None) -> torch.Tensor:
    """Q4_0 uint8 [N][K/32*18] -> the offline-packed layout, uint8 [bytes]."""
    N, K = _q4_0_shape(w)
    nbytes = q4_0_pack_bytes(N, K)
    if nbytes < 0:
        raise Bq8Error("q4_0_pack", 2, status_string(2))
    wp = _out(wp, (nbytes,), torch.uint8, w.device, "wp")
    _check("q4_0_pack", lib().q4_0_pack(_dev(w, "w", torch.uint8), N, K,
                                        _dev(wp, "wp", torch.uint8), wp.numel(), _stream()))
    return wp


def q4_0_mmvq_packed(wp: torch.Tensor, N: int, K: int, xq: torch.Tensor, M: int,
                     y: torch.Tensor | None = None, ws: torch.Tensor | None = None
                     ) -> torch.Tensor:
    """y f32 [M][N] = packed Q4_0 weight times the M Q8_1 rows of xq.  With a
    workspace ws (from q4_0_mmvq_packed_workspace) the launch balances the
    tiles over the CUs (q4_0_mmvq_packed_ws): the tiles past the last
    multiple of the CU count are summed in K ranges, so their outputs differ
    from the plain launch's in binary32 rounding only."""
    y = _out(y, (M, N), torch.float32, wp.device, "y")
    if ws is None:
        _check("q4_0_mmvq_packed", lib().q4_0_mmvq_packed(
            _dev(wp, "wp", torch.uint8), N, K, _dev(xq, "xq", torch.uint8), M,
            _dev(y, "y", torch.float32), _stream()))
    else:
        _check("q4_0_mmvq_packed_ws", lib().q4_0_mmvq_packed_ws(
            _dev(wp, "wp", torch.uint8), N, K, _dev(xq, "xq", torch.uint8), M,
            _dev(y, "y", torch.float32), _dev(ws, "ws", torch.uint8), ws.numel(), _stream()))
    return y


def q4_0_mmvq_packed_ws_bytes() -> int:
    """Workspace bytes q4_0_mmvq_packed_ws needs on the current device."""
    n = int(lib().q4_0_mmvq_packed_ws_bytes())
    if n < 0:
        raise Bq8Error("q4_0_mmvq_packed_ws_bytes", 5, "no current HIP device")
    return n


def q4_0_mmvq_packed_workspace(device=None) -> torch.Tensor:
    """A zeroed workspace for q4_0_mmvq_packed_ws on device (the current one
    by default).  One per stream: calls that overlap in time must not share
    one."""
    device = torch.device("cuda", torch.cuda.current_device()) if device is None else device
    with torch.cuda.device(device):
        return torch.zeros(q4_0_mmvq_packed_ws_bytes(), dtype=torch.uint8, device=device)


def q4_0_mmvq_packed_splits(N: int, K: int) -> int:
    return int(lib().q4_0_mmvq_packed_splits(N, K))


def q4_0_mmvq_packed_splits_rows(N: int, K: int, M: int) -> int:
    """The K-range count for a split launch of M rows on the current device
    (-1 for an invalid shape, or without a device at M >= 11)."""
    return int(lib().q4_0_mmvq_packed_splits_rows(N, K, M))


def q4_0_mmvq_packed_split(wp: torch.Tensor, N: int, K: int, xq: torch.Tensor, M: int,
                           nsplit: int, ypart: torch.Tensor | None = None) -> torch.Tensor:
    """ypart f32 [nsplit][M][N]: the packed product with K cut into nsplit
    chunk ranges; y = ypart[0] + ypart[1] + ... in that order."""
    ypart = _out(ypart, (nsplit, M, N), torch.float32, wp.device, "ypart")
    _check("q4_0_mmvq_packed_split", lib().q4_0_mmvq_packed_split(
        _dev(wp, "wp", torch.uint8), N, K, _dev(xq, "xq", torch.uint8), M, nsplit,
        _dev(ypart, "ypart", torch.float32), _stream()))
    return ypart


def q4_0_gate_up_silu_q8_1_packed(wg: torch.Tensor, wu: torch.Tensor, N: int, K: int,
                                  xq: torch.Tensor, M: int, hq: torch.Tensor | None = None,
                                  g: torch.Tensor | None = None, u: torch.Tensor | None = None,
                                  h: torch.Tensor | None = None,
                                  ws: torch.Tensor | None = None) -> torch.Tensor:
    """hq = Q8_1(SiLU(W_gate X) * (W_up X)) in one launch, from the packed gate
    and up weights (q4_0_pack of Q4_0 [N][K] each) and the M Q8_1 rows of xq.
    g, u, h, if given (f32 [M][N]), receive the two products and SiLU(g)*u.
    With a workspace ws (q4_0_mmvq_packed_workspace) the launch balances the
    32-column groups over the CUs (q4_0_gate_up_silu_q8_1_packed_ws)."""
    hq = _out(hq, (M, N // QK * Q8_1_BYTES), torch.uint8, wg.device, "hq")
    opt = [None if t is None else _dev(_out(t, (M, N), torch.float32, wg.device, name), name)
           for t, name in ((g, "g"), (u, "u"), (h, "h"))]
    if ws is None:
        _check("q4_0_gate_up_silu_q8_1_packed", lib().q4_0_gate_up_silu_q8_1_packed(
            _dev(wg, "wg", torch.uint8), _dev(wu, "wu", torch.uint8), N, K,
            _dev(xq, "xq", torch.uint8), M, *opt, _dev(hq, "hq", torch.uint8), _stream()))
    else:
        _check("q4_0_gate_up_silu_q8_1_packed_ws", lib().q4_0_gate_up_silu_q8_1_packed_ws(
            _dev(wg, "wg", torch.uint8), _dev(wu, "wu", torch.uint8), N, K,
            _dev(xq, "xq", torch.uint8), M, *opt, _dev(hq, "hq", torch.uint8),
            _dev(ws, "ws", torch.uint8), ws.numel(), _stream()))
    return hq


# ------------------------------------------------------- verifier stream
def q4_0_ffn_stream_layout(M: int, hidden: int, ffn: int) -> dict:
    """Byte offsets of the stage buffers in the stream workspace and its size."""
    off = (ctypes.c_int64 * 5)()
    _check("q4_0_ffn_stream_layout", lib().q4_0_ffn_stream_layout(M, hidden, ffn, off))
    return dict(xq=off[0], g=off[1], u=off[2], hq=off[3], total=off[4])


def stream_weight_table(ws) -> ctypes.Array:
    """Host array of the device addresses of a list of weight tensors."""
    return (ctypes.c_void_p * len(ws))(*[_dev(w, "weight", torch.uint8) for w in ws])


def q4_0_ffn_stream(w_gate, w_up, w_down, x0: torch.Tensor, eps: float,
                    y: torch.Tensor | None = None, work: torch.Tensor | None = None,
                    tables=None, packed: bool = False, hidden: int | None = None,
                    ffn: int | None = None):
    """Enqueue a whole verifier FFN pass over len(w_gate) layers.

    Standard weights: w_gate/w_up Q4_0 uint8 [ffn][hidden/32*18] per layer,
    w_down Q4_0 uint8 [hidden][ffn/32*18].  packed=True: the q4_0_pack of each
    matrix (uint8 vectors of the same byte count).  x0: f32 [M][hidden].
    Returns (y, work); the stage buffers of the last layer are views of work
    (see stream_stages).  ``tables`` may hold the three prebuilt
    stream_weight_table arrays."""
    M, hid = x0.shape
    layers = len(w_gate)
    if layers < 1 or len(w_up) != layers or len(w_down) != layers:
        raise ValueError("w_gate, w_up and w_down must list the same number of layers (>= 1)")
    if packed:
        if ffn is None:
            raise ValueError("packed weights need ffn")
        nbytes = q4_0_pack_bytes(ffn, hid)
        for w in (*w_gate, *w_up, *w_down):
            if w.dim() != 1 or w.numel() != nbytes:
                raise ValueError("every packed weight must be a uint8 vector of q4_0_pack_bytes")
    else:
        ffn, k = _q4_0_shape(w_gate[0])
        if k != hid:
            raise ValueError("gate weights must have K = hidden")
        for w in (*w_gate, *w_up):
            if _q4_0_shape(w) != (ffn, hid):
                raise ValueError("every gate/up weight must be Q4_0 [ffn][hidden/32]")
        for w in w_down:
            if _q4_0_shape(w) != (hid, ffn):
                raise ValueError("every down weight must be Q4_0 [hidden][ffn/32]")
    lay = q4_0_ffn_stream_layout(M, hid, ffn)
    y = _out(y, (M, hid), torch.float32, x0.device, "y")
    work = _out(work, (lay["total"],), torch.uint8, x0.device, "work")
    tg, tu, td = tables if tables is not None else (
        stream_weight_table(w_gate), stream_weight_table(w_up), stream_weight_table(w_down))
    fn = lib().q4_0_ffn_stream_packed if packed else lib().q4_0_ffn_stream
    _check("q4_0_ffn_stream" + ("_packed" if packed else ""), fn(
        tg, tu, td, layers, M, hid, ffn, _dev(x0, "x0", torch.float32), float(eps),
        _dev(y, "y", torch.float32), _dev(work, "work", torch.uint8), work.numel(), _stream()))
    return y, work


def stream_stages(work: torch.Tensor, M: int, hidden: int, ffn: int) -> dict:
    """Views of the last layer's stage buffers inside a stream workspace."""
    lay = q4_0_ffn_stream_layout(M, hidden, ffn)
    nq_h, nq_f = hidden // QK * Q8_1_BYTES, ffn // QK * Q8_1_BYTES
    return dict(
        xq=work[lay["xq"]:lay["xq"] + M * nq_h].view(M, nq_h),
        g=work[lay["g"]:lay["g"] + 4 * M * ffn].view(torch.float32).view(M, ffn),
        u=work[lay["u"]:lay["u"] + 4 * M * ffn].view(torch.float32).view(M, ffn),
        hq=work[lay["hq"]:lay["hq"] + M * nq_f].view(M, nq_f))


__all__ = ["Bq8Error", "lib", "status_string", "abi_version", "q8_1_quantize", "q4_0_mmvq",
           *[f"q4_0_mmvq_m{m}" for m in range(1, MAX_M + 1)], "q6k_pack_bytes",
           "q6k_pack_expand", "q6k_lmhead_top1_scratch_bytes", "q6k_lmhead_top1",
           "q6k_lmhead_candidate_max", "q6k_compact_bytes", "q6k_pack_compact",
           "silu_mul_q8_1", "rms_norm_q8_1", "rms_norm_q8_1_sum", "q4_0_pack_bytes", "q4_0_pack",
           "q4_0_mmvq_packed", "q4_0_mmvq_packed_split", "q4_0_mmvq_packed_splits",
           "q4_0_mmvq_packed_splits_rows",
           "q4_0_gate_up_silu_q8_1_packed", "q4_0_ffn_stream_layout", "q4_0_ffn_stream",
           "stream_weight_table", "stream_stages", "synth"]


def hbm_read_probe(buf: torch.Tensor, workgroups: int, unroll: int,
                   out: torch.Tensor | None = None) -> torch.Tensor:
    """Read every byte of buf (a contiguous device tensor, a multiple of 16
    bytes) once with 16-byte loads; returns the per-wave XOR words (uint32
    [4 * workgroups] as int32), the only thing written."""
    out = _out(out, (4 * workgroups,), torch.int32, buf.device, "out")
    _check("bq8_hbm_read_probe", lib().bq8_hbm_read_probe(
        _dev(buf, "buf"), buf.numel() * buf.element_size(), workgroups, unroll,
        _dev(out, "out", torch.int32), _stream()))
    return out
