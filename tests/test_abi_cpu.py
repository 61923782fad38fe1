"""The C-ABI library loads, exports every symbol the header declares, and
rejects bad arguments on the host before touching the device.  None of these
calls reaches the GPU: every case fails validation, which happens before any
HIP call, or is a host-only size query."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "bq8.h")

OK, NULL, SHAPE, ALIGN, SIZE, HIP = 0, 1, 2, 3, 4, 5


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*[a-z_0-9 ]+?\*?\s*\b([a-z_0-9]+)\s*\(", text, re.M)) -
                  {"if", "extern"})


@pytest.fixture(scope="module")
def L():
    import block_quantized_gemv_q8_amd as b

    return b.lib()


def test_header_declares_expected_entry_points():
    names = _declared_functions()
    for m in range(1, 18):
        assert f"q4_0_mmvq_m{m}" in names
    for n in ["q8_1_quantize", "q4_0_mmvq", "q6k_pack_bytes", "q6k_pack_expand",
              "q6k_lmhead_top1_scratch_bytes", "q6k_lmhead_top1", "bq8_status_string",
              "bq8_abi_version", "silu_mul_q8_1", "rms_norm_q8_1", "q4_0_ffn_stream_layout",
              "q4_0_ffn_stream", "q4_0_pack_bytes", "q4_0_pack", "q4_0_mmvq_packed",
              "q4_0_ffn_stream_packed", "q4_0_gate_up_silu_q8_1_packed",
              "q4_0_mmvq_packed_split", "q4_0_mmvq_packed_splits", "rms_norm_q8_1_sum",
              "q6k_lmhead_candidate_max", "q6k_compact_bytes", "q6k_pack_compact",
              "q6k_lmhead_top1_compact", "q6k_lmhead_candidate_max_compact",
              "bq8_hbm_read_probe", "q4_0_mmvq_packed_ws", "q4_0_mmvq_packed_ws_bytes",
              "q4_0_gate_up_silu_q8_1_packed_ws", "q6k_lmhead_top1_noalloc",
              "q4_0_mmvq_packed_splits_rows"]:
        assert n in names


def test_library_exports_every_declared_symbol(L):
    for name in _declared_functions():
        assert hasattr(L, name), name


def test_exports_nothing_else():
    import subprocess
    import block_quantized_gemv_q8_amd as b

    out = subprocess.run(["nm", "-D", "--defined-only", b.api.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = {ln.split()[-1] for ln in out.splitlines() if " T " in ln}
    assert exported == set(_declared_functions())


def test_version_and_status_strings(L):
    import block_quantized_gemv_q8_amd as b

    assert b.abi_version() == 1
    for s in range(6):
        assert len(b.status_string(s)) > 0
    assert b.status_string(99) == "unknown status"


def test_pack_bytes_and_scratch_queries(L):
    import block_quantized_gemv_q8_amd as b

    assert b.q6k_pack_bytes(248320, 5120) == 1360793600
    assert b.q6k_pack_bytes(1, 256) == 256 + 16 + 2
    assert b.q6k_pack_bytes(0, 256) == -1
    assert b.q6k_pack_bytes(4, 255) == -1
    assert b.q6k_pack_bytes(4, 384) == -1
    s = b.q6k_lmhead_top1_scratch_bytes(248320, 5120, 5)
    assert 0 < s < 1 << 20
    assert b.q6k_lmhead_top1_scratch_bytes(248320, 5120, 0) == -1
    assert b.q6k_lmhead_top1_scratch_bytes(248320, 5120, 9) == -1
    assert b.q6k_lmhead_top1_scratch_bytes(2 ** 31, 256, 1) == -1


# Fake, never-dereferenced device addresses: every call below must fail
# validation and return without any HIP call.
A = 0x10000  # 64 KiB aligned


def test_quantize_validation(L):
    assert L.q8_1_quantize(None, 1, 32, A, None) == NULL
    assert L.q8_1_quantize(A, 1, 32, None, None) == NULL
    assert L.q8_1_quantize(A, 0, 32, A, None) == SHAPE
    assert L.q8_1_quantize(A, 1, 48, A, None) == SHAPE
    assert L.q8_1_quantize(A, 1, 0, A, None) == SHAPE
    assert L.q8_1_quantize(A, 1 << 16, 1 << 15, A, None) == SHAPE
    assert L.q8_1_quantize(A + 2, 1, 32, A, None) == ALIGN
    assert L.q8_1_quantize(A, 1, 32, A + 1, None) == ALIGN


@pytest.mark.parametrize("m", [1, 6, 17])
def test_mmvq_validation(L, m):
    f = getattr(L, f"q4_0_mmvq_m{m}")
    assert f(None, 8, 64, A, A, None) == NULL
    assert f(A, 8, 64, None, A, None) == NULL
    assert f(A, 8, 64, A, None, None) == NULL
    assert f(A, 0, 64, A, A, None) == SHAPE
    assert f(A, 8, 48, A, A, None) == SHAPE
    assert f(A, 8, 0, A, A, None) == SHAPE
    assert f(A, 1 << 31, 64, A, A, None) == SHAPE
    assert f(A + 4, 8, 64, A, A, None) == ALIGN
    assert f(A, 8, 64, A + 2, A, None) == ALIGN
    assert f(A, 8, 64, A + 4, A, None) == ALIGN   # xq: 16-byte pieces go to LDS
    assert f(A, 8, 64, A, A + 2, None) == ALIGN


def test_mmvq_dispatch_rejects_bad_m(L):
    assert L.q4_0_mmvq(A, 8, 64, A, 0, A, None) == SHAPE
    assert L.q4_0_mmvq(A, 8, 64, A, 18, A, None) == SHAPE
    assert L.q4_0_mmvq(None, 8, 64, A, 6, A, None) == NULL


def test_expand_validation(L):
    n = 1360793600
    assert L.q6k_pack_expand(None, 248320, 5120, A, n, None) == NULL
    assert L.q6k_pack_expand(A, 248320, 5120, None, n, None) == NULL
    assert L.q6k_pack_expand(A, 248320, 5000, A, n, None) == SHAPE
    assert L.q6k_pack_expand(A, 0, 5120, A, n, None) == SHAPE
    assert L.q6k_pack_expand(A + 1, 248320, 5120, A, n, None) == ALIGN
    assert L.q6k_pack_expand(A, 248320, 5120, A + 8, n, None) == ALIGN
    assert L.q6k_pack_expand(A, 248320, 5120, A, n - 1, None) == SIZE
    assert L.q6k_pack_expand(A, 248320, 5120, A, n + 16, None) == SIZE


def test_top1_validation(L):
    s = L.q6k_lmhead_top1_scratch_bytes(248320, 5120, 5)
    args = dict(pack=A, N=248320, K=5120, x=A, M=6, row0=1, rows=5, ids=A, scratch=A, sb=s)

    def call(**kw):
        a = dict(args, **kw)
        return L.q6k_lmhead_top1(a["pack"], a["N"], a["K"], a["x"], a["M"], a["row0"], a["rows"],
                                 a["ids"], a["scratch"], a["sb"], None)

    assert call(pack=None) == NULL
    assert call(x=None) == NULL
    assert call(ids=None) == NULL
    assert call(scratch=None) == NULL
    assert call(K=5000) == SHAPE
    assert call(N=0) == SHAPE
    assert call(rows=0) == SHAPE
    assert call(rows=9, M=12) == SHAPE
    assert call(row0=2) == SHAPE          # rows 2..6 of 6
    assert call(row0=-1) == SHAPE
    assert call(pack=A + 4) == ALIGN
    assert call(x=A + 2) == ALIGN
    assert call(scratch=A + 8) == ALIGN
    assert call(sb=s - 1) == SIZE


NOALLOC_MAX = 262144   # BQ8_TOP1_NOALLOC_SCRATCH_BYTES


def test_top1_noalloc_validation(L):
    """The allocation-free head checks what q6k_lmhead_top1 checks, then that
    the shape's scratch fits its built-in array -- all before any HIP call."""
    args = dict(pack=A, N=248320, K=5120, x=A, M=6, row0=1, rows=5, ids=A)

    def call(**kw):
        a = dict(args, **kw)
        return L.q6k_lmhead_top1_noalloc(a["pack"], a["N"], a["K"], a["x"], a["M"], a["row0"],
                                         a["rows"], a["ids"], None)

    assert call(pack=None) == NULL
    assert call(x=None) == NULL
    assert call(ids=None) == NULL
    assert call(K=5000) == SHAPE
    assert call(rows=9, M=12) == SHAPE
    assert call(row0=2) == SHAPE
    assert call(pack=A + 4) == ALIGN
    assert call(x=A + 2) == ALIGN
    assert call(ids=A + 2) == ALIGN
    # the hot shape needs 72 KiB; K = 16384 fits at rows 8 and any N; eight
    # rows at K = 24576 need more than the array whatever N is
    assert L.q6k_lmhead_top1_scratch_bytes(248320, 5120, 5) <= NOALLOC_MAX
    assert L.q6k_lmhead_top1_scratch_bytes(2 ** 31 - 2, 16384, 8) <= NOALLOC_MAX
    assert L.q6k_lmhead_top1_scratch_bytes(1, 24576, 8) > NOALLOC_MAX
    assert call(K=24576, M=9, rows=8) == SIZE


def test_layer_glue_validation(L):
    assert L.silu_mul_q8_1(None, A, 6, 64, None, A, None) == NULL
    assert L.silu_mul_q8_1(A, A, 6, 48, None, A, None) == SHAPE
    assert L.silu_mul_q8_1(A, A, 6, 64, A + 2, A, None) == ALIGN
    assert L.rms_norm_q8_1(None, 6, 64, ctypes.c_float(1e-6), None, A, None) == NULL
    assert L.rms_norm_q8_1(A, 65, 64, ctypes.c_float(1e-6), None, A, None) == SHAPE
    assert L.rms_norm_q8_1(A, 6, 64, ctypes.c_float(0.0), None, A, None) == SHAPE
    assert L.rms_norm_q8_1(A, 1, 32768 + 32, ctypes.c_float(1e-6), None, A, None) == SHAPE
    assert L.rms_norm_q8_1(A, 6, 64, ctypes.c_float(1e-6), None, A + 1, None) == ALIGN


def test_stream_layout(L):
    import block_quantized_gemv_q8_amd as b

    lay = b.q4_0_ffn_stream_layout(6, 5120, 17408)
    assert lay["xq"] == 0
    assert lay["g"] >= 6 * 160 * 36 and lay["g"] % 256 == 0
    assert lay["u"] >= lay["g"] + 6 * 17408 * 4 and lay["u"] % 256 == 0
    assert lay["hq"] >= lay["u"] + 6 * 17408 * 4 and lay["hq"] % 256 == 0
    assert lay["total"] >= lay["hq"] + 6 * 544 * 36
    off = (ctypes.c_int64 * 5)()
    assert L.q4_0_ffn_stream_layout(0, 5120, 17408, off) == SHAPE
    assert L.q4_0_ffn_stream_layout(18, 5120, 17408, off) == SHAPE
    assert L.q4_0_ffn_stream_layout(6, 5000, 17408, off) == SHAPE
    assert L.q4_0_ffn_stream_layout(6, 5120, 17400, off) == SHAPE
    assert L.q4_0_ffn_stream_layout(6, 32768 + 32, 17408, off) == SHAPE
    assert L.q4_0_ffn_stream_layout(6, 32768, 17408, off) == OK
    assert L.q4_0_ffn_stream_layout(6, 5120, 17408, None) == NULL


def test_stream_validation(L):
    import block_quantized_gemv_q8_amd as b

    total = b.q4_0_ffn_stream_layout(6, 5120, 17408)["total"]
    layers = 3
    good = (ctypes.c_void_p * layers)(A, A + 0x100, A + 0x200)
    args = dict(g=good, u=good, d=good, layers=layers, M=6, hidden=5120, ffn=17408, x0=A,
                eps=1e-6, y=A, work=A, wb=total)

    def call(**kw):
        a = dict(args, **kw)
        return L.q4_0_ffn_stream(a["g"], a["u"], a["d"], a["layers"], a["M"], a["hidden"],
                                 a["ffn"], a["x0"], ctypes.c_float(a["eps"]), a["y"], a["work"],
                                 a["wb"], None)

    assert call(g=None) == NULL
    assert call(x0=None) == NULL
    assert call(work=None) == NULL
    assert call(u=(ctypes.c_void_p * layers)(A, None, A)) == NULL       # a null layer
    assert call(layers=0) == SHAPE
    assert call(M=18) == SHAPE
    assert call(hidden=5000) == SHAPE
    assert call(eps=0.0) == SHAPE
    assert call(d=(ctypes.c_void_p * layers)(A, A, A + 8)) == ALIGN    # last layer misaligned
    assert call(x0=A + 2) == ALIGN
    assert call(work=A + 16) == ALIGN
    assert call(wb=total - 1) == SIZE


def test_packed_q4_0_queries_and_validation(L):
    import block_quantized_gemv_q8_amd as b

    assert b.q4_0_pack_bytes(17408, 5120) == 50135040
    assert b.q4_0_pack_bytes(5120, 17408) == 50135040
    assert b.q4_0_pack_bytes(1, 512) == 16 * 18
    assert b.q4_0_pack_bytes(4, 256) == -1           # K % 512 != 0
    assert b.q4_0_pack_bytes(0, 512) == -1
    n = 17408 * 160 * 18
    assert L.q4_0_pack(None, 17408, 5120, A, n, None) == NULL
    assert L.q4_0_pack(A, 17408, 5120, None, n, None) == NULL
    assert L.q4_0_pack(A, 17408, 4096 + 256, A, n, None) == SHAPE
    assert L.q4_0_pack(A + 1, 17408, 5120, A, n, None) == ALIGN
    assert L.q4_0_pack(A, 17408, 5120, A + 8, n, None) == ALIGN
    assert L.q4_0_pack(A, 17408, 5120, A, n - 1, None) == SIZE
    assert L.q4_0_mmvq_packed(None, 17408, 5120, A, 6, A, None) == NULL
    assert L.q4_0_mmvq_packed(A, 17408, 5120, A, 0, A, None) == SHAPE
    assert L.q4_0_mmvq_packed(A, 17408, 5120, A, 18, A, None) == SHAPE
    assert L.q4_0_mmvq_packed(A, 17408, 5376, A, 6, A, None) == SHAPE  # K % 512 != 0
    assert L.q4_0_mmvq_packed(A + 8, 17408, 5120, A, 6, A, None) == ALIGN
    assert L.q4_0_mmvq_packed(A, 17408, 5120, A + 2, 6, A, None) == ALIGN
    assert L.q4_0_mmvq_packed(A, 17408, 5120, A + 4, 6, A, None) == ALIGN
    assert L.q4_0_mmvq_packed(A, 17408, 5120, A + 8, 6, A, None) == ALIGN
    # the balanced launch: the same checks first, then its workspace's
    ws = 1 << 20
    assert L.q4_0_mmvq_packed_ws(A, 17408, 5120, A, 6, A, None, ws, None) == NULL
    assert L.q4_0_mmvq_packed_ws(None, 17408, 5120, A, 6, A, A, ws, None) == NULL
    assert L.q4_0_mmvq_packed_ws(A, 17408, 5120, A, 18, A, A, ws, None) == SHAPE
    assert L.q4_0_mmvq_packed_ws(A, 17408, 5376, A, 6, A, A, ws, None) == SHAPE
    assert L.q4_0_mmvq_packed_ws(A + 8, 17408, 5120, A, 6, A, A, ws, None) == ALIGN
    assert L.q4_0_mmvq_packed_ws(A, 17408, 5120, A, 6, A, A + 128, ws, None) == ALIGN


def test_gate_up_silu_validation(L):
    f = L.q4_0_gate_up_silu_q8_1_packed

    def call(wg=A, wu=A, N=17408, K=5120, xq=A, M=6, g=None, u=None, h=None, hq=A):
        return f(wg, wu, N, K, xq, M, g, u, h, hq, None)

    assert call(wg=None) == NULL
    assert call(wu=None) == NULL
    assert call(xq=None) == NULL
    assert call(hq=None) == NULL
    assert call(M=0) == SHAPE
    assert call(M=18) == SHAPE
    assert call(N=17408 + 16) == SHAPE   # N % 32 != 0
    assert call(N=0) == SHAPE
    assert call(K=5376) == SHAPE         # K % 512 != 0
    assert call(M=17, K=2 ** 27) == SHAPE
    assert call(wg=A + 8) == ALIGN
    assert call(wu=A + 8) == ALIGN
    assert call(xq=A + 2) == ALIGN
    assert call(xq=A + 4) == ALIGN
    assert call(hq=A + 2) == ALIGN
    assert call(g=A + 2) == ALIGN
    assert call(u=A + 1) == ALIGN
    assert call(h=A + 3) == ALIGN
    # the balanced launch: its workspace is required and 256-byte aligned
    ws = 1 << 24
    J = L.q4_0_gate_up_silu_q8_1_packed_ws
    assert J(A, A, 17408, 5120, A, 6, None, None, None, A, None, ws, None) == NULL
    assert J(A, A, 17400, 5120, A, 6, None, None, None, A, A, ws, None) == SHAPE
    assert J(A, A, 17408, 5120, A, 6, None, None, None, A, A + 128, ws, None) == ALIGN


def test_split_product_and_summed_rms_validation(L):
    import block_quantized_gemv_q8_amd as b

    assert b.q4_0_mmvq_packed_splits(17408, 5120) == 1
    assert b.q4_0_mmvq_packed_splits(5120, 17408) == 4
    assert b.q4_0_mmvq_packed_splits(16, 512) == 2        # capped at the 2 chunks
    assert b.q4_0_mmvq_packed_splits(16, 4096) == 8       # capped at 8
    assert b.q4_0_mmvq_packed_splits(16, 256) == -1
    # the per-M count: the shape's count up to M = 10; from M = 11 it reads the
    # device's occupancy, so with no device it reports -1
    for m in range(1, 11):
        assert b.q4_0_mmvq_packed_splits_rows(5120, 17408, m) == 4
        assert b.q4_0_mmvq_packed_splits_rows(17408, 5120, m) == 1
    for m in range(11, 18):
        assert b.q4_0_mmvq_packed_splits_rows(5120, 17408, m) == -1
    for bad in ((5120, 17408, 0), (5120, 17408, 18), (16, 256, 6), (16, 256, 12)):
        assert b.q4_0_mmvq_packed_splits_rows(*bad) == -1
    f = L.q4_0_mmvq_packed_split
    assert f(None, 5120, 17408, A, 6, 4, A, None) == NULL
    assert f(A, 5120, 17408, A, 6, 0, A, None) == SHAPE
    assert f(A, 5120, 17408, A, 6, 9, A, None) == SHAPE
    assert f(A, 16, 512, A, 6, 3, A, None) == SHAPE        # more ranges than chunks
    assert f(A, 5120, 17408, A, 18, 4, A, None) == SHAPE
    assert f(A, 5120, 17408, A, 6, 4, A + 2, None) == ALIGN
    r = L.rms_norm_q8_1_sum
    assert r(None, 4, 6, 5120, 1e-6, A, None, A, None) == NULL
    assert r(A, 4, 6, 5120, 1e-6, None, None, None, None) == NULL   # nothing asked for
    assert r(A, 0, 6, 5120, 1e-6, None, None, A, None) == SHAPE
    assert r(A, 9, 6, 5120, 1e-6, None, None, A, None) == SHAPE
    assert r(A, 4, 65, 5120, 1e-6, None, None, A, None) == SHAPE
    assert r(A, 4, 6, 5120 + 16, 1e-6, None, None, A, None) == SHAPE
    assert r(A, 4, 6, 5120, 0.0, None, None, A, None) == SHAPE
    assert r(A + 2, 4, 6, 5120, 1e-6, None, None, A, None) == ALIGN
    assert r(A, 4, 6, 5120, 1e-6, A + 2, None, None, None) == ALIGN


def test_candidate_max_validation(L):
    import block_quantized_gemv_q8_amd as b

    N, K = 248320, 5120
    need = b.q6k_lmhead_top1_scratch_bytes(N, K, 5)
    f = L.q6k_lmhead_candidate_max

    def call(pack=A, x=A, M=6, row0=1, rows=5, cand=A, ncand=2, ids=A, vals=A, scores=A,
             scratch=A, nbytes=need):
        return f(pack, N, K, x, M, row0, rows, cand, ncand, ids, vals, scores, scratch, nbytes,
                 None)

    assert call(vals=None) == NULL
    assert call(cand=None) == NULL
    assert call(scores=None) == NULL
    assert call(ncand=9) == SHAPE
    assert call(ncand=-1) == SHAPE
    assert call(rows=9) == SHAPE
    assert call(row0=2) == SHAPE            # row0 + rows > M
    assert call(vals=A + 2) == ALIGN
    assert call(cand=A + 2) == ALIGN
    assert call(scores=A + 1) == ALIGN
    assert call(nbytes=need - 1) == SIZE


def test_compact_q6k_validation(L):
    import block_quantized_gemv_q8_amd as b

    assert b.q6k_compact_bytes(248320, 5120) == 1_042_944_000
    assert b.q6k_compact_bytes(1, 256) == 210
    assert b.q6k_compact_bytes(4, 384) == -1
    assert b.q6k_compact_bytes(0, 256) == -1
    n = b.q6k_compact_bytes(248320, 5120)
    assert L.q6k_pack_compact(None, 248320, 5120, A, n, None) == NULL
    assert L.q6k_pack_compact(A, 248320, 5120 + 128, A, n, None) == SHAPE
    assert L.q6k_pack_compact(A + 1, 248320, 5120, A, n, None) == ALIGN
    assert L.q6k_pack_compact(A, 248320, 5120, A + 8, n, None) == ALIGN
    assert L.q6k_pack_compact(A, 248320, 5120, A, n + 1, None) == SIZE
    need = b.q6k_lmhead_top1_scratch_bytes(248320, 5120, 5)
    t = L.q6k_lmhead_top1_compact
    assert t(None, 248320, 5120, A, 6, 1, 5, A, A, need, None) == NULL
    assert t(A, 248320, 5120, A, 6, 2, 5, A, A, need, None) == SHAPE
    assert t(A + 8, 248320, 5120, A, 6, 1, 5, A, A, need, None) == ALIGN
    assert t(A, 248320, 5120, A, 6, 1, 5, A, A, need - 1, None) == SIZE
    c = L.q6k_lmhead_candidate_max_compact
    assert c(A, 248320, 5120, A, 6, 1, 5, A, 2, A, None, A, A, need, None) == NULL
    assert c(A, 248320, 5120, A, 6, 1, 5, A, 9, A, A, A, A, need, None) == SHAPE


def test_hbm_read_probe_validation(L):
    P = 1 << 12                       # fake, aligned: never dereferenced
    f = L.bq8_hbm_read_probe
    assert f(None, 1024, 4, 4, P, None) == NULL
    assert f(P, 1024, 4, 4, None, None) == NULL
    assert f(P, 8, 4, 4, P, None) == SHAPE             # under 16 bytes
    assert f(P, 1032, 4, 4, P, None) == SHAPE          # not a multiple of 16
    assert f(P, 1024, 0, 4, P, None) == SHAPE          # no workgroup
    assert f(P, 1024, (1 << 20) + 1, 4, P, None) == SHAPE
    for u in (0, 3, 16):
        assert f(P, 1024, 4, u, P, None) == SHAPE
    assert f(P + 8, 1024, 4, 4, P, None) == ALIGN
    assert f(P, 1024, 4, 4, P + 2, None) == ALIGN
