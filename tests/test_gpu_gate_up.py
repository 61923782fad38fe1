"""GPU parity of the joint gate/up kernel (q4_0_gate_up_silu_q8_1_packed).

Bars, per shape:
  * g and u within |gpu - oracle| <= 1e-5 * sum_b |t_b| + 1e-6 of the
    oracle's Q4_0 x Q8_1 products of the standard-layout weights;
  * h within 1e-5 relative (+1e-6) of the oracle's SiLU(g) * u of the GPU's
    own g and u;
  * hq bit for bit the oracle's Q8_1 of the GPU's own h (the quant decision is
    taken in binary32 on both sides);
  * h and hq bitwise equal to the standalone silu_mul_q8_1 of the same g, u,
    and hq independent of whether the optional outputs are requested.
Shapes span one to many 32-column workgroups, two to 160 chunks of 8 blocks
and every M class (1..8, 9..16, 17), up to the full ffn_up shape.
"""
import sys

import numpy as np
import pytest

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu
if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

import oracle  # noqa: E402
import block_quantized_gemv_q8_amd as bq  # noqa: E402
from block_quantized_gemv_q8_amd import synth  # noqa: E402

DEV = "cuda:0"
REL, ABS = 1e-5, 1e-6


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


def assert_close(gpu, ref, bound, what):
    err = np.abs(gpu.astype(np.float64) - ref)
    tol = REL * bound + ABS
    bad = err > tol
    assert not bad.any(), (f"{what}: {bad.sum()} of {bad.size} outside tolerance; first at "
                           f"{tuple(np.argwhere(bad)[0])}")


def run_case(wg, wu, x, N, K, M, ws=None):
    """Joint kernel with every optional output, checked stage by stage (the
    CU-balanced launch through workspace ws if given)."""
    xq = oracle.q8_1_quantize(x)
    pg, pu, xqd = bq.q4_0_pack(dev(wg)), bq.q4_0_pack(dev(wu)), dev(xq)
    g = torch.empty((M, N), dtype=torch.float32, device=DEV)
    u = torch.empty_like(g)
    h = torch.empty_like(g)
    hq = host(bq.q4_0_gate_up_silu_q8_1_packed(pg, pu, N, K, xqd, M, g=g, u=u, h=h, ws=ws))
    gg, ug, hg = host(g), host(u), host(h)

    ref_g, bound_g = oracle.q4_0_gemv(wg, N, K, xq, M)
    assert_close(gg, ref_g, bound_g, f"gate M{M} N{N} K{K}")
    ref_u, bound_u = oracle.q4_0_gemv(wu, N, K, xq, M)
    assert_close(ug, ref_u, bound_u, f"up M{M} N{N} K{K}")
    ref_h = oracle.silu_mul(gg, ug)
    err = np.abs(hg.astype(np.float64) - ref_h)
    assert (err <= REL * np.abs(ref_h) + ABS).all(), "h outside tolerance"
    assert (hq == oracle.q8_1_quantize(hg)).all(), "hq differs from Q8_1 of the GPU's h"

    # the epilogue is the standalone SiLU*up requant, bit for bit
    h2 = torch.empty_like(g)
    hq2 = host(bq.silu_mul_q8_1(g, u, h=h2))
    assert np.array_equal(host(h2).view(np.uint32), hg.view(np.uint32))
    assert (hq2 == hq).all()
    # no optional outputs: same hq
    hq3 = host(bq.q4_0_gate_up_silu_q8_1_packed(pg, pu, N, K, xqd, M, ws=ws))
    assert (hq3 == hq).all()
    return gg, ug, hg, hq


SHAPES = [(1, 64, 512), (8, 32, 512), (3, 96, 2048), (17, 1024, 1536), (16, 4096, 1024),
          (9, 544, 4608), (6, 64, 5120), (5, 2048, 5120)]


@pytest.mark.parametrize("M,N,K", SHAPES)
def test_gate_up_silu_small(M, N, K):
    say(f"gate_up_silu M={M} N={N} K={K}")
    wg, x = synth.random_q4_0_case(6100 + M + N + K, N, K, M)
    wu, _ = synth.random_q4_0_case(6200 + M + N + K, N, K, 1)
    run_case(wg, wu, x, N, K, M)


@pytest.mark.parametrize("M", [6, 1, 17])
def test_gate_up_silu_full_ffn_shape(M):
    N, K = synth.FFN_UP["N"], synth.FFN_UP["K"]
    say(f"gate_up_silu full ffn shape M={M}")
    wu, x = synth.ffn_up(M=max(M, 6))
    wg, _ = synth.random_q4_0_case(6300, N, K, 1)
    run_case(wg, wu, x[:M], N, K, M)


def test_gate_up_silu_zero_activation():
    M, N, K = 6, 256, 1024
    say("gate_up_silu zero activation")
    wg, _ = synth.random_q4_0_case(6400, N, K, 1)
    wu, _ = synth.random_q4_0_case(6401, N, K, 1)
    x = np.zeros((M, K), np.float32)
    x[2] = 1.0  # one live row among zero rows
    gg, ug, hg, hq = run_case(wg, wu, x, N, K, M)
    for m in (0, 1, 3, 4, 5):
        assert not gg[m].any() and not ug[m].any() and not hg[m].any()
        assert not hq[m].any()   # d = s = 0, every quant 0



# The CU-balanced launch (q4_0_gate_up_silu_q8_1_packed_ws): with at least
# as many 32-column groups as CUs, the groups past the last multiple of the
# CU count are cut into min(4, K/256) ranges of K that meet in the workspace
# (fewer groups: nothing is cut).  Every bar above holds for it; the
# uncut groups' g, u and hq are bitwise the plain launch's; results repeat
# bit for bit; the workspace's counters are back at zero after each call.
def _cus():
    return torch.cuda.get_device_properties(0).multi_processor_count


def _ws_shapes():
    c = _cus()
    return [(6, 64, 512), (17, 1024, 1536), (6, 32 * (c + 37), 2048), (9, 32 * (c + 5), 4608),
            (1, 32 * (2 * c + 3), 1024), (12, 32 * (c + 11), 1024), (4, 32 * (c + 7), 512),
            (14, 32 * (2 * c + 1), 512)]


@pytest.mark.parametrize("case", range(8))
def test_gate_up_silu_ws(case):
    M, N, K = _ws_shapes()[case]
    say(f"gate_up_silu_ws M={M} N={N} K={K}")
    wg, x = synth.random_q4_0_case(6500 + M + N + K, N, K, M)
    wu, _ = synth.random_q4_0_case(6600 + M + N + K, N, K, 1)
    _check_ws(wg, wu, x, N, K, M)


@pytest.mark.parametrize("M", [1, 3, 6, 9, 12, 16, 17])
def test_gate_up_silu_ws_full_ffn_shape(M):
    N, K = synth.FFN_UP["N"], synth.FFN_UP["K"]
    say(f"gate_up_silu_ws full ffn shape M={M}")
    wu, x = synth.ffn_up(M=max(M, 6))
    wg, _ = synth.random_q4_0_case(6700, N, K, 1)
    _check_ws(wg, wu, x[:M], N, K, M)


def _check_ws(wg, wu, x, N, K, M):
    ws = bq.q4_0_mmvq_packed_workspace()
    count_bytes = (_cus() * 4 + 255) // 256 * 256
    gg, ug, hg, hq = run_case(wg, wu, x, N, K, M, ws=ws)
    assert not host(ws[:count_bytes]).any()
    groups = N // 32
    whole = groups - groups % _cus() if groups >= _cus() else groups
    pg, pu = bq.q4_0_pack(dev(wg)), bq.q4_0_pack(dev(wu))
    xqd = dev(oracle.q8_1_quantize(x))
    g = torch.empty((M, N), dtype=torch.float32, device=DEV)
    u = torch.empty_like(g)
    hq_p = host(bq.q4_0_gate_up_silu_q8_1_packed(pg, pu, N, K, xqd, M, g=g, u=u))
    c = 32 * whole
    assert np.array_equal(gg[:, :c].view(np.uint32), host(g)[:, :c].view(np.uint32))
    assert np.array_equal(ug[:, :c].view(np.uint32), host(u)[:, :c].view(np.uint32))
    assert (hq.reshape(M, groups, 36)[:, :whole] == hq_p.reshape(M, groups, 36)[:, :whole]).all()
    again = host(bq.q4_0_gate_up_silu_q8_1_packed(pg, pu, N, K, xqd, M, ws=ws))
    assert (again == hq).all()
    assert not host(ws[:count_bytes]).any()
