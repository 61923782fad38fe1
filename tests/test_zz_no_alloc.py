"""GPU test of the allocation-free LM head (q6k_lmhead_top1_noalloc).

It runs through the C ABI with the library's own per-GPU scratch and must
return, bit for bit, the ids of q6k_lmhead_top1 with a caller's scratch on
the same inputs -- on two calls in a row, the second on a smaller input, and
then once more on the first input (each call overwrites what the previous
one left in the shared array).  A shape whose scratch exceeds the array is
refused before anything is enqueued, leaving the ids untouched.
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


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


def _case(seed, N, K, M):
    rng = np.random.default_rng(seed)
    raw = synth.q6k_raw_weights(rng, N, K)
    x = synth.normal_rows(rng, M, K)
    raw[N - 1] = raw[N // 3]           # equal rows: the lower id wins a tie
    return bq.q6k_pack_expand(dev(raw), N, K), dev(x)


def test_noalloc_head_equals_scratch_head():
    big = (70001, 5120, 6, 1, 5)       # split tiles, a ragged last tile
    small = (1000, 1280, 4, 1, 3)
    cases = {c: _case(9100 + c[0] % 997, *c[:3]) for c in (big, small)}
    for (N, K, M, row0, rows) in (big, small, big):
        pack, x = cases[(N, K, M, row0, rows)]
        say(f"q6k_lmhead_top1_noalloc N={N} K={K} rows {row0}..{row0 + rows - 1}")
        want = host(bq.q6k_lmhead_top1(pack, N, K, x, row0, rows))
        got = host(bq.q6k_lmhead_top1_noalloc(pack, N, K, x, row0, rows))
        assert np.array_equal(got, want), (got, want)


def test_noalloc_head_refuses_oversized_scratch():
    N, K = 64, 24576                   # 8 rows at this K need more than 256 KiB
    assert bq.q6k_lmhead_top1_scratch_bytes(N, K, 8) > 262144
    pack = torch.zeros((bq.q6k_pack_bytes(N, K),), dtype=torch.uint8, device=DEV)
    x = torch.zeros((8, K), dtype=torch.float32, device=DEV)
    ids = torch.full((8,), -7, dtype=torch.int32, device=DEV)
    with pytest.raises(bq.Bq8Error) as e:
        bq.q6k_lmhead_top1_noalloc(pack, N, K, x, 0, 8, ids=ids)
    assert e.value.status == 4
    assert (host(ids) == -7).all()
