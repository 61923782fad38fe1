"""bench.py times the step through raw calls of the two C entry points
(raw_step); they must compute exactly what the binding's step computes, on
the full ffn_up workload the bench times: the same Q8_1 rows and the same
outputs, bit for bit, for steps on different weight copies."""
import os
import sys

import pytest

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu
if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
import block_quantized_gemv_q8_amd as bq  # noqa: E402
from block_quantized_gemv_q8_amd import synth  # noqa: E402


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def test_raw_step_equals_the_binding_step():
    say("bench step: raw calls against the binding, ffn_up [17408 x 5120], M = 6")
    s = bench.setup_ffn_up(torch, bq, synth)
    raw = bench.raw_step(torch, bq, s)
    for i in (0, 5, 11):
        s["xq"].fill_(0x5A)
        s["y"].fill_(float("nan"))
        bench.step_packed(bq, s, i)
        torch.cuda.synchronize()
        xq_b, y_b = s["xq"].clone(), s["y"].clone()
        s["xq"].fill_(0xA5)
        s["y"].fill_(float("nan"))
        raw(i)
        torch.cuda.synchronize()
        assert torch.equal(s["xq"], xq_b), f"step {i}: Q8_1 rows differ"
        assert torch.equal(s["y"].view(torch.int32), y_b.view(torch.int32)), \
            f"step {i}: outputs differ"
        assert not torch.isnan(y_b).any()
