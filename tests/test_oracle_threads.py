"""The oracle's loops over output rows give bitwise the same results on one
thread and on every host thread (each row's sum stays in one thread in its
fixed order), so its CPU timings on either count time the same computation."""
import numpy as np

import oracle
from block_quantized_gemv_q8_amd import synth


def test_one_thread_equals_all_threads():
    N, K, M = 700, 2048, 6
    w, x = synth.random_q4_0_case(77, N, K, M)
    xq = oracle.q8_1_quantize(x)
    full = oracle.num_threads()
    try:
        ref, bound = oracle.q4_0_gemv(w, N, K, xq, M)
        oracle.set_num_threads(1)
        assert oracle.num_threads() == 1
        one, bound1 = oracle.q4_0_gemv(w, N, K, xq, M)
    finally:
        oracle.set_num_threads(full)
    assert oracle.num_threads() == full
    assert np.array_equal(one.view(np.uint64), ref.view(np.uint64))
    assert np.array_equal(bound1.view(np.uint64), bound.view(np.uint64))
