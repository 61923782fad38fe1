"""The library's calls captured in a HIP graph (torch.cuda.CUDAGraph) give,
on every replay, exactly what the same calls give eagerly.

Each replay is separated from the next by eager library work on other
buffers and a synchronization, and every replay's outputs are compared bit
for bit with the eager results (the kernels are deterministic).  No call
enqueues a memset, so captured graphs hold kernel nodes only.
"""
import sys

import numpy as np
import pytest

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu
if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

import block_quantized_gemv_q8_amd as bq  # noqa: E402
from block_quantized_gemv_q8_amd import synth  # noqa: E402

DEV = "cuda:0"


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def _capture(fn):
    fn()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def test_graph_of_quantize_and_products():
    N, K, M = 2000, 1024, 6
    ws, xs = [], []
    for i in range(3):
        w, x = synth.random_q4_0_case(500 + i, N, K, M)
        ws.append(torch.from_numpy(w).to(DEV))
        xs.append(torch.from_numpy(x).to(DEV))
    wps = [bq.q4_0_pack(w) for w in ws]
    xq = torch.empty((M, K // 32 * 36), dtype=torch.uint8, device=DEV)
    ys = [torch.empty((M, N), dtype=torch.float32, device=DEV) for _ in range(6)]

    def steps():
        for i in range(3):
            bq.q8_1_quantize(xs[i], xq)
            bq.q4_0_mmvq_packed(wps[i], N, K, xq, M, ys[2 * i])
            bq.q4_0_mmvq_m6(ws[i], xq, ys[2 * i + 1])

    steps()
    torch.cuda.synchronize()
    ref = [y.clone() for y in ys]
    g = _capture(steps)
    other = torch.randn((M, K), device=DEV)
    for rep in range(3):
        say(f"graph replay {rep}")
        for y in ys:
            y.fill_(float("nan"))
        bq.q8_1_quantize(other)            # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for a, b in zip(ys, ref):
            assert torch.equal(a, b)


def test_graph_of_packed_stream_and_top1():
    M, H, F, L = 6, 512, 1024, 3
    wg = [bq.q4_0_pack(synth.q4_0_weights_device(960 + 3 * l, F, H)) for l in range(L)]
    wu = [bq.q4_0_pack(synth.q4_0_weights_device(961 + 3 * l, F, H)) for l in range(L)]
    wd = [bq.q4_0_pack(synth.q4_0_weights_device(962 + 3 * l, H, F)) for l in range(L)]
    x0 = torch.from_numpy(synth.stream_x0(M, H, seed=79)).to(DEV)
    y = torch.empty((M, H), dtype=torch.float32, device=DEV)
    work = torch.empty((bq.q4_0_ffn_stream_layout(M, H, F)["total"],), dtype=torch.uint8,
                       device=DEV)
    Nv, Kv = 3000, 1024
    raw = synth.q6k_raw_weights_device(97, Nv, Kv)
    pack = bq.q6k_pack_expand(raw, Nv, Kv)
    xv = torch.from_numpy(synth.normal_rows(np.random.default_rng(98), 6, Kv)).to(DEV)
    ids = torch.empty((5,), dtype=torch.int32, device=DEV)
    scratch = torch.empty((bq.q6k_lmhead_top1_scratch_bytes(Nv, Kv, 5),), dtype=torch.uint8,
                          device=DEV)
    # candidate-max on the compact pack, all six rows, two candidates each
    cpk = bq.q6k_pack_compact(raw, Nv, Kv)
    cand = torch.tensor([[r, 2999 - r] for r in range(6)], dtype=torch.int32, device=DEV)
    cids = torch.empty((6,), dtype=torch.int32, device=DEV)
    cvals = torch.empty((6,), dtype=torch.float32, device=DEV)
    cscores = torch.empty((6, 2), dtype=torch.float32, device=DEV)
    scratch6 = torch.empty((bq.q6k_lmhead_top1_scratch_bytes(Nv, Kv, 6),), dtype=torch.uint8,
                           device=DEV)

    def work_fn():
        bq.q4_0_ffn_stream(wg, wu, wd, x0, 1e-6, y=y, work=work, packed=True, ffn=F)
        bq.q6k_lmhead_top1(pack, Nv, Kv, xv, 1, 5, ids, scratch)
        bq.q6k_lmhead_candidate_max(cpk, Nv, Kv, xv, 0, 6, cand, scratch6, compact=True,
                                    ids=cids, vals=cvals, scores=cscores)

    outs = (y, ids, cids, cvals, cscores)
    work_fn()
    torch.cuda.synchronize()
    refs = [t.clone() for t in outs]
    g = _capture(work_fn)
    for rep in range(3):
        say(f"graph replay {rep}")
        for t in outs:
            t.fill_(-7)
        scratch.fill_(0xEE)                # the scratch's contents on entry must not matter
        scratch6.fill_(0xEE)
        bq.q8_1_quantize(torch.randn((4, 256), device=DEV))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for t, r in zip(outs, refs):
            assert torch.equal(t, r)


def test_graph_of_noalloc_head():
    """q6k_lmhead_top1_noalloc, the entry point for callers under capture,
    captured with two calls of different shapes: every replay gives the ids
    of the eager q6k_lmhead_top1, with eager calls of the same entry point
    (which share its per-GPU scratch) between replays."""
    shapes = [(4096 + 17, 1024, 5), (3000, 512, 3)]
    packs, xs, ids, refs = [], [], [], []
    for i, (Nv, Kv, rows) in enumerate(shapes):
        raw = synth.q6k_raw_weights_device(120 + i, Nv, Kv)
        packs.append(bq.q6k_pack_expand(raw, Nv, Kv))
        xs.append(torch.from_numpy(synth.normal_rows(np.random.default_rng(130 + i), 6,
                                                     Kv)).to(DEV))
        ids.append(torch.empty((rows,), dtype=torch.int32, device=DEV))
        refs.append(bq.q6k_lmhead_top1(packs[i], Nv, Kv, xs[i], 1, rows))

    def heads():
        for i, (Nv, Kv, rows) in enumerate(shapes):
            bq.q6k_lmhead_top1_noalloc(packs[i], Nv, Kv, xs[i], 1, rows, ids[i])

    heads()
    torch.cuda.synchronize()
    for a, r in zip(ids, refs):
        assert torch.equal(a, r)
    g = _capture(heads)
    other = torch.from_numpy(synth.normal_rows(np.random.default_rng(140), 6, 1024)).to(DEV)
    for rep in range(3):
        say(f"graph replay {rep}")
        for t in ids:
            t.fill_(-7)
        # eager use of the same per-GPU scratch between replays
        bq.q6k_lmhead_top1_noalloc(packs[0], shapes[0][0], 1024, other, 0, 6)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for a, r in zip(ids, refs):
            assert torch.equal(a, r)
