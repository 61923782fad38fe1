"""Benchmark of the width-6 verifier projection on one MI355X.

    python bench.py [--gpus 1] [--steps 2000] [--warmup 2000]

A step is one verifier projection of the ffn_up workload: Q8_1 quantization
of the six f32 activation rows [6][5120] followed by the Q4_0 x Q8_1
product against an [17408][5120] Q4_0 weight held in the library's
offline-packed layout (q8_1_quantize + q4_0_mmvq_packed, M = 6).  The
packing -- the same 18 bytes per 32 weights, regrouped once at load time,
as the pages' verifier did with its offline-packed width-6 projections --
is not timed, like the Q6_K expansion of the LM head.  Twelve copies of the
weight (601 MB, more than twice the 256 MB last-level cache) are used
round-robin so every step streams its weight from HBM; inputs are resident
in device memory before timing starts.  The K timed steps' library calls
are issued behind an untimed backlog of steps, so the timed region holds
the K steps back to back.  The same K steps from an idle GPU, as one
replayed HIP graph and issued through the binding, are reported beside it.

Printed: one JSON line with the effective weight bandwidth of a step
(value, GB/s), the product kernel's roofline against the 8 TB/s HBM peak,
the same projection on the weight's plain GGUF block layout
(q4_0_mmvq_m6), the joint gate/up + SiLU*up + Q8_1 launch against the same
three steps as separate launches (ffn_up shape, M = 6), the fused Q6_K
LM-head top-1 time on the lm_head workload (lmhead_top1_us: the faster of
the compact and the expanded pack, which give bitwise the same ids; both are
reported, with the six-row and candidate-max variants),
the per-M times of the down_sweep workload on both layouts, ms per full
width-6 pass of the 64-layer verifier FFN stream (both layouts), and the
oracle's CPU throughput on a bounded sample.

Profiling helpers (one kernel family per process, for rocprofv3):
    python bench.py --profile-target \\
        packed_m6|packed_m6_graph|mmvq_m6|gate_up|lmhead_top1|lmhead_compact|down_sweep|stream|stream_packed|copy|probe
        [--reps R]
    python bench.py --profile-target packed_one --shape ffn_up|down --m M \\
        --launch whole|ws|split [--reps R]
"""
from __future__ import annotations

import argparse
import gc
import hashlib
import json
import os
import subprocess
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
ROTATE = 12
WARMUP_MIN_S = 0.3  # untimed steps before the timed region, at least this long
STEP_BACKLOG = 200  # untimed steps queued ahead of the timed ones
PMC_RECORD = os.path.join(ROOT, "profiles", "pmc_q4_0_mmvq_packed_m6_ffn_up.json")
PMC_RECORD_GATE_UP = os.path.join(ROOT, "profiles", "pmc_q4_0_gate_up_silu_q8_1_packed_m6_ffn.json")
KERNEL_SOURCES = ["block_quantized_gemv_q8_amd/csrc/q4_0_packed.hip",
                  "block_quantized_gemv_q8_amd/csrc/bq8_dev.h",
                  "block_quantized_gemv_q8_amd/csrc/bq8_host.h"]

METRIC = "µs + effective weight GB/s (% of HBM peak) per Q4_0 M=6 proj; LM-head top-1 µs"


def q4_0_bytes(N, K):
    return N * (K // 32) * 18


def kernel_source_hash():
    """Hash of the kernel sources' code: comments dropped and whitespace
    collapsed, so that a counter record stays valid across comment edits and
    lapses with any change to the code itself."""
    import re

    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel)) as f:
            text = f.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()[:16]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


class Timer:
    """HIP events on torch's current stream (the stream every launch uses)."""

    def __init__(self, torch):
        self.torch = torch
        self.a = torch.cuda.Event(enable_timing=True)
        self.b = torch.cuda.Event(enable_timing=True)

    def __enter__(self):
        self.torch.cuda.synchronize()
        self.a.record()
        return self

    def __exit__(self, *exc):
        self.b.record()
        self.torch.cuda.synchronize()
        self.ms = self.a.elapsed_time(self.b)


def time_calls(torch, fn, reps, warm=10):
    """µs per call of fn(i), i = call index, after `warm` untimed calls."""
    for i in range(warm):
        fn(i)
    with Timer(torch) as t:
        for i in range(reps):
            fn(i)
    return t.ms * 1000.0 / reps


def time_batches(torch, fn, per_batch, batches=10, warm=10):
    """µs per call of fn(i) over `batches` batches of per_batch back-to-back
    calls, each batch bracketed by its own HIP events (call indices run on
    across batches, so rotating weights keep rotating): median, p10 and p90
    of the batch means."""
    for i in range(warm):
        fn(i)
    us = []
    k = 0
    for _ in range(batches):
        with Timer(torch) as t:
            for _ in range(per_batch):
                fn(k)
                k += 1
        us.append(t.ms * 1000.0 / per_batch)
    return {"median": float(np.median(us)), "p10": float(np.percentile(us, 10)),
            "p90": float(np.percentile(us, 90)), "batches": batches, "calls_per_batch": per_batch}


def stats_us(st, nd=3):
    return {"us_median": round(st["median"], nd), "us_p10": round(st["p10"], nd),
            "us_p90": round(st["p90"], nd)}


def hbm_probe(torch, bq, bufs, per_batch, batches=5):
    """The read-only probe over the same buffers a kernel streams (rotating
    through them like the kernel's calls): the fastest of a small sweep of
    launch shapes, as µs per buffer read."""
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    nbytes = bufs[0].numel() * bufs[0].element_size()
    best = None
    for per_cu in (4, 8, 16):
        wgs = cus * per_cu
        out = torch.empty((4 * wgs,), dtype=torch.int32, device="cuda")
        for unroll in (2, 4, 8):
            st = time_batches(torch, lambda i: bq.hbm_read_probe(bufs[i % len(bufs)], wgs, unroll,
                                                                 out), per_batch, batches)
            if best is None or st["median"] < best[0]["median"]:
                best = (st, {"workgroups": wgs, "threads_per_workgroup": 256, "unroll": unroll})
    st, shape = best
    return {"bytes_per_read": nbytes, **stats_us(st),
            "GBps": round(nbytes / st["median"] / 1e3, 1),
            "pct_hbm_peak": round(100 * nbytes / st["median"] / 1e3 / HBM_PEAK_GBS, 2),
            "launch": shape, "buffers_rotated": len(bufs)}


def capture(torch, fn, n):
    """A HIP graph of the calls fn(0) .. fn(n-1), captured on torch's capture
    stream (every library call enqueues on torch's current stream).  fn(0)
    runs once eagerly first, so one-time set-up stays outside the graph."""
    fn(0)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(n):
            fn(i)
    torch.cuda.synchronize()
    return g


def setup_ffn_up(torch, bq, synth):
    cfg = synth.FFN_UP
    N, K, M = cfg["N"], cfg["K"], cfg["M"]
    w, x = synth.ffn_up()
    w0 = torch.from_numpy(w).to("cuda")
    ws = [w0] + [w0.clone() for _ in range(ROTATE - 1)]
    wps = [bq.q4_0_pack(wi) for wi in ws]
    xd = torch.from_numpy(x).to("cuda")
    xq = torch.empty((M, K // 32 * 36), dtype=torch.uint8, device="cuda")
    y = torch.empty((M, N), dtype=torch.float32, device="cuda")
    u = torch.empty((M, N), dtype=torch.float32, device="cuda")
    hq = torch.empty((M, N // 32 * 36), dtype=torch.uint8, device="cuda")
    # the product's workspace: the CU-balanced launch (q4_0_mmvq_packed_ws)
    pws = bq.q4_0_mmvq_packed_workspace()
    return dict(N=N, K=K, M=M, ws=ws, wps=wps, pws=pws, x=xd, xq=xq, y=y, u=u, hq=hq)


def raw_step(torch, bq, s):
    """step_packed as direct calls of the two C entry points the binding
    wraps (q8_1_quantize, q4_0_mmvq_packed_ws), with the same arguments as
    raw pointers taken once; a nonzero status raises."""
    L = bq.lib()
    st = torch.cuda.current_stream().cuda_stream
    xp, xqp, yp = s["x"].data_ptr(), s["xq"].data_ptr(), s["y"].data_ptr()
    wps = [w.data_ptr() for w in s["wps"]]
    wsp, wsn = s["pws"].data_ptr(), s["pws"].numel()
    N, K, M = s["N"], s["K"], s["M"]

    def step(i):
        if (L.q8_1_quantize(xp, M, K, xqp, st) != 0 or
                L.q4_0_mmvq_packed_ws(wps[i % ROTATE], N, K, xqp, M, yp, wsp, wsn, st) != 0):
            raise RuntimeError("step launch failed")
    return step


def step_packed(bq, s, i):
    bq.q8_1_quantize(s["x"], s["xq"])
    bq.q4_0_mmvq_packed(s["wps"][i % ROTATE], s["N"], s["K"], s["xq"], s["M"], s["y"],
                        ws=s["pws"])


def step_standard(bq, s, i):
    bq.q8_1_quantize(s["x"], s["xq"])
    bq.q4_0_mmvq_m6(s["ws"][i % ROTATE], s["xq"], s["y"])


def gate_up_joint(bq, s, i):
    """Joint gate/up + SiLU*up + Q8_1 on the ffn_up shape: gate is packed copy
    i, up copy i + 6 (two different 50 MB weights per launch)."""
    bq.q4_0_gate_up_silu_q8_1_packed(s["wps"][i % ROTATE], s["wps"][(i + 6) % ROTATE], s["N"],
                                     s["K"], s["xq"], s["M"], s["hq"], ws=s["pws"])


def gate_up_separate(bq, s, i):
    bq.q4_0_mmvq_packed(s["wps"][i % ROTATE], s["N"], s["K"], s["xq"], s["M"], s["y"],
                        ws=s["pws"])
    bq.q4_0_mmvq_packed(s["wps"][(i + 6) % ROTATE], s["N"], s["K"], s["xq"], s["M"], s["u"],
                        ws=s["pws"])
    bq.silu_mul_q8_1(s["y"], s["u"], s["hq"])


def gate_up_separate_gguf(bq, s, i):
    bq.q4_0_mmvq_m6(s["ws"][i % ROTATE], s["xq"], s["y"])
    bq.q4_0_mmvq_m6(s["ws"][(i + 6) % ROTATE], s["xq"], s["u"])
    bq.silu_mul_q8_1(s["y"], s["u"], s["hq"])


def setup_lm_head(torch, bq, synth):
    cfg = synth.LM_HEAD
    N, K = cfg["N"], cfg["K"]
    raw = synth.q6k_raw_weights_device(cfg["seed"], N, K)
    pack = bq.q6k_pack_expand(raw, N, K)
    rng = np.random.default_rng(cfg["seed"])
    x = torch.from_numpy(synth.normal_rows(rng, cfg["M"], K)).to("cuda")
    ids = torch.empty((cfg["rows"],), dtype=torch.int32, device="cuda")
    scratch = torch.empty((bq.q6k_lmhead_top1_scratch_bytes(N, K, cfg["rows"]),),
                          dtype=torch.uint8, device="cuda")
    return dict(N=N, K=K, raw=raw, pack=pack, x=x, ids=ids, scratch=scratch, row0=cfg["row0"],
                rows=cfg["rows"])


def lm_head_call(bq, s):
    bq.q6k_lmhead_top1(s["pack"], s["N"], s["K"], s["x"], s["row0"], s["rows"], s["ids"],
                       s["scratch"])


def time_down_sweep(torch, bq, synth, reps):
    cfg = synth.DOWN_SWEEP
    N, K = cfg["N"], cfg["K"]
    w, x = synth.down_sweep()
    w0 = torch.from_numpy(w).to("cuda")
    ws = [w0] + [w0.clone() for _ in range(ROTATE - 1)]
    wps = [bq.q4_0_pack(wi) for wi in ws]
    xq = bq.q8_1_quantize(torch.from_numpy(x).to("cuda"))
    wb = q4_0_bytes(N, K)
    pw = bq.q4_0_mmvq_packed_workspace()
    out = {"packed_split_ranges": {m: bq.q4_0_mmvq_packed_splits_rows(N, K, m) for m in cfg["Ms"]},
           "packed_launch": "q4_0_mmvq_packed_ws"}
    for m in cfg["Ms"]:
        f = getattr(bq, f"q4_0_mmvq_m{m}")
        xm = xq[:m]
        P = out["packed_split_ranges"][m]
        y = torch.empty((m, N), dtype=torch.float32, device="cuda")
        yp = torch.empty((P, m, N), dtype=torch.float32, device="cuda")
        usp = time_batches(torch, lambda i: bq.q4_0_mmvq_packed(wps[i % ROTATE], N, K, xm, m, y,
                                                                ws=pw), reps // 5, 5)["median"]
        # every tile whole (the launch without a workspace)
        usw = time_batches(torch, lambda i: bq.q4_0_mmvq_packed(wps[i % ROTATE], N, K, xm, m, y),
                           reps // 5, 5)["median"]
        uss = time_batches(torch, lambda i: bq.q4_0_mmvq_packed_split(
            wps[i % ROTATE], N, K, xm, m, P, yp), reps // 5, 5)["median"]
        us = time_batches(torch, lambda i: f(ws[i % ROTATE], xm, y), reps // 5, 5)["median"]
        out[str(m)] = {"packed_us": round(usp, 3), "packed_GBps": round(wb / usp / 1e3, 1),
                       "packed_whole_tiles_us": round(usw, 3),
                       "packed_split_us": round(uss, 3),
                       "packed_split_GBps": round(wb / uss / 1e3, 1),
                       "gguf_us": round(us, 3), "gguf_GBps": round(wb / us / 1e3, 1)}
    return out


def time_stream(torch, bq, synth, passes, packed):
    """ms per full width-6 pass of the 64-layer verifier FFN stream (weights
    generated on the device, 9.6 GB, far beyond the caches); median, p10 and
    p90 over `passes` passes, each bracketed by its own HIP events."""
    cfg = synth.STREAM
    L, M, H, F = cfg["layers"], cfg["M"], cfg["hidden"], cfg["ffn"]
    wg, wu, wd = synth.stream_weights_device(L, H, F)
    if packed:
        for ws in (wg, wu, wd):
            for i in range(L):
                ws[i] = bq.q4_0_pack(ws[i])
    tables = tuple(bq.stream_weight_table(ws) for ws in (wg, wu, wd))
    x0 = torch.from_numpy(synth.stream_x0()).to("cuda")
    kw = dict(tables=tables, packed=packed, ffn=F)
    y, work = bq.q4_0_ffn_stream(wg, wu, wd, x0, 1e-6, **kw)
    for _ in range(2):
        bq.q4_0_ffn_stream(wg, wu, wd, x0, 1e-6, y=y, work=work, **kw)
    ms = []
    for _ in range(passes):
        with Timer(torch) as t:
            bq.q4_0_ffn_stream(wg, wu, wd, x0, 1e-6, y=y, work=work, **kw)
        ms.append(t.ms)
    # the same pass captured once as a HIP graph and replayed
    g = capture(torch, lambda i: bq.q4_0_ffn_stream(wg, wu, wd, x0, 1e-6, y=y, work=work, **kw), 1)
    gms = []
    for _ in range(passes):
        with Timer(torch) as t:
            g.replay()
        gms.append(t.ms)
    wbytes = L * (2 * q4_0_bytes(F, H) + q4_0_bytes(H, F))
    med = float(np.median(ms))
    gmed = float(np.median(gms))
    return {"layers": L, "M": M, "hidden": H, "ffn": F, "passes": passes,
            "layout": "packed" if packed else "gguf",
            "ms_median": round(med, 4), "ms_p10": round(float(np.percentile(ms, 10)), 4),
            "ms_p90": round(float(np.percentile(ms, 90)), 4), "weight_bytes": wbytes,
            "GBps": round(wbytes / med / 1e6, 1), "launches_per_pass": (3 if packed else 5) * L,
            "graph_ms_median": round(gmed, 4),
            "graph_ms_p10": round(float(np.percentile(gms, 10)), 4),
            "graph_ms_p90": round(float(np.percentile(gms, 90)), 4),
            "graph_GBps": round(wbytes / gmed / 1e6, 1)}


SHARDS = 8
ROTATE_BYTES = 600_000_000  # weight bytes in rotation: over twice the 256 MB last-level cache


def time_shards(torch, bq, synth, per_batch=100):
    """One GPU's share of the path under 8-way sharding, at its real shape:
    the gate/up column shard (N = 17408/8 = 2176 of K = 5120: a plain packed
    product and the joint gate/up launch), the down row shard (K = 17408/8 =
    2176 of N = 5120, on the GGUF block layout: 2176 is not a multiple of
    512, the packed layout's K granule) and the LM head's vocabulary shard
    (248320/8 = 31040 rows, rows 1..5 projected, both packs).  Enough weight
    copies rotate that every call reads its weight from HBM."""
    M = 6
    rng = np.random.default_rng(synth.FFN_UP["seed"])
    K = synth.FFN_UP["K"]
    Ns = synth.FFN_UP["N"] // SHARDS
    sb = q4_0_bytes(Ns, K)
    n = -(-ROTATE_BYTES // sb)
    wps = [bq.q4_0_pack(synth.q4_0_weights_device(1000 + i, Ns, K)) for i in range(n)]
    xq = bq.q8_1_quantize(torch.from_numpy(synth.normal_rows(rng, M, K)).to("cuda"))
    y = torch.empty((M, Ns), dtype=torch.float32, device="cuda")
    hq = torch.empty((M, Ns // 32 * 36), dtype=torch.uint8, device="cuda")
    pw = bq.q4_0_mmvq_packed_workspace()
    prod = time_batches(torch, lambda i: bq.q4_0_mmvq_packed(wps[i % n], Ns, K, xq, M, y, ws=pw),
                        per_batch)
    joint = time_batches(torch, lambda i: bq.q4_0_gate_up_silu_q8_1_packed(
        wps[i % n], wps[(i + n // 2) % n], Ns, K, xq, M, hq, ws=pw), per_batch)
    del wps
    Nd, Kd = synth.DOWN_SWEEP["N"], synth.DOWN_SWEEP["K"] // SHARDS
    db = q4_0_bytes(Nd, Kd)
    nd = -(-ROTATE_BYTES // db)
    wd = [synth.q4_0_weights_device(2000 + i, Nd, Kd) for i in range(nd)]
    xqd = bq.q8_1_quantize(torch.from_numpy(synth.normal_rows(rng, M, Kd, 0.5)).to("cuda"))
    yd = torch.empty((M, Nd), dtype=torch.float32, device="cuda")
    down = time_batches(torch, lambda i: bq.q4_0_mmvq_m6(wd[i % nd], xqd, yd), per_batch)
    del wd
    Nv = synth.LM_HEAD["N"] // SHARDS
    raws = [synth.q6k_raw_weights_device(3000 + i, Nv, K) for i in range(5)]
    cpks = [bq.q6k_pack_compact(r, Nv, K) for r in raws]
    packs = [bq.q6k_pack_expand(r, Nv, K) for r in raws]
    del raws
    x6 = torch.from_numpy(synth.normal_rows(rng, M, K)).to("cuda")
    ids = torch.empty((5,), dtype=torch.int32, device="cuda")
    scratch = torch.empty((bq.q6k_lmhead_top1_scratch_bytes(Nv, K, 5),), dtype=torch.uint8,
                          device="cuda")
    lmc = time_batches(torch, lambda i: bq.q6k_lmhead_top1(cpks[i % 5], Nv, K, x6, 1, 5, ids,
                                                           scratch, compact=True), 20)
    lme = time_batches(torch, lambda i: bq.q6k_lmhead_top1(packs[i % 5], Nv, K, x6, 1, 5, ids,
                                                           scratch), 20)
    cb, eb = cpks[0].numel(), packs[0].numel()
    del cpks, packs

    def line(st, nbytes, **kw):
        return {**kw, "weight_bytes": nbytes, **stats_us(st),
                "GBps": round(nbytes / st["median"] / 1e3, 1)}

    return {"ways": SHARDS,
            "gate_up_column_shard": {
                "packed_product": line(prod, sb, N=Ns, K=K, M=M),
                "joint_gate_up_silu_q8_1": line(joint, 2 * sb, N=Ns, K=K, M=M),
                "copies_rotated": n},
            "down_row_shard": {**line(down, db, N=Nd, K=Kd, M=M, layout="gguf (q4_0_mmvq_m6)"),
                               "copies_rotated": nd},
            "lm_head_vocab_shard": {
                "N": Nv, "K": K, "rows": "1..5",
                "compact": line(lmc, cb), "expanded": line(lme, eb), "copies_rotated": 5}}


def cpu_baseline(synth, budget_s=10.0):
    """The oracle, as written, on the full ffn_up workload, repeated for
    about budget_s seconds of wall time on the host's cores."""
    import oracle

    cfg = synth.FFN_UP
    N, K, M = cfg["N"], cfg["K"], cfg["M"]
    w, x = synth.ffn_up()
    oracle.lib()
    n = 0
    t0 = time.perf_counter()
    while True:
        xq = oracle.q8_1_quantize(x)
        oracle.q4_0_gemv(w, N, K, xq, M)
        n += 1
        el = time.perf_counter() - t0
        if el >= budget_s and n >= 3:
            break
    return {"value": round(n * q4_0_bytes(N, K) / el / 1e9, 4), "unit": "GB/s",
            "cores": oracle.num_threads(), "kind": "oracle",
            "sample": f"{n} full ffn_up projections (Q8_1 quantize of [6][5120] + Q4_0 GEMV "
                      f"[17408x5120], M=6) in {el:.1f} s"}


def cpu_one_thread(synth, budget_s=5.0):
    """The same oracle sample on one host thread (the oracle's results do not
    depend on its thread count)."""
    import oracle

    cfg = synth.FFN_UP
    N, K, M = cfg["N"], cfg["K"], cfg["M"]
    w, x = synth.ffn_up()
    full = oracle.num_threads()
    oracle.set_num_threads(1)
    try:
        n = 0
        t0 = time.perf_counter()
        while True:
            xq = oracle.q8_1_quantize(x)
            oracle.q4_0_gemv(w, N, K, xq, M)
            n += 1
            el = time.perf_counter() - t0
            if el >= budget_s and n >= 2:
                break
    finally:
        oracle.set_num_threads(full)
    return {"GBps": round(n * q4_0_bytes(N, K) / el / 1e9, 4), "threads": 1,
            "ms_per_projection": round(1000 * el / n, 1), "projections": n}


def host_info():
    """The host the oracle is timed on: CPU model and logical CPUs."""
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"cpu_model": model, "logical_cpus": os.cpu_count()}


def clocks_under_load(torch, fn, max_s=10.0):
    """The clocks rocm-smi reports while fn(i) runs back to back, untimed: the
    child process starts first and batches of 200 calls are issued until it
    exits.  None where rocm-smi is missing or fails."""
    try:
        p = subprocess.Popen(["rocm-smi", "--showclocks", "--json"], stdout=subprocess.PIPE,
                             stderr=subprocess.DEVNULL, text=True)
    except OSError:
        return None
    t0 = time.perf_counter()
    i = 0
    while p.poll() is None and time.perf_counter() - t0 < max_s:
        for _ in range(200):
            fn(i)
            i += 1
        torch.cuda.synchronize()
    try:
        out, _ = p.communicate(timeout=30)
        card = next(iter(json.loads(out).values()))
        return {k.strip(" :"): v for k, v in card.items()
                if "clk" in k.lower() or "clock" in k.lower()}
    except Exception:
        p.kill()
        return None


def rocm_version():
    """The ROCm release installed at /opt/rocm, or None."""
    try:
        with open("/opt/rocm/.info/version") as f:
            return f.read().strip()
    except OSError:
        return None


def device_info(torch, clocks=None):
    p = torch.cuda.get_device_properties(0)
    return {"name": p.name, "arch": getattr(p, "gcnArchName", None), "rocm": rocm_version(),
            "compute_units": p.multi_processor_count,
            "memory_GiB": round(p.total_memory / 2**30, 1), "torch": torch.__version__,
            "hip": getattr(torch.version, "hip", None), "numpy": np.__version__,
            "clocks_under_load": clocks}


def pmc_traffic(record=PMC_RECORD):
    """HBM bytes per launch from a committed rocprofv3 counter record, if it
    was taken on the current kernel source; else None."""
    try:
        with open(record) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("kernel_source_hash") != kernel_source_hash():
        return None
    return rec.get("hbm_bytes_per_launch")


def profile_target(torch, bq, synth, target, reps, args=None):
    if target == "copy":
        n = 1 << 30
        a = torch.empty(n, dtype=torch.uint8, device="cuda")
        b = torch.empty(n, dtype=torch.uint8, device="cuda")
        a.fill_(1)
        torch.cuda.synchronize()
        for _ in range(reps):
            b.copy_(a)
        torch.cuda.synchronize()
        log(f"copy: {reps} x {n} bytes")
        return
    if target == "probe":
        # the read probe at the launch shape bench.py finds fastest over the 12
        # packed ffn_up copies: 8 workgroups per CU, 8 loads in flight per thread
        s = setup_ffn_up(torch, bq, synth)
        wgs = 8 * torch.cuda.get_device_properties(0).multi_processor_count
        out = torch.empty((4 * wgs,), dtype=torch.int32, device="cuda")
        for i in range(reps):
            bq.hbm_read_probe(s["wps"][i % ROTATE], wgs, 8, out)
        torch.cuda.synchronize()
        log(f"probe: {reps} reads of {s['wps'][0].numel()} bytes")
        return
    if target == "packed_m6_graph":
        # the roofline kernel as bench.py times it, back to back: one HIP
        # graph of 100 launches rotating the 12 weight copies, replayed reps
        # times, so that a kernel trace sees the launches without the host's
        # per-launch gaps
        s = setup_ffn_up(torch, bq, synth)
        N, K, M = s["N"], s["K"], s["M"]
        bq.q8_1_quantize(s["x"], s["xq"])
        g = capture(torch, lambda i: bq.q4_0_mmvq_packed(
            s["wps"][i % ROTATE], N, K, s["xq"], M, s["y"], ws=s["pws"]), 100)
        for _ in range(reps):
            g.replay()
        torch.cuda.synchronize()
        log(f"packed_m6_graph: {reps} replays of 100 launches")
        return
    if target in ("packed_m6", "mmvq_m6", "gate_up"):
        s = setup_ffn_up(torch, bq, synth)
        step = {"packed_m6": step_packed, "mmvq_m6": step_standard,
                "gate_up": gate_up_joint}[target]
        bq.q8_1_quantize(s["x"], s["xq"])
        for i in range(reps):
            step(bq, s, i)
    elif target == "lmhead_top1":
        s = setup_lm_head(torch, bq, synth)
        for _ in range(reps):
            lm_head_call(bq, s)
    elif target == "lmhead_compact":
        s = setup_lm_head(torch, bq, synth)
        cpk = bq.q6k_pack_compact(s["raw"], s["N"], s["K"])
        for _ in range(reps):
            bq.q6k_lmhead_top1(cpk, s["N"], s["K"], s["x"], s["row0"], s["rows"], s["ids"],
                               s["scratch"], compact=True)
    elif target == "down_sweep":
        time_down_sweep(torch, bq, synth, reps)
    elif target == "packed_one":
        # one launch kind at one M on one shape, so that a counter record
        # holds nothing else: --shape ffn_up|down, --m, --launch
        # whole (no workspace) | ws (CU-balanced) | split (the split count for m rows)
        cfg = synth.FFN_UP if args.shape == "ffn_up" else synth.DOWN_SWEEP
        N, K, m = cfg["N"], cfg["K"], args.m
        w0 = synth.q4_0_weights_device(cfg["seed"], N, K)
        wps = [bq.q4_0_pack(w0)] + [None] * (ROTATE - 1)
        for i in range(1, ROTATE):
            wps[i] = wps[0].clone()
        del w0
        xq = bq.q8_1_quantize(torch.randn((m, K), device="cuda"))
        P = bq.q4_0_mmvq_packed_splits_rows(N, K, m)
        y = torch.empty((P, m, N), dtype=torch.float32, device="cuda")
        pw = bq.q4_0_mmvq_packed_workspace()
        for i in range(reps):
            wp = wps[i % ROTATE]
            if args.launch == "split":
                bq.q4_0_mmvq_packed_split(wp, N, K, xq, m, P, y)
            elif args.launch == "ws":
                bq.q4_0_mmvq_packed(wp, N, K, xq, m, y[0], ws=pw)
            else:
                bq.q4_0_mmvq_packed(wp, N, K, xq, m, y[0])
    elif target in ("stream", "stream_packed"):
        time_stream(torch, bq, synth, reps, target == "stream_packed")
    else:
        raise SystemExit(f"unknown profile target {target}")
    torch.cuda.synchronize()
    log(f"{target}: done")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2000)
    ap.add_argument("--warmup", type=int, default=2000)
    ap.add_argument("--profile-target", default=None)
    ap.add_argument("--reps", type=int, default=200)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--shape", choices=("ffn_up", "down"), default="ffn_up",
                    help="packed_one profile target: the workload shape")
    ap.add_argument("--m", type=int, default=6, help="packed_one profile target: M")
    ap.add_argument("--launch", choices=("whole", "ws", "split"), default="whole",
                    help="packed_one profile target: which launch")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path (each MI355X runs its "
              "own shard; see the sharding notes). Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch
    import block_quantized_gemv_q8_amd as bq
    from block_quantized_gemv_q8_amd import synth

    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)
    bq.lib()

    if args.profile_target:
        profile_target(torch, bq, synth, args.profile_target, args.reps, args)
        return

    log("bench: ffn_up setup (12 weight copies, packed once)")
    s = setup_ffn_up(torch, bq, synth)
    N, K, M = s["N"], s["K"], s["M"]
    wbytes = q4_0_bytes(N, K)
    # untimed warm-up: --warmup steps, then more until WARMUP_MIN_S of wall
    # time has passed (the first short region after a pause runs slow, and
    # the driver's --warmup 5 is a few tens of microseconds); its last
    # batch runs inside a Timer, so the timing events' first use is not in
    # the timed region
    warm_steps = 0
    t0 = time.perf_counter()
    while warm_steps < args.warmup or time.perf_counter() - t0 < WARMUP_MIN_S:
        for _ in range(20):
            step_packed(bq, s, warm_steps)
            warm_steps += 1
        if warm_steps % 200 == 0:
            torch.cuda.synchronize()
    with Timer(torch):
        for _ in range(20):
            step_packed(bq, s, warm_steps)
            warm_steps += 1
    # the K timed steps: the step's two C entry points called on raw device
    # pointers (the host then spends about 9 us a step, under the GPU's
    # 12.6), behind an untimed backlog of STEP_BACKLOG steps, so that the
    # GPU is still busy when the first timing event is recorded and runs the
    # K steps back to back; the collector is paused meanwhile
    raw = raw_step(torch, bq, s)
    ev_a = torch.cuda.Event(enable_timing=True)
    ev_b = torch.cuda.Event(enable_timing=True)
    gc.disable()
    try:
        torch.cuda.synchronize()
        for i in range(STEP_BACKLOG):
            raw(warm_steps + i)
        ev_a.record()
        for i in range(args.steps):
            raw(warm_steps + STEP_BACKLOG + i)
        ev_b.record()
        torch.cuda.synchronize()
    finally:
        gc.enable()
    step_us = ev_a.elapsed_time(ev_b) * 1000.0 / args.steps
    value = wbytes / step_us / 1e3  # GB/s
    log(f"bench: step (quantize + packed M=6) {step_us:.3f} us, {value:.1f} GB/s")
    # the same K steps from an idle GPU: as one replayed HIP graph (each
    # graph launch costs the GPU about 10 us: 13.3 us a step at K = 20,
    # 12.8 at K = 200), and issued eagerly through the binding
    g = capture(torch, lambda i: step_packed(bq, s, warm_steps + i), args.steps)
    g.replay()
    with Timer(torch) as t:
        g.replay()
    del g
    step_graph_us = t.ms * 1000.0 / args.steps
    log(f"bench: step as one replayed graph from an idle GPU {step_graph_us:.3f} us")
    # the same steps issued eagerly, one library call at a time
    with Timer(torch) as t:
        for i in range(args.steps):
            step_packed(bq, s, warm_steps + i)
    eager_step_us = t.ms * 1000.0 / args.steps
    log(f"bench: step issued eagerly {eager_step_us:.3f} us")
    step_b = time_batches(torch, lambda i: step_packed(bq, s, i), args.steps, 10)
    bq.q8_1_quantize(s["x"], s["xq"])
    reps = max(args.steps, 100)
    # the roofline kernel: the median of 20 batch means, each batch 100
    # back-to-back launches rotating the 12 weight copies, after 1000 untimed
    # launches of the kernel alone (its first milliseconds after the step
    # phase run a few percent slower than its steady state)
    packed_b = time_batches(torch, lambda i: bq.q4_0_mmvq_packed(
        s["wps"][i % ROTATE], N, K, s["xq"], M, s["y"], ws=s["pws"]), 100, 20, warm=1000)
    packed_us = packed_b["median"]
    achieved = wbytes / packed_us / 1e3
    log(f"bench: q4_0_mmvq_packed M=6 {packed_us:.3f} us (p10 {packed_b['p10']:.3f}, p90 "
        f"{packed_b['p90']:.3f}), {achieved:.1f} GB/s")
    probe_ffn = hbm_probe(torch, bq, s["wps"], 100)
    log(f"bench: HBM read probe over the same 12 packed copies {probe_ffn['us_median']:.3f} us, "
        f"{probe_ffn['GBps']} GB/s ({probe_ffn['launch']})")
    clocks = clocks_under_load(torch, lambda i: bq.q4_0_mmvq_packed(
        s["wps"][i % ROTATE], N, K, s["xq"], M, s["y"], ws=s["pws"]))
    log(f"bench: clocks while the product runs untimed: {clocks}")
    std_us = time_calls(torch, lambda i: bq.q4_0_mmvq_m6(s["ws"][i % ROTATE], s["xq"], s["y"]),
                        reps, warm=20)
    std_step_us = time_calls(torch, lambda i: step_standard(bq, s, i), reps, warm=20)
    log(f"bench: q4_0_mmvq_m6 (GGUF layout) {std_us:.3f} us; step {std_step_us:.3f} us")
    quant_us = time_calls(torch, lambda i: bq.q8_1_quantize(s["x"], s["xq"]), reps, warm=20)
    joint_b = time_batches(torch, lambda i: gate_up_joint(bq, s, i), reps // 10, 10, warm=20)
    joint_us = joint_b["median"]
    sep_us = time_calls(torch, lambda i: gate_up_separate(bq, s, i), reps, warm=20)
    sep_gguf_us = time_calls(torch, lambda i: gate_up_separate_gguf(bq, s, i), reps, warm=20)
    log(f"bench: gate/up + SiLU*up + Q8_1: joint {joint_us:.3f} us, separate {sep_us:.3f} us, "
        f"separate GGUF layout {sep_gguf_us:.3f} us")
    del s

    log("bench: lm_head setup")
    lm = setup_lm_head(torch, bq, synth)
    lm_b = time_batches(torch, lambda i: lm_head_call(bq, lm), 10, 10, warm=5)
    lm_us = lm_b["median"]
    pack_bytes = lm["pack"].numel()
    log(f"bench: lmhead_top1 {lm_us:.2f} us, {pack_bytes / lm_us / 1e3:.1f} GB/s")
    # head variants: all six target-side rows, and candidate-max (one drafted
    # candidate per row) on rows 1..5
    scratch6 = torch.empty((bq.q6k_lmhead_top1_scratch_bytes(lm["N"], lm["K"], 6),),
                           dtype=torch.uint8, device="cuda")
    ids6 = torch.empty((6,), dtype=torch.int32, device="cuda")
    lm6_us = time_calls(torch, lambda i: bq.q6k_lmhead_top1(
        lm["pack"], lm["N"], lm["K"], lm["x"], 0, 6, ids6, scratch6), 50, warm=5)
    cand = torch.arange(5, dtype=torch.int32, device="cuda").view(5, 1) * 1000
    cm_us = time_calls(torch, lambda i: bq.q6k_lmhead_candidate_max(
        lm["pack"], lm["N"], lm["K"], lm["x"], 1, 5, cand, lm["scratch"]), 50, warm=5)
    log(f"bench: lmhead rows 0..5 {lm6_us:.2f} us; candidate-max rows 1..5 {cm_us:.2f} us")
    # the compact pack (raw Q6_K bits re-tiled) of the same weights
    cpk = bq.q6k_pack_compact(lm["raw"], lm["N"], lm["K"])
    lmc_b = time_batches(torch, lambda i: bq.q6k_lmhead_top1(
        cpk, lm["N"], lm["K"], lm["x"], lm["row0"], lm["rows"], lm["ids"], lm["scratch"],
        compact=True), 10, 10, warm=5)
    lmc_us = lmc_b["median"]
    cpk_bytes = cpk.numel()
    log(f"bench: lmhead_top1 compact {lmc_us:.2f} us, {cpk_bytes / lmc_us / 1e3:.1f} GB/s")
    probe_lm = hbm_probe(torch, bq, [cpk], 10)
    log(f"bench: HBM read probe over the compact pack {probe_lm['us_median']:.2f} us, "
        f"{probe_lm['GBps']} GB/s")
    del cpk
    del lm

    log("bench: down_sweep")
    sweep = time_down_sweep(torch, bq, synth, 100)
    log(f"bench: sweep {sweep}")

    log("bench: 8-way shard shapes")
    shards = time_shards(torch, bq, synth)
    log(f"bench: shards {shards}")

    log("bench: stream (packed)")
    stream_p = time_stream(torch, bq, synth, 20, packed=True)
    log(f"bench: stream packed {stream_p['ms_median']:.3f} ms per pass, {stream_p['GBps']} GB/s")
    log("bench: stream (GGUF layout)")
    stream_s = time_stream(torch, bq, synth, 10, packed=False)
    log(f"bench: stream gguf {stream_s['ms_median']:.3f} ms per pass")

    cpu = cpu1 = None
    if not args.no_cpu_baseline:
        log("bench: cpu baseline (oracle)")
        cpu = cpu_baseline(synth)
        cpu1 = cpu_one_thread(synth)

    traffic = pmc_traffic()
    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_us / 1000.0, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "q4_0 x q8_1 (int8 MFMA dot, f32 accumulate)",
        "data": "synthetic (seeded; weights and activations resident in HBM, 12 rotating "
                "weight copies)",
        "config": {
            "workload": "ffn_up: Q8_1 quantize of [6][5120] f32 + Q4_0 [17408x5120] M=6 "
                        "projection (weight in the offline-packed layout, packed once, untimed)",
            "N": N, "K": K, "M": M,
            "weight_bytes": wbytes,
            # the 4-bit codes alone (16 of every 18 bytes), the basis of the
            # pages' "~45 MB" for this projection
            "nibble_bytes": wbytes * 16 // 18,
            "step_GBps_nibble_only": round(wbytes * 16 / 18 / step_us / 1e3, 1),
            "packed_mmvq_GBps_nibble_only": round(wbytes * 16 / 18 / packed_us / 1e3, 1),
            "step_us": round(step_us, 3),
            "warmup_steps_run": warm_steps,
            "warmup_min_s": WARMUP_MIN_S,
            "step_timing": "the K steps' library calls issued behind an untimed backlog "
                           f"of {STEP_BACKLOG} steps, so the region between the two events "
                           "holds the K steps back to back",
            "step_graph_us_from_idle": round(step_graph_us, 3),
            "step_eager_us": round(eager_step_us, 3),
            "step_eager_us_batches": stats_us(step_b),
            "product_launch": "q4_0_mmvq_packed_ws; at M <= 8 it runs every 16-row tile "
                              "whole (the q4_0_mmvq_packed launch)",
            "packed_mmvq_us": round(packed_us, 3),
            "packed_mmvq_us_batches": stats_us(packed_b),
            "hbm_read_probe": probe_ffn,
            "pct_of_probe_mmvq": round(100 * probe_ffn["us_median"] / packed_us, 2),
            "quantize_us": round(quant_us, 3),
            "pct_hbm_peak_step": round(100 * value / HBM_PEAK_GBS, 2),
            "pct_hbm_peak_mmvq": round(100 * achieved / HBM_PEAK_GBS, 2),
            "gguf_layout": {"q4_0_mmvq_m6_us": round(std_us, 3),
                            "GBps": round(wbytes / std_us / 1e3, 1),
                            "step_us": round(std_step_us, 3)},
            "gate_up_silu_q8_1": {
                "joint_us": round(joint_us, 3),
                "joint_us_batches": stats_us(joint_b),
                "joint_GBps": round(2 * wbytes / joint_us / 1e3, 1),
                "separate_packed_us": round(sep_us, 3),
                "separate_gguf_us": round(sep_gguf_us, 3),
                "pct_hbm_peak": round(100 * 2 * wbytes / joint_us / 1e3 / HBM_PEAK_GBS, 2),
                "traffic": pmc_traffic(PMC_RECORD_GATE_UP),
                "algorithmic_weight_bytes": 2 * wbytes,
                "what": "gate [17408x5120] + up [17408x5120] Q4_0, M=6, SiLU(g)*u requantized "
                        "to Q8_1: one joint launch (CU-balanced, q4_0_gate_up_silu_q8_1_packed_ws) "
                        "vs two packed products + silu_mul_q8_1"},
            "lmhead_top1_us": round(min(lm_us, lmc_us), 2),
            "lmhead_top1_expanded_pack_us": round(lm_us, 2),
            "lmhead_top1_expanded_pack_us_batches": stats_us(lm_b, 2),
            "lmhead_target_rows_0_5_us": round(lm6_us, 2),
            "lmhead_top1_compact": {"us": round(lmc_us, 2), **stats_us(lmc_b, 2),
                                    "pack_bytes": cpk_bytes,
                                    "GBps": round(cpk_bytes / lmc_us / 1e3, 1),
                                    "hbm_read_probe": probe_lm,
                                    "pct_of_probe": round(100 * probe_lm["us_median"] / lmc_us,
                                                          2)},
            "lmhead_candidate_max_rows_1_5_us": round(cm_us, 2),
            "lmhead_expanded_pack_bytes": pack_bytes,
            "lmhead_expanded_GBps": round(pack_bytes / lm_us / 1e3, 1),
            "lmhead_expanded_pct_hbm_peak": round(100 * pack_bytes / lm_us / 1e3 / HBM_PEAK_GBS,
                                                  2),
            "down_sweep": sweep,
            "shards_8_way": shards,
            "stream_64_layer_pass": stream_p,
            "stream_64_layer_pass_gguf_layout": stream_s,
            "device": device_info(torch, clocks),
            "cpu_oracle_one_thread": cpu1,
            "host": host_info(),
        },
        "roofline": {
            "bound": "hbm",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": traffic,
            "kernel": "q4_0_mmvq_packed M=6 (ffn_up, 50,135,040 algorithmic weight bytes per "
                      "launch)",
        },
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
