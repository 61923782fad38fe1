"""First calls into libbq8 from several host threads at once, in a fresh
process, so that each kernel's one-time dynamic-LDS opt-in and each cached
device property is first reached by threads racing for it.

Every thread runs one entry point on a stream of its own, into outputs of its
own (and a workspace of its own where the call takes one).  Afterwards each
result must equal, bit for bit, the same call made again from the main thread
on the default stream.  Prints "threads ok" when all of them do."""
import os
import sys
import threading

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402
import torch  # noqa: E402

from block_quantized_gemv_q8_amd import api as bq  # noqa: E402
from block_quantized_gemv_q8_amd import synth  # noqa: E402

N, K = 4096, 5120


def jobs(wp, wgp, wup, w, xq):
    """name -> a call that returns the tensors to compare."""
    def ws():
        return bq.q4_0_mmvq_packed_workspace()

    out = {}
    for M in (1, 6, 9, 17):
        out[f"packed M={M}"] = lambda M=M: [bq.q4_0_mmvq_packed(wp, N, K, xq[M], M)]
    for M in (6, 12):
        out[f"packed_ws M={M}"] = lambda M=M: [bq.q4_0_mmvq_packed(wp, N, K, xq[M], M, ws=ws())]
    out["packed_split M=2 x4"] = lambda: [bq.q4_0_mmvq_packed_split(wp, N, K, xq[2], 2, 4)]
    out["gate_up M=6"] = lambda: [bq.q4_0_gate_up_silu_q8_1_packed(wgp, wup, N, K, xq[6], 6)]
    out["gate_up_ws M=9"] = lambda: [bq.q4_0_gate_up_silu_q8_1_packed(wgp, wup, N, K, xq[9], 9,
                                                                       ws=ws())]
    for M in (6, 17):
        out[f"gguf M={M}"] = lambda M=M: [bq.q4_0_mmvq(w, xq[M], M)]
    return out


def bits(t):
    a = t.detach().cpu().contiguous().numpy()
    return a.view(np.uint8).copy()


def main():
    dev = torch.device("cuda", 0)
    rng = np.random.default_rng(9900)
    w = torch.from_numpy(synth.q4_0_weights(rng, N, K)).to(dev)
    wg = torch.from_numpy(synth.q4_0_weights(rng, N, K)).to(dev)
    wu = torch.from_numpy(synth.q4_0_weights(rng, N, K)).to(dev)
    x = torch.from_numpy(synth.normal_rows(rng, 17, K)).to(dev)
    # set-up on the main thread: packing and quantizing use no LDS opt-in
    wp, wgp, wup = bq.q4_0_pack(w), bq.q4_0_pack(wg), bq.q4_0_pack(wu)
    xq = {M: bq.q8_1_quantize(x[:M].contiguous()) for M in (1, 2, 6, 9, 12, 17)}
    torch.cuda.synchronize()

    calls = jobs(wp, wgp, wup, w, xq)
    names = list(calls)
    streams = [torch.cuda.Stream(device=dev) for _ in names]
    results, errors = {}, []
    gate = threading.Barrier(len(names))

    def run(name, stream):
        try:
            torch.cuda.set_device(dev)
            with torch.cuda.stream(stream):
                gate.wait()
                results[name] = calls[name]()
            stream.synchronize()
        except Exception as e:  # reported below, after every thread ends
            errors.append(f"{name}: {e!r}")

    print(f"starting {len(names)} threads: {', '.join(names)}", flush=True)
    threads = [threading.Thread(target=run, args=(n, s)) for n, s in zip(names, streams)]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=120)
    if any(t.is_alive() for t in threads):
        print("a thread did not finish", flush=True)
        return 1
    torch.cuda.synchronize()
    if errors:
        print("\n".join(errors), flush=True)
        return 1

    bad = []
    for name in names:
        again = calls[name]()
        torch.cuda.synchronize()
        for a, b in zip(results[name], again):
            if not np.array_equal(bits(a), bits(b)):
                bad.append(name)
    if bad:
        print("differ from the main thread's calls: " + ", ".join(bad), flush=True)
        return 1
    print("threads ok", flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
