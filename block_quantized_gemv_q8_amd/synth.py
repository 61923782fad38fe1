"""Seeded synthetic inputs for the hot path's workloads.

This module is shared by the GPU path's tests and benchmark and by the CPU
oracle's tests.  It holds none of the method's arithmetic: it draws random
numbers, rounds scales to fp16 with numpy's own conversion and lays the
random bytes out in the block formats (Q4_0: fp16 d then 16 nibble bytes;
raw Q6_K: ql[128], qh[64], scales[16], fp16 d).  Quantization, unpacking,
dot products and reductions live only in the oracle and in the HIP kernels.

Workloads (shapes and distributions of the width-6 speculative verifier and
the draft LM head in "Qwen3.6 27B Q4_0 DFlash/SYCL closure" and "Q6_K M=6
fused DFlash top-1 production record"; the pages publish no data, so every
input is synthetic):

* tiny        Q4_0 N=256, K=256, M=1.                                 seed 1
* ffn_up      Q4_0 N=17408, K=5120, M=6; x ~ N(0,1) with 51 of the 5120
              channels (1%) scaled by 20, the same channels in every row. seed 2
* down_sweep  Q4_0 N=5120, K=17408, M in {1,2,3,4,5,6,9,12,17}; x ~ N(0, 0.5^2),
              rows 0..M-1 of one [17][17408] draw.                       seed 3
* lm_head     Q6_K N=248320, K=5120 raw blocks: 6-bit codes uniform (random
              ql/qh bytes, so q = code-32 is uniform on [-32, 31]), int8
              subscales ~U{-64..63}, fp16 d ~U[1e-4, 1e-3]; x [6][5120] ~ N(0,1),
              rows 1..5 projected.                                       seed 4
* stream      64 layers of Q4_0 gate/up [5120->17408] and down [17408->5120]
              at M=6, generated on the device (``torch``).               seed 5

Q4_0 scales are d ~U[1e-3, 2e-2] (drawn in f32, rounded to fp16), nibbles
uniform on 0..15 (random bytes).
"""
from __future__ import annotations

import numpy as np

QK = 32
QK_K = 256
Q4_0_BYTES = 18
Q6_K_BYTES = 210

Q4_0_D_RANGE = (1e-3, 2e-2)
Q6_K_D_RANGE = (1e-4, 1e-3)
Q6_K_SC_RANGE = (-64, 63)

TINY = dict(name="tiny", N=256, K=256, M=1, seed=1)
FFN_UP = dict(name="ffn_up", N=17408, K=5120, M=6, seed=2, outlier_frac=0.01, outlier_scale=20.0)
DOWN_SWEEP = dict(name="down_sweep", N=5120, K=17408, Ms=(1, 2, 3, 4, 5, 6, 9, 12, 17), seed=3,
                  x_std=0.5)
LM_HEAD = dict(name="lm_head", N=248320, K=5120, M=6, row0=1, rows=5, seed=4)
LM_HEAD_TIES = ((0, 248319), (1, 256), (255, 256))
STREAM = dict(name="stream", layers=64, hidden=5120, ffn=17408, M=6, seed=5)


def random_bytes(rng: np.random.Generator, shape) -> np.ndarray:
    """Uniform random bytes (``Generator.bytes``) as a uint8 array."""
    n = int(np.prod(shape))
    return np.frombuffer(rng.bytes(n), dtype=np.uint8).reshape(shape)


def _f16_bits(values_f32: np.ndarray) -> np.ndarray:
    """fp16 bit patterns of f32 values (numpy's round-to-nearest-even)."""
    return np.asarray(values_f32, np.float32).astype(np.float16).view(np.uint16)


def q4_0_weights(rng: np.random.Generator, N: int, K: int,
                 d_range=Q4_0_D_RANGE) -> np.ndarray:
    """Random Q4_0 weight [N][K/32] blocks as uint8 [N][K/32*18].

    Draw order: all scales (f32 uniform), then all nibble bytes."""
    assert K % QK == 0
    nb = K // QK
    d = rng.uniform(d_range[0], d_range[1], size=(N, nb)).astype(np.float32)
    qs = random_bytes(rng, (N, nb, 16))
    w = np.empty((N, nb, Q4_0_BYTES), np.uint8)
    w[:, :, 0:2] = _f16_bits(d).astype("<u2").view(np.uint8).reshape(N, nb, 2)
    w[:, :, 2:] = qs
    return w.reshape(N, nb * Q4_0_BYTES)


def q6k_raw_weights(rng: np.random.Generator, N: int, K: int,
                    d_range=Q6_K_D_RANGE, sc_range=Q6_K_SC_RANGE) -> np.ndarray:
    """Random raw Q6_K [N][K/256] superblocks as uint8 [N][K/256*210].

    Draw order: ql/qh bytes (192 per superblock), subscales, scales."""
    assert K % QK_K == 0
    ns = K // QK_K
    raw = np.empty((N, ns, Q6_K_BYTES), np.uint8)
    raw[:, :, 0:192] = random_bytes(rng, (N, ns, 192))
    raw[:, :, 192:208] = rng.integers(sc_range[0], sc_range[1] + 1, size=(N, ns, 16),
                                      dtype=np.int8).view(np.uint8)
    d = rng.uniform(d_range[0], d_range[1], size=(N, ns)).astype(np.float32)
    raw[:, :, 208:210] = _f16_bits(d).astype("<u2").view(np.uint8).reshape(N, ns, 2)
    return raw.reshape(N, ns * Q6_K_BYTES)


def normal_rows(rng: np.random.Generator, M: int, K: int, std: float = 1.0) -> np.ndarray:
    return (rng.standard_normal((M, K), dtype=np.float32) * np.float32(std)).astype(np.float32)


def with_outlier_channels(rng: np.random.Generator, x: np.ndarray, frac: float,
                          scale: float) -> np.ndarray:
    """Scale round(frac*K) columns (the same in every row, drawn without
    replacement) by ``scale``."""
    K = x.shape[1]
    cols = rng.choice(K, size=int(round(frac * K)), replace=False)
    x = x.copy()
    x[:, cols] *= np.float32(scale)
    return x


# ------------------------------------------------------------------ configs
def tiny():
    rng = np.random.default_rng(TINY["seed"])
    w = q4_0_weights(rng, TINY["N"], TINY["K"])
    x = normal_rows(rng, TINY["M"], TINY["K"])
    return w, x


def ffn_up(N: int = FFN_UP["N"], K: int = FFN_UP["K"], M: int = FFN_UP["M"],
           seed: int = FFN_UP["seed"]):
    rng = np.random.default_rng(seed)
    w = q4_0_weights(rng, N, K)
    x = normal_rows(rng, M, K)
    x = with_outlier_channels(rng, x, FFN_UP["outlier_frac"], FFN_UP["outlier_scale"])
    return w, x


def down_sweep(N: int = DOWN_SWEEP["N"], K: int = DOWN_SWEEP["K"], seed: int = DOWN_SWEEP["seed"]):
    """Weights and the [17][K] activation draw; M rows are rows 0..M-1."""
    rng = np.random.default_rng(seed)
    w = q4_0_weights(rng, N, K)
    x = normal_rows(rng, max(DOWN_SWEEP["Ms"]), K, std=DOWN_SWEEP["x_std"])
    return w, x


def lm_head(N: int = LM_HEAD["N"], K: int = LM_HEAD["K"], seed: int = LM_HEAD["seed"]):
    rng = np.random.default_rng(seed)
    raw = q6k_raw_weights(rng, N, K)
    x = normal_rows(rng, LM_HEAD["M"], K)
    return raw, x


def random_q4_0_case(seed: int, N: int, K: int, M: int, x_std: float = 1.0):
    """Generic seeded Q4_0 case for parity sweeps over shapes."""
    rng = np.random.default_rng(seed)
    w = q4_0_weights(rng, N, K)
    x = normal_rows(rng, M, K, std=x_std)
    return w, x


# ------------------------------------------------------- device generator
def stream_layer_seed(layer: int, which: str) -> int:
    """Per-layer, per-matrix sub-seed of the 64-layer stream."""
    return STREAM["seed"] * 1_000_000 + layer * 10 + {"gate": 0, "up": 1, "down": 2}[which]


def q4_0_weights_device(seed: int, N: int, K: int, device="cuda", d_range=Q4_0_D_RANGE):
    """Random Q4_0 blocks generated on the device with a seeded torch
    generator (same distributions as ``q4_0_weights``; a different stream of
    random numbers).  Returns a uint8 tensor [N][K/32*18]."""
    import torch

    nb = K // QK
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    d = torch.empty((N, nb), dtype=torch.float32, device=device)
    d.uniform_(d_range[0], d_range[1], generator=g)
    qs = torch.randint(0, 256, (N, nb, 16), dtype=torch.uint8, device=device, generator=g)
    dbytes = d.to(torch.float16).view(torch.uint8).reshape(N, nb, 2)
    return torch.cat([dbytes, qs], dim=2).reshape(N, nb * Q4_0_BYTES).contiguous()


def q6k_raw_weights_device(seed: int, N: int, K: int, device="cuda", d_range=Q6_K_D_RANGE,
                           sc_range=Q6_K_SC_RANGE):
    """Random raw Q6_K superblocks generated on the device (same
    distributions as ``q6k_raw_weights``; a different random stream).
    Returns a uint8 tensor [N][K/256*210]."""
    import torch

    ns = K // QK_K
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    qbytes = torch.randint(0, 256, (N, ns, 192), dtype=torch.uint8, device=device, generator=g)
    sc = torch.randint(sc_range[0], sc_range[1] + 1, (N, ns, 16), dtype=torch.int8, device=device,
                       generator=g).view(torch.uint8)
    d = torch.empty((N, ns), dtype=torch.float32, device=device)
    d.uniform_(d_range[0], d_range[1], generator=g)
    dbytes = d.to(torch.float16).view(torch.uint8).reshape(N, ns, 2)
    return torch.cat([qbytes, sc, dbytes], dim=2).reshape(N, ns * Q6_K_BYTES).contiguous()


def stream_weights_device(layers: int = STREAM["layers"], hidden: int = STREAM["hidden"],
                          ffn: int = STREAM["ffn"], device="cuda"):
    """Gate, up ([ffn][hidden/32] Q4_0) and down ([hidden][ffn/32] Q4_0)
    weights of every stream layer, generated on the device from the
    per-layer sub-seeds.  Returns three lists of uint8 tensors."""
    gate = [q4_0_weights_device(stream_layer_seed(l, "gate"), ffn, hidden, device)
            for l in range(layers)]
    up = [q4_0_weights_device(stream_layer_seed(l, "up"), ffn, hidden, device)
          for l in range(layers)]
    down = [q4_0_weights_device(stream_layer_seed(l, "down"), hidden, ffn, device)
            for l in range(layers)]
    return gate, up, down


def stream_x0(M: int = STREAM["M"], hidden: int = STREAM["hidden"], seed: int = STREAM["seed"]):
    """Layer-0 input of the stream: f32 [M][hidden] ~ N(0, 1)."""
    return normal_rows(np.random.default_rng(seed), M, hidden)
