"""Seeded synthetic inputs shared by the oracle tests, the GPU tests and the bench.

This module only draws random numbers and stores them in the input formats
(float32, or bfloat16 bit patterns rounded to nearest-even).  It holds none of
the routing / layout / planning arithmetic and imports neither the oracle nor
the HIP binding.

Workloads (router logits for one GPU's token batch; all values synthetic, no
trained router is involved):

  tiny     N=128    E=8   K=2  fp32 N(0,1)                 softmax top-2, A=1,   R=2
  small    N=4096   E=8   K=2  bf16 N(0,1)                 softmax top-2, A=128, R=8
  skewed   N=16384  E=128 K=8  bf16 N(0,2)+1.5 on e<4      softmax top-8, A=128, R=8
  dsv3     N=65536  E=256 K=8  fp32 N(0,1), bias U(-.1,.1) sigmoid, 8 groups keep 4, A=128, R=8
  dsv3big  N=262144 E=256 K=8  bf16 N(0,1), 10% rows equal sigmoid grouped as above, R=32

N(0,2) is read as variance 2 (standard deviation sqrt(2)).
"""
from __future__ import annotations

from dataclasses import dataclass, field, replace

import numpy as np

F32, BF16 = 0, 1
SOFTMAX, SIGMOID = 0, 1


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (nearest, ties to even); return uint16 bit patterns."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).copy()
    lsb = (u >> 16) & np.uint32(1)
    u += np.uint32(0x7FFF)      # no wrap for finite inputs: |bits| <= 0xFF7FFFFF
    u += lsb
    u >>= 16
    return u.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


@dataclass(frozen=True)
class Workload:
    name: str
    N: int
    E: int
    K: int
    dtype: int            # F32 or BF16
    score_fn: int         # SOFTMAX or SIGMOID
    renormalize: bool
    n_group: int
    topk_group: int
    group_topn: int
    scale: float
    alignment: int
    R: int
    num_channels: int
    seed: int
    num_src: int = 0      # 0 -> R (one virtual source shard per rank)
    extra: dict = field(default_factory=dict, compare=False, hash=False)

    @property
    def S(self) -> int:
        return self.num_src if self.num_src > 0 else self.R

    @property
    def epn(self) -> int:
        return self.E // self.R

    @property
    def NvS(self) -> int:
        return self.N * min(self.K, self.epn) + self.epn * (self.alignment - 1)


WORKLOADS = {
    "tiny": Workload("tiny", 128, 8, 2, F32, SOFTMAX, True, 1, 1, 2, 1.0, 1, 2, 24, seed=1),
    "small": Workload("small", 4096, 8, 2, BF16, SOFTMAX, True, 1, 1, 2, 1.0, 128, 8, 24, seed=2),
    "skewed": Workload("skewed", 16384, 128, 8, BF16, SOFTMAX, True, 1, 1, 2, 1.0, 128, 8, 24,
                       seed=3, extra={"std": 2.0 ** 0.5, "hot": 4, "hot_shift": 1.5}),
    "dsv3": Workload("dsv3", 65536, 256, 8, F32, SIGMOID, True, 8, 4, 2, 2.5, 128, 8, 24,
                     seed=4, extra={"bias": 0.1}),
    "dsv3big": Workload("dsv3big", 262144, 256, 8, BF16, SIGMOID, True, 8, 4, 2, 2.5, 128, 32, 24,
                        seed=5, extra={"bias": 0.1, "dup_frac": 0.10}),
}


@dataclass
class Inputs:
    logits: np.ndarray          # float32 [N,E] or uint16 bf16 bits [N,E]
    bias: np.ndarray | None     # float32 [E] (sigmoid scoring) or None
    wl: Workload


def make_inputs(wl: Workload, N: int | None = None) -> Inputs:
    """Draw the workload's logits (and bias). N overrides the token count (prefix of the draw
    is not guaranteed; the draw is repeated with the same seed at the new size)."""
    n_tok = wl.N if N is None else N
    rng = np.random.Generator(np.random.PCG64(wl.seed))
    std = wl.extra.get("std", 1.0)
    x = rng.standard_normal((n_tok, wl.E), dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    hot = wl.extra.get("hot", 0)
    if hot:
        x[:, :hot] += np.float32(wl.extra["hot_shift"])
    dup_frac = wl.extra.get("dup_frac", 0.0)
    if dup_frac > 0.0 and n_tok > 1:
        n_dup = int(round(dup_frac * n_tok))
        rows = rng.choice(n_tok, size=n_dup, replace=False)
        x[rows] = x[rows[0]]
    bias = None
    if wl.score_fn == SIGMOID:
        b = wl.extra.get("bias", 0.0)
        bias = rng.uniform(-b, b, size=wl.E).astype(np.float32)
    logits = f32_to_bf16_bits(x) if wl.dtype == BF16 else np.ascontiguousarray(x)
    return Inputs(logits, bias, wl if N is None else replace(wl, N=n_tok))


def random_ids(N: int, E: int, K: int, seed: int, hot: int = 0) -> np.ndarray:
    """Top-K style id rows: K distinct experts per token, optionally skewed toward `hot` experts."""
    rng = np.random.Generator(np.random.PCG64(seed))
    keys = rng.random((N, E))
    if hot:
        keys[:, :hot] += 0.5
    return np.argsort(-keys, axis=1, kind="stable")[:, :K].astype(np.int32)
