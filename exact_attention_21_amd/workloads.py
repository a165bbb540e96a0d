"""Seeded synthetic workloads: shapes, value distributions and rounding to fp16/bf16.

This module holds no attention arithmetic.  It only draws the random inputs and
rounds them to the storage dtype; both the GPU path and the CPU oracle consume
what it returns.  It imports numpy only.

The five workloads are the attention-forward shapes the method is measured on:
a tiny correctness case, the 8-head N=8192 d=64 fp16 headline shape, a causal
training-style d=128 bf16 shape, a long-context causal N=32768 shape and a
d=256 bf16 shape with a ragged length and a wide score range.  Two masked
workloads exercise fa2_fwd_masked: a 4096-key causal sliding window over a
long sequence, and a causal batch of right-padded sequences of mixed lengths.
Two more run the chunked kernel of head dims 512 and 1024.

Draw recipe (one generator per call): ``numpy.random.default_rng(seed)``
(PCG64); Q, then K, then V, each drawn as one float64 array of shape
[B, H, N, d] in C order.  "normal" is ``standard_normal() * sigma``;
"uniform" is ``uniform(-1, 1)``.  fp16 rounding is numpy's float64 -> float16
cast (round to nearest even).  bf16 rounding is float64 -> float32 (numpy, round
to nearest even) followed by round-to-nearest-even of the float32 bit pattern to
its upper 16 bits.  Upcasting the rounded values to float64 is exact.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

FP16 = "fp16"
BF16 = "bf16"


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    N: int
    d: int
    dtype: str
    causal: bool
    q_dist: tuple = ("normal", 1.0)
    k_dist: tuple = ("normal", 1.0)
    v_dist: tuple = ("normal", 1.0)
    scale: float = field(default=None)
    # fa2_fwd_masked arguments: (left, right) window bounds (negative: none)
    # and per-sequence key lengths; None for the unmasked workloads.
    window: tuple = None
    key_lens: tuple = None

    @property
    def masked(self) -> bool:
        return self.window is not None or self.key_lens is not None

    def softmax_scale(self) -> float:
        return self.scale if self.scale is not None else 1.0 / float(np.sqrt(self.d))

    def visible_keys(self, rows=None) -> np.ndarray:
        """Number of keys each query row sees, [B, R] (R: all rows, or `rows`):
        j < key length, i - left <= j <= i + right (a negative bound is none;
        causal adds right = 0)."""
        i = np.arange(self.N) if rows is None else np.asarray(rows)
        left, right = self.window if self.window is not None else (-1, -1)
        if self.causal:
            right = 0 if right < 0 else min(right, 0)
        lens = self.key_lens if self.key_lens is not None else (self.N,) * self.B
        lo = np.zeros_like(i) if left < 0 else np.maximum(0, i - left)
        out = []
        for n_b in lens:
            hi = np.full_like(i, n_b) if right < 0 else np.minimum(n_b, i + right + 1)
            out.append(np.maximum(hi - lo, 0))
        return np.array(out)

    def flops(self) -> float:
        """Forward FLOPs of the metric: 4*d per visible (query, key) pair and
        head, i.e. 4*B*H*N^2*d, halved when causal; masked workloads count
        their visible pairs exactly."""
        if not self.masked:
            f = 4.0 * self.B * self.H * self.N * self.N * self.d
            return f / 2.0 if self.causal else f
        return 4.0 * self.H * self.d * float(self.visible_keys().sum())

    def backward_flops(self) -> float:
        """The metric's FLOP count of the backward pass: five products of
        2 N^2 d per (batch, head) (S, dP, dV, dK, dQ), 2.5 times the forward's,
        halved under the causal mask."""
        return 2.5 * self.flops()

    def describe(self) -> dict:
        out = {"B": self.B, "H": self.H, "N": self.N, "d": self.d, "dtype": self.dtype,
               "causal": self.causal, "scale": self.softmax_scale()}
        if self.window is not None:
            out["window"] = list(self.window)
        if self.key_lens is not None:
            out["key_lens"] = list(self.key_lens)
        return out


TINY = Workload("tiny_b1h1n128d64_fp16", 1, 1, 128, 64, FP16, False)
HEADLINE = Workload("headline_b1h8n8192d64_fp16", 1, 8, 8192, 64, FP16, False)
CAUSAL_TRAIN = Workload("causal_b2h16n4096d128_bf16", 2, 16, 4096, 128, BF16, True)
LONG_CAUSAL = Workload("longctx_causal_b1h4n32768d64_fp16", 1, 4, 32768, 64, FP16, True)
WIDE_RAGGED = Workload("wide_ragged_b4h8n2047d256_bf16", 4, 8, 2047, 256, BF16, False,
                       q_dist=("normal", 3.0), k_dist=("normal", 3.0), v_dist=("uniform", 1.0))

WORKLOADS = [TINY, HEADLINE, CAUSAL_TRAIN, LONG_CAUSAL, WIDE_RAGGED]

WINDOW = Workload("window4096_b1h8n32768d64_fp16", 1, 8, 32768, 64, FP16, False, window=(4095, 0))
PADDED_CAUSAL = Workload("padded_causal_b8h16n4096d128_bf16", 8, 16, 4096, 128, BF16, True,
                         key_lens=(4096, 3001, 2048, 517, 4096, 1290, 3777, 64))
MASKED_WORKLOADS = [WINDOW, PADDED_CAUSAL]

# Head dims past 256 (the chunked kernel).
D512 = Workload("d512_b2h4n8192_fp16", 2, 4, 8192, 512, FP16, False)
D1024_CAUSAL = Workload("d1024_causal_b2h2n8192_bf16", 2, 2, 8192, 1024, BF16, True)
HEADDIM_WORKLOADS = [D512, D1024_CAUSAL]
ALL_WORKLOADS = WORKLOADS + MASKED_WORKLOADS + HEADDIM_WORKLOADS


def _draw(rng: np.random.Generator, shape, dist) -> np.ndarray:
    kind, width = dist
    if kind == "normal":
        return rng.standard_normal(shape) * width
    if kind == "uniform":
        return rng.uniform(-width, width, shape)
    raise ValueError(f"unknown distribution {kind!r}")


def round_to_storage(x: np.ndarray, dtype: str) -> np.ndarray:
    """Round float64 values to the storage dtype.

    Returns float16 values for fp16 and uint16 bf16 bit patterns for bf16.
    """
    if dtype == FP16:
        return np.asarray(x, dtype=np.float64).astype(np.float16)
    if dtype == BF16:
        bits = np.asarray(x, dtype=np.float64).astype(np.float32).view(np.uint32)
        bias = np.uint32(0x7FFF) + ((bits >> np.uint32(16)) & np.uint32(1))
        return ((bits + bias) >> np.uint32(16)).astype(np.uint16)
    raise ValueError(f"unknown dtype {dtype!r}")


def to_float64(x: np.ndarray, dtype: str) -> np.ndarray:
    """Exact upcast of storage values (float16, or uint16 bf16 bits) to float64."""
    if dtype == FP16:
        return np.asarray(x, dtype=np.float16).astype(np.float64)
    if dtype == BF16:
        return (np.asarray(x, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    raise ValueError(f"unknown dtype {dtype!r}")


def make_inputs(w: Workload, seed: int = 0, N: int | None = None, B: int | None = None,
                H: int | None = None):
    """Draw Q, K, V for a workload (optionally with B, H or N overridden).

    Returns three storage arrays (float16, or uint16 bf16 bits) of shape [B, H, N, d].
    """
    shape = (B or w.B, H or w.H, N or w.N, w.d)
    rng = np.random.default_rng(seed)
    q = round_to_storage(_draw(rng, shape, w.q_dist), w.dtype)
    k = round_to_storage(_draw(rng, shape, w.k_dist), w.dtype)
    v = round_to_storage(_draw(rng, shape, w.v_dist), w.dtype)
    return q, k, v


def make_grad_output(w: Workload, seed: int = 0, N: int | None = None, B: int | None = None,
                     H: int | None = None, sigma: float = 1.0):
    """Draw the output gradient dO for a workload's backward pass: N(0, sigma^2)
    of shape [B, H, N, d] from its own generator, ``default_rng([seed, 1])``,
    rounded to the storage dtype (so Q, K, V of ``make_inputs`` are unchanged)."""
    shape = (B or w.B, H or w.H, N or w.N, w.d)
    rng = np.random.default_rng([seed, 1])
    return round_to_storage(rng.standard_normal(shape) * sigma, w.dtype)
