"""Seeded synthetic inputs for the guarded W8A8 linear layer.

This module only draws random numbers and rounds them to bf16 storage; it
holds none of the method's arithmetic.  The same bytes feed the CPU oracle
and the GPU library.  bf16 arrays are numpy ``uint16`` bit patterns; the
float32 -> bf16 rounding of the drawn values uses torch's CPU conversion
(round to nearest even).

The five workloads stand in for the linear layers of the TurboT2VA generator
(LTX-2 joint audio-video DiT at 1024x1792, 121 frames), whose trained weights
and prompts are not available here: token-row activations ~N(0,1) with a few
large-magnitude outlier channels, weights and biases ~N(0, sigma).

Draw order for every workload: outlier column indices, X, W, bias (then any
further tensors in the order listed), then lengths.  All use
``numpy.random.Generator(PCG64(seed))`` with seed 0 unless stated.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np


def to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """float32 array -> bf16 bit patterns (uint16), round to nearest even."""
    import torch

    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()


def from_bf16_bits(h: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> float32 values (exact widening)."""
    return (np.ascontiguousarray(h, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def _normal(rng, shape, sigma):
    a = rng.standard_normal(size=shape, dtype=np.float32)
    if sigma != 1.0:
        a *= np.float32(sigma)
    return a


def activations(rng, M, K, outlier_frac=0.0, outlier_count=None, factor=1.0):
    """X ~ N(0,1) [M, K]; round(frac*K) distinct outlier columns (or an exact
    count) scaled by ``factor`` before the bf16 rounding."""
    n_out = outlier_count if outlier_count is not None else int(round(outlier_frac * K))
    cols = np.sort(rng.choice(K, size=n_out, replace=False)) if n_out > 0 else np.zeros(0, np.int64)
    x = _normal(rng, (M, K), 1.0)
    if n_out > 0:
        x[:, cols] *= np.float32(factor)
    return to_bf16_bits(x), cols


@dataclass
class Linear:
    """One linear layer's inputs: X [M, K], W [N, K] (torch Linear layout), bias [N]."""
    name: str
    x: np.ndarray
    w: np.ndarray
    bias: np.ndarray
    act: int = 0  # 0 none, 1 GELU-tanh on the output
    outlier_cols: np.ndarray = field(default_factory=lambda: np.zeros(0, np.int64))

    @property
    def shape(self):
        return self.x.shape[0], self.w.shape[0], self.x.shape[1]


def tiny(seed=0):
    """X [64x256] ~N(0,1) with 4 outlier columns x20; W [128x256] ~N(0,0.02); b [128] ~N(0,0.01)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    x, cols = activations(rng, 64, 256, outlier_count=4, factor=20.0)
    w = to_bf16_bits(_normal(rng, (128, 256), 0.02))
    b = to_bf16_bits(_normal(rng, (128,), 0.01))
    return Linear("tiny", x, w, b, 0, cols)


def audio(seed=0, M=2048):
    """Audio-branch linear: X [2048x2048] ~N(0,1), 1% outlier columns x30;
    W [2048x2048] ~N(0,0.02); b ~N(0,0.01)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    x, cols = activations(rng, M, 2048, outlier_frac=0.01, factor=30.0)
    w = to_bf16_bits(_normal(rng, (2048, 2048), 0.02))
    b = to_bf16_bits(_normal(rng, (2048,), 0.01))
    return Linear("audio", x, w, b, 0, cols)


def video_attn_proj(seed=0, M=24576):
    """Video-branch attention projection: X [24576x4096] ~N(0,1), 0.5% outlier
    columns x50; W [4096x4096] ~N(0,0.015); b ~N(0,0.01)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    x, cols = activations(rng, M, 4096, outlier_frac=0.005, factor=50.0)
    w = to_bf16_bits(_normal(rng, (4096, 4096), 0.015))
    b = to_bf16_bits(_normal(rng, (4096,), 0.01))
    return Linear("video_attn_proj", x, w, b, 0, cols)


@dataclass
class FFNPair:
    """Video FFN pair: up X[M x 4096] W1[16384 x 4096] (+GELU-tanh), down W2[4096 x 16384]."""
    x: np.ndarray
    w1: np.ndarray
    b1: np.ndarray
    w2: np.ndarray
    b2: np.ndarray


def video_ffn(seed=0, M=24576, D=4096, F=16384):
    """X ~N(0,1); W1 [F x D], W2 [D x F] ~N(0,0.01); b1 [F], b2 [D] ~N(0,0.01)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    x, _ = activations(rng, M, D)
    w1 = to_bf16_bits(_normal(rng, (F, D), 0.01))
    b1 = to_bf16_bits(_normal(rng, (F,), 0.01))
    w2 = to_bf16_bits(_normal(rng, (D, F), 0.01))
    b2 = to_bf16_bits(_normal(rng, (D,), 0.01))
    return FFNPair(x, w1, b1, w2, b2)


@dataclass
class GuardedMixed:
    """Text rows [B x L x D] with per-sample valid lengths (prefix mask), one
    conforming projection, and two shapes the INT8 kernel cannot serve."""
    x: np.ndarray          # [B, L, D] bf16
    mask: np.ndarray       # [B, L] uint8, 1 = valid
    lengths: np.ndarray    # [B]
    w: np.ndarray          # [4096, 4096] conforming projection
    b: np.ndarray
    w_a: np.ndarray        # [4100, 4096]: N = 4100 (not a multiple of 64)
    b_a: np.ndarray
    x_b: np.ndarray        # [2048, 2050]: K = 2050 (not a multiple of 128)
    w_b: np.ndarray        # [2048, 2050]
    b_b: np.ndarray


def guarded_mixed(seed=0, B=8, L=512, D=4096):
    """Text X [8x512x4096] ~N(0,1) with lengths ~U{64..512} (prefix masks);
    W [4096x4096] ~N(0,0.02); fallback A W [4100x4096]; fallback B X [2048x2050],
    W [2048x2050]; all weights ~N(0,0.02), biases ~N(0,0.01)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    x = to_bf16_bits(_normal(rng, (B, L, D), 1.0))
    w = to_bf16_bits(_normal(rng, (4096, D), 0.02))
    b = to_bf16_bits(_normal(rng, (4096,), 0.01))
    w_a = to_bf16_bits(_normal(rng, (4100, D), 0.02))
    b_a = to_bf16_bits(_normal(rng, (4100,), 0.01))
    x_b = to_bf16_bits(_normal(rng, (2048, 2050), 1.0))
    w_b = to_bf16_bits(_normal(rng, (2048, 2050), 0.02))
    b_b = to_bf16_bits(_normal(rng, (2048,), 0.01))
    lengths = rng.integers(64, L, size=B, endpoint=True)
    mask = (np.arange(L)[None, :] < lengths[:, None]).astype(np.uint8)
    return GuardedMixed(x, mask, lengths, w, b, w_a, b_a, x_b, w_b, b_b)


def sample_rows(M, n, seed=1):
    """n distinct seeded row indices of [0, M), sorted, always including 0 and M-1."""
    rng = np.random.Generator(np.random.PCG64(seed))
    n = min(n, M)
    if n >= M:
        return np.arange(M)
    rows = set(rng.choice(M, size=n, replace=False).tolist())
    rows.update({0, M - 1})
    return np.array(sorted(rows), dtype=np.int64)
