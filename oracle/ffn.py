"""SwiGLU expert and top-k-weighted combine, in float64.

The expert computes down(silu(gate(x)) * up(x)) ([Edge0] "어떻게 동작하나": every
path evaluates this same expression; [NVMe-8GB] "엔진" item 4 names the NVFP4
SwiGLU expert kernel).  The GPU and host partial sums are merged by addition
([FT-deep] §4 design pattern ③; [FT-blog] §六 "两条分支的结果可以精确合并"),
which for one token is out[t] = sum_k w[t, k] * y_{ids[t, k]}(x_t).
Output rounding to bf16 is nearest-even.
"""
from __future__ import annotations

import numpy as np

from .formats import bf16_bits_to_f64, f64_to_bf16_bits


def silu(z: np.ndarray) -> np.ndarray:
    return z / (1.0 + np.exp(-z))


def expert_ffn(Wg: np.ndarray, Wu: np.ndarray, Wd: np.ndarray, x: np.ndarray) -> np.ndarray:
    """y [n, H] for x [n, H] (float64) through one expert (Wg, Wu [I, H]; Wd [H, I])."""
    g = x @ Wg.T
    u = x @ Wu.T
    return (silu(g) * u) @ Wd.T


def combine(y: np.ndarray, w: np.ndarray) -> np.ndarray:
    """out [B, H] = sum over k ascending of w[:, k] * y[:, k, :]  (float64)."""
    out = np.zeros((y.shape[0], y.shape[2]), np.float64)
    for k in range(y.shape[1]):
        out += w[:, k:k + 1] * y[:, k, :]
    return out


def combine_bf16(y: np.ndarray, w: np.ndarray) -> np.ndarray:
    return f64_to_bf16_bits(combine(y, w))


def x_f64(x_bits: np.ndarray) -> np.ndarray:
    return bf16_bits_to_f64(x_bits)
