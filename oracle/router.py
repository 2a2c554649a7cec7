"""Router: logits, top-k, softmax weights.

[FT-deep] §2 (the paper's own framing): routing is computed exactly and the
model is left untouched; only how misses are served changes.  [FT-blog] §二
draws the router on the GPU feeding the hit/miss split.

Readings (pages silent):
* logit[t, e] = sum_j x[t, j] * W_r[e, j] in fp32.  Products of two bf16 values
  are exact in fp32, so only the order of the additions matters, and it is
  fixed: 64 lanes; with V the largest of 8, 4, 2, 1 such that H % (64*V) == 0,
  lane l adds j = 64*V*c + V*l + i for c = 0, 1, ... (outer) and i = 0..V-1
  (inner), one fp32 addition each; then the lanes are folded pairwise,
  s[l] += s[l + o] for o = 32, 16, 8, 4, 2, 1.  Because the routing ids must be
  reproduced bit for bit, this fp32 order is part of the definition.
* top-K by (logit descending, expert id ascending).
* weights = softmax over the K selected logits (renormalised over the K).
"""
from __future__ import annotations

import numpy as np

from .formats import bf16_bits_to_f64


def lane_width(H: int) -> int:
    for V in (8, 4, 2, 1):
        if H % (64 * V) == 0:
            return V
    raise ValueError("H must be a multiple of 64")


def logits_fixed_order(x_bits: np.ndarray, w_bits: np.ndarray) -> np.ndarray:
    """fp32 logits [B, E] from bf16 x [B, H] and bf16 router weights [E, H] (bit arrays)."""
    x = bf16_bits_to_f64(x_bits).astype(np.float32)
    w = bf16_bits_to_f64(w_bits).astype(np.float32)
    B, H = x.shape
    E = w.shape[0]
    V = lane_width(H)
    R = H // (64 * V)
    prod = (x[:, None, :] * w[None, :, :]).astype(np.float32)  # exact in fp32
    prod = prod.reshape(B, E, R, 64, V)
    acc = np.zeros((B, E, 64), np.float32)
    for c in range(R):
        for i in range(V):
            acc = (acc + prod[:, :, c, :, i]).astype(np.float32)
    o = 32
    while o >= 1:
        acc[:, :, :o] = (acc[:, :, :o] + acc[:, :, o:2 * o]).astype(np.float32)
        o //= 2
    return acc[:, :, 0].copy()


def topk_softmax(logits: np.ndarray, K: int):
    """(ids int32 [B, K] ordered by (logit desc, id asc), weights float64 [B, K])."""
    logits = np.asarray(logits, np.float32)
    B, E = logits.shape
    ids = np.empty((B, K), np.int32)
    for b in range(B):
        order = sorted(range(E), key=lambda e: (-float(logits[b, e]), e))
        ids[b] = order[:K]
    sel = np.take_along_axis(logits.astype(np.float64), ids.astype(np.int64), axis=1)
    ex = np.exp(sel - sel[:, :1])
    return ids, ex / ex.sum(axis=1, keepdims=True)


def route(x_bits: np.ndarray, w_bits: np.ndarray, K: int):
    lg = logits_fixed_order(x_bits, w_bits)
    ids, w = topk_softmax(lg, K)
    return ids, w, lg
