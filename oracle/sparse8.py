"""ReLU^2 gate, per-token top-k sparsification and INT8 codes (oracle; test infrastructure).

BitNet a4.8 abstract: intermediate states are sparsified and then quantized to
8 bits.  toshoseti review, «Метод»: the out projection's input is sparsified by
top-k at 50 % sparsity, and the FFN gate uses ReLU^2 instead of swish to drive
the down projection's input towards sparsity.  9pt.com article (methodology):
sparsification drops the low-magnitude entries.  toshoseti review, opening
lines: b1.58 activations are absmax INT8.

Readings:
* h = ReLU(gate)^2 * up, elementwise, as fl(fl(r * r) * up) in fp32 with
  r = max(gate, 0) (exact for bf16 inputs of normal range);
* per token keep the k entries of largest |h| (k = K/2 by default); among equal
  magnitudes the lower index wins (the survivors are the first k of the order
  "magnitude descending, index ascending");
* INT8 absmax over the survivors: a' = max(max |h_survivor|, 1e-5),
  inv = fl(127 / a'), s = fl(a' / 127), q = clamp(rne(fl(h * inv)), -128, 127)
  for survivors, 0 for dropped entries.
* top-k applies to both out_proj and down_proj inputs; k = K turns it off
  (the b1.58 INT8 path).
"""
from __future__ import annotations

import numpy as np

EPS = np.float32(1e-5)


def relu2_gate(gate: np.ndarray, up: np.ndarray) -> np.ndarray:
    g = np.ascontiguousarray(gate, dtype=np.float32)
    u = np.ascontiguousarray(up, dtype=np.float32)
    r = np.where(g > 0, g, np.float32(0.0)).astype(np.float32)
    return ((r * r) * u).astype(np.float32)


def topk_mask(h: np.ndarray, k: int) -> np.ndarray:
    """bool [M][K]: True for the k survivors of each row (|h| descending, index ascending)."""
    h = np.ascontiguousarray(h, dtype=np.float32)
    M, K = h.shape
    if not 1 <= k <= K:
        raise ValueError("k must be in [1, K]")
    key = np.abs(h).astype(np.float64)
    idx = np.broadcast_to(np.arange(K), (M, K))
    order = np.lexsort((idx, -key), axis=-1)  # primary: -|h| ascending, then index
    keep = np.zeros((M, K), dtype=bool)
    np.put_along_axis(keep, order[:, :k], True, axis=1)
    return keep


def quantize_int8(h: np.ndarray, keep: np.ndarray):
    """INT8 absmax codes of the survivors: (codes int8 [M][K], scales float32 [M])."""
    h = np.ascontiguousarray(h, dtype=np.float32)
    mag = np.where(keep, np.abs(h), np.float32(0.0))
    a = np.maximum(mag.max(axis=1), EPS).astype(np.float32)
    inv = np.float32(127.0) / a
    s = a / np.float32(127.0)
    t = h * inv[:, None]
    q = np.clip(np.rint(t), -128, 127)
    q = np.where(keep, q, 0).astype(np.int8)
    return q, s.astype(np.float32)


def sparse_a8(gate_or_x: np.ndarray, up: np.ndarray | None, k: int):
    """Full sparse front end: (h, keep mask, codes, scales).  up=None means the
    plain-input front end (out_proj): h = x."""
    h = relu2_gate(gate_or_x, up) if up is not None else np.ascontiguousarray(gate_or_x, dtype=np.float32)
    keep = topk_mask(h, k)
    q, s = quantize_int8(h, keep)
    return h, keep, q, s


def mask_words(keep: np.ndarray) -> np.ndarray:
    """Survivor mask as uint32 [M][K/32]: bit i of word w is entry 32w + i."""
    M, K = keep.shape
    b = keep.reshape(M, K // 32, 32).astype(np.uint64)
    return (b << np.arange(32, dtype=np.uint64)).sum(axis=-1).astype(np.uint32)
