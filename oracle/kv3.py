"""3-bit KV-cache codec with 4-bit special tokens (oracle; test infrastructure).

toshoseti review, «Эксперименты»: the KV caches are quantized to 3 bits except
the <bos> and <eos> tokens, which are more sensitive and stay at 4 bits.
BitNet a4.8 abstract: the model supports a 3-bit KV cache.

Readings:
* one scale per (batch, position, head) vector of head_dim values, absmax;
* 3-bit: inv = fl(3 / a'), s3 = fl(a' / 3), q = clamp(rne(fl(x * inv)), -4, 3);
* 4-bit (special positions): inv = fl(7 / a'), s4 = fl(a' / 7),
  q = clamp(rne(fl(x * inv)), -8, 7);
* a' = max(max |x|, 1e-5); dequantized value = fl(q * s) in fp32;
* the caller marks special positions with 0 <= slot_of[b][s] < n_special (the
  index of a side-slab slot); any other value marks an ordinary token; every
  token also gets its 3-bit main-slab codes;
* main slab: per vector 3*D/8 bytes; per group of 32 codes three little-endian
  uint32 words W0, W1, W2 holding the fields u = q + 4 in [0, 7].  Byte i of
  the three words carries the eight codes 8i .. 8i+7 of the group (u_0 .. u_7
  below): W0 byte = u_0 | u_1 << 3 | (u_6 & 3) << 6,
  W1 byte = u_2 | u_3 << 3 | (u_6 >> 2) << 6 | (u_7 & 1) << 7,
  W2 byte = u_4 | u_5 << 3 | (u_7 >> 1) << 6 (a storage format of this
  library: the pages fix the bit width, not the bit order);
* side slab: per slot and head D/2 bytes of 4-bit codes, even d in the low nibble.
"""
from __future__ import annotations

import numpy as np

EPS = np.float32(1e-5)


def _absmax_last(x: np.ndarray) -> np.ndarray:
    return np.maximum(np.abs(x).max(axis=-1), EPS).astype(np.float32)


def quantize(x: np.ndarray, qmax: int, lo: int, hi: int):
    """Per-vector absmax codes over the last axis: (int8 codes, float32 scales)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    a = _absmax_last(x)
    inv = np.float32(qmax) / a
    s = a / np.float32(qmax)
    q = np.clip(np.rint(x * inv[..., None]), lo, hi).astype(np.int8)
    return q, s.astype(np.float32)


def planes_encode(q3: np.ndarray) -> np.ndarray:
    """int8 codes [..., D] in [-4, 3] -> uint8 [..., 3*D/8] (three words per 32 codes)."""
    D = q3.shape[-1]
    u = (q3.astype(np.int16) + 4).astype(np.uint8).reshape(q3.shape[:-1] + (D // 32, 4, 8))
    w0 = u[..., 0] | (u[..., 1] << 3) | ((u[..., 6] & 3) << 6)
    w1 = u[..., 2] | (u[..., 3] << 3) | ((u[..., 6] >> 2) << 6) | ((u[..., 7] & 1) << 7)
    w2 = u[..., 4] | (u[..., 5] << 3) | ((u[..., 7] >> 1) << 6)
    words = np.stack([w0, w1, w2], axis=-2).astype(np.uint8)  # [..., group][word][byte i]
    return words.reshape(q3.shape[:-1] + (3 * D // 8,))


def planes_decode(p: np.ndarray, D: int) -> np.ndarray:
    b = np.ascontiguousarray(p, dtype=np.uint8).reshape(p.shape[:-1] + (D // 32, 3, 4)).astype(np.int16)
    b0, b1, b2 = b[..., 0, :], b[..., 1, :], b[..., 2, :]
    u = np.stack([b0 & 7, (b0 >> 3) & 7, b1 & 7, (b1 >> 3) & 7, b2 & 7, (b2 >> 3) & 7,
                  (b0 >> 6) | (((b1 >> 6) & 1) << 2), (b1 >> 7) | ((b2 >> 6) << 1)], axis=-1)
    return (u - 4).astype(np.int8).reshape(p.shape[:-1] + (D,))


def nibbles_encode(q4: np.ndarray) -> np.ndarray:
    c = q4.astype(np.int16) & 0xF
    return (c[..., 0::2] | (c[..., 1::2] << 4)).astype(np.uint8)


def nibbles_decode(p: np.ndarray) -> np.ndarray:
    p = np.asarray(p, dtype=np.uint8)
    out = np.empty(p.shape[:-1] + (2 * p.shape[-1],), dtype=np.int16)
    out[..., 0::2] = p & 0xF
    out[..., 1::2] = p >> 4
    return np.where(out >= 8, out - 16, out).astype(np.int8)


def is_special(slot_of: np.ndarray, n_special: int) -> np.ndarray:
    """bool mask of the positions whose slot_of names a side-slab slot."""
    slot_of = np.asarray(slot_of)
    return (slot_of >= 0) & (slot_of < n_special)


def kv_pack3(x: np.ndarray, slot_of: np.ndarray, n_special: int):
    """x float32 [B][S][H][D] -> (p3 uint8 [B][S][H][3D/8], s3 f32 [B][S][H],
    p4 uint8 [n_special][H][D/2], s4 f32 [n_special][H]).  Side-slab slots that
    no position names stay zero."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    B, S, H, D = x.shape
    q3, s3 = quantize(x, 3, -4, 3)
    p3 = planes_encode(q3)
    p4 = np.zeros((n_special, H, D // 2), dtype=np.uint8)
    s4 = np.zeros((n_special, H), dtype=np.float32)
    bs = np.argwhere(is_special(slot_of, n_special))
    if len(bs):
        xs = x[bs[:, 0], bs[:, 1]]  # [n][H][D]
        q4, sc4 = quantize(xs, 7, -8, 7)
        slots = slot_of[bs[:, 0], bs[:, 1]]
        p4[slots] = nibbles_encode(q4)
        s4[slots] = sc4
    return p3, s3, p4, s4


def kv_unpack3(p3, s3, p4, s4, slot_of, D: int, n_special: int | None = None) -> np.ndarray:
    """Dequantize to float32 [B][S][H][D]; special positions (slot_of naming one of
    the n_special side slots, by default every row of p4) read their 4-bit slot."""
    if n_special is None:
        n_special = np.asarray(p4).shape[0]
    q3 = planes_decode(p3, D)
    out = (q3.astype(np.float32) * np.asarray(s3, dtype=np.float32)[..., None]).astype(np.float32)
    bs = np.argwhere(is_special(slot_of, n_special))
    if len(bs):
        slots = slot_of[bs[:, 0], bs[:, 1]]
        q4 = nibbles_decode(p4[slots])
        out[bs[:, 0], bs[:, 1]] = (q4.astype(np.float32) * s4[slots][..., None]).astype(np.float32)
    return out


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 to bf16 (round-half-to-even), returning the uint16 bit patterns."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)
