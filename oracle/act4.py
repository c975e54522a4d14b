"""4-bit activation quantizers (oracle; test infrastructure).

BitNet a4.8 abstract: the inputs of the attention and FFN projections carry
4-bit activations, run through INT4 or FP4 kernels.  toshoseti review, «Метод»:
only the q/k/v/gate/up group is quantized to 4 bits (its activations are close
to Gaussian), and FP4 is considered beside INT4 for its wider dynamic range.

Readings (the pages give no formula):
* one scale per token (row), from the row's absolute maximum, the activation
  scale the review attributes to BitNet b1.58 (absmax);
* INT4: inv = fl(7 / a'), s = fl(a' / 7), q = clamp(rne(fl(x * inv)), -8, 7),
  a' = max(max|x|, 1e-5); absmax never clips, so codes stay in [-7, 7];
* FP4 is the e2m1 format (magnitudes 0, .5, 1, 1.5, 2, 3, 4, 6) with
  inv = fl(6 / a'), s = fl(a' / 6); t = fl(x * inv) goes to the nearest grid
  magnitude, ties to the even code (mantissa bit 0), saturating at 6, sign bit
  copied from t;
* packed storage: two codes per byte, the even k in the low nibble.
* a second storage of the same INT4 values (not from the pages: the operand
  format of the fp6 matrix instructions): each value q as a 6-bit e2m3 field
  (sign bit, then |q| in five bits, which the OCP Microscaling e2m3 format -
  1 sign, 2 exponent bits with bias 1, 3 mantissa bits, subnormals - reads as
  q/8); per 64 values, the 24-byte little-endian bit streams S0 (values 0..31)
  and S1 (values 32..63) are stored as S0[0:16], S1[0:16], S0[16:24],
  S1[16:24].
"""
from __future__ import annotations

import numpy as np

EPS = np.float32(1e-5)

E2M1_MAGNITUDES = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0], dtype=np.float64)


def _f32(x) -> np.ndarray:
    return np.ascontiguousarray(x, dtype=np.float32)


def row_absmax(x: np.ndarray) -> np.ndarray:
    """a' = max(max_k |x[m,k]|, 1e-5) per row, fp32 (exact: max is order-free)."""
    return np.maximum(np.abs(_f32(x)).max(axis=1), EPS)


def quantize_int4(x: np.ndarray):
    """Per-token absmax INT4 codes and scales.

    Returns (codes int8 [M][K] in [-8, 7], scales float32 [M]) such that
    x ~= codes * scales[:, None].
    """
    x = _f32(x)
    a = row_absmax(x)
    inv = np.float32(7.0) / a
    s = a / np.float32(7.0)
    t = x * inv[:, None]
    q = np.clip(np.rint(t), -8, 7).astype(np.int8)
    return q, s.astype(np.float32)


def e2m1_encode(t: np.ndarray) -> np.ndarray:
    """Nearest e2m1 code (0..15) of each fp32 value: brute-force search over the
    eight magnitudes, ties to the even code index, sign bit = sign bit of t."""
    t = _f32(t)
    out = np.empty(t.shape, dtype=np.uint8)
    flat_t = t.reshape(-1)
    flat_o = out.reshape(-1)
    even = (np.arange(8) % 2) == 0
    step = 1 << 20
    for lo in range(0, flat_t.size, step):
        tt = flat_t[lo : lo + step]
        mag = np.minimum(np.abs(tt.astype(np.float64)), 6.0)
        d = np.abs(mag[:, None] - E2M1_MAGNITUDES[None, :])
        best = d == d.min(axis=1, keepdims=True)
        pick_even = best & even[None, :]
        idx = np.where(pick_even.any(axis=1), np.argmax(pick_even, axis=1), np.argmax(best, axis=1))
        flat_o[lo : lo + step] = idx.astype(np.uint8) | (np.signbit(tt).astype(np.uint8) << 3)
    return out


def e2m1_decode(codes: np.ndarray) -> np.ndarray:
    """Value of each e2m1 code (float64, exact)."""
    c = np.asarray(codes, dtype=np.uint8)
    v = E2M1_MAGNITUDES[c & 7]
    return np.where((c & 8) != 0, -v, v)


def quantize_fp4(x: np.ndarray):
    """Per-token absmax e2m1 codes (uint8 [M][K], 0..15) and scales float32 [M]."""
    x = _f32(x)
    a = row_absmax(x)
    inv = np.float32(6.0) / a
    s = a / np.float32(6.0)
    t = x * inv[:, None]
    return e2m1_encode(t), s.astype(np.float32)


def pack_nibbles(codes: np.ndarray) -> np.ndarray:
    """[M][K] 4-bit codes (two's complement int or 0..15) -> uint8 [M][K/2], even k in the low nibble."""
    c = np.asarray(codes).astype(np.int16) & 0xF
    assert c.shape[-1] % 2 == 0
    lo = c[..., 0::2]
    hi = c[..., 1::2]
    return (lo | (hi << 4)).astype(np.uint8)


def unpack_nibbles(packed: np.ndarray, signed: bool) -> np.ndarray:
    """Inverse of pack_nibbles; signed=True sign-extends the 4-bit two's complement codes."""
    p = np.asarray(packed, dtype=np.uint8)
    out = np.empty(p.shape[:-1] + (p.shape[-1] * 2,), dtype=np.int16)
    out[..., 0::2] = p & 0xF
    out[..., 1::2] = p >> 4
    if signed:
        out = np.where(out >= 8, out - 16, out)
    return out.astype(np.int8) if signed else out.astype(np.uint8)


def e2m3_fields(q: np.ndarray) -> np.ndarray:
    """6-bit field of each INT4 value: (q < 0) << 5 | |q| (uint8)."""
    q = np.asarray(q).astype(np.int16)
    assert q.min(initial=0) >= -15 and q.max(initial=0) <= 15
    return (((q < 0).astype(np.int16) << 5) | np.abs(q)).astype(np.uint8)


def pack_int4_e2m3(q: np.ndarray) -> np.ndarray:
    """[M][K] INT4 values (K % 64 == 0) -> uint8 [M][3K/4] in the e2m3 storage.

    Four fields f0..f3 make 24 bits f0 | f1 << 6 | f2 << 12 | f3 << 18, three
    little-endian bytes; eight such runs form the 24-byte stream of 32 values."""
    q = np.asarray(q)
    M, K = q.shape
    assert K % 64 == 0
    f = e2m3_fields(q).astype(np.uint32).reshape(M, K // 64, 2, 8, 4)
    run = f[..., 0] | (f[..., 1] << 6) | (f[..., 2] << 12) | (f[..., 3] << 18)
    stream = np.stack([run & 0xFF, (run >> 8) & 0xFF, run >> 16], axis=-1).astype(np.uint8)
    stream = stream.reshape(M, K // 64, 2, 24)  # [row][group][S0/S1][byte]
    group = np.concatenate([stream[:, :, 0, :16], stream[:, :, 1, :16], stream[:, :, 0, 16:], stream[:, :, 1, 16:]],
                           axis=-1)
    return np.ascontiguousarray(group.reshape(M, K // 64 * 48))


def e2m3_value(f: np.ndarray) -> np.ndarray:
    """Value of each 6-bit e2m3 field (float64): sign bit 5, exponent bits 4..3
    (bias 1), mantissa bits 2..0; exponent 0 is subnormal (mantissa / 8)."""
    f = np.asarray(f).astype(np.int64)
    sign = np.where((f >> 5) & 1, -1.0, 1.0)
    e = (f >> 3) & 3
    m = (f & 7).astype(np.float64)
    mag = np.where(e == 0, m / 8.0, np.exp2(e - 1.0) * (1.0 + m / 8.0))
    return sign * mag


def unpack_int4_e2m3(packed: np.ndarray, K: int) -> np.ndarray:
    """Inverse of pack_int4_e2m3 by another route: the group's bytes back into
    the two streams, the streams into bits (numpy's little-endian bit order),
    six bits per field, and each field's e2m3 value times 8."""
    p = np.asarray(packed, dtype=np.uint8)
    M = p.shape[0]
    g = p.reshape(M, K // 64, 48)
    s0 = np.concatenate([g[:, :, 0:16], g[:, :, 32:40]], axis=-1)
    s1 = np.concatenate([g[:, :, 16:32], g[:, :, 40:48]], axis=-1)
    streams = np.stack([s0, s1], axis=2)  # [M][groups][2][24]
    bits = np.unpackbits(streams, axis=-1, bitorder="little").reshape(M, K // 64, 2, 32, 6)
    fields = (bits.astype(np.int64) << np.arange(6)).sum(axis=-1)
    v = e2m3_value(fields) * 8.0
    q = np.rint(v)
    assert np.array_equal(q, v), "field is not an integer multiple of 1/8"
    return q.reshape(M, K).astype(np.int8)
