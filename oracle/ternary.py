"""Absmean ternary weights and their 2-bit packing (oracle; test infrastructure).

toshoseti review, opening lines: BitNet b1.58 replaced binary weights with
ternary ones {-1, 0, +1}; BitNet a4.8 keeps those weights (its abstract calls
the model a 1-bit LLM and compares it with b1.58).

Readings (the pages give no formula):
* one scale per weight tensor, beta = mean |W|, computed as
  fp32( fp64(sum |w|) / (N*K) ) where fp64(sum) is the exact sum of the fp32
  magnitudes rounded once to fp64 (``math.fsum``) -- an order-free definition;
* beta' = max(beta, 1e-5); t = RoundClip(w / beta', -1, 1) with ties to even,
  which for exact arithmetic is t = sign(w) * [2|w| > beta'] (a value exactly
  half of beta' rounds to 0); 2|w| is exact in fp32, so no division is rounded.

Packed layout (version 1): 2 bits per weight, code 00 = 0, 01 = +1, 11 = -1.
The logical [N][K] tensor (nn.Linear out x in) is cut into tiles of 16 output
channels x 64 inputs, 256 bytes each, stored tile-row-major:
byte offset of tile (nb, kb) = (nb * K/64 + kb) * 256.  Inside a tile, output
channel c (0..15) owns bytes [16c, 16c+16): four little-endian uint32 words,
word j covering inputs k = 64*kb + 16*j + (0..15).  Code i of a word sits at
bits [2i, 2i+2); which of the 16 inputs it holds depends on the role of the
weight:
* ROLE_A4 (q/k/v/gate/up, meeting 4-bit activations): code i holds input
  offset (8 if i is odd else 0) + i // 2;
* ROLE_A8 (out/down, meeting 8-bit activations): code i holds input offset
  4 * (i % 4) + i // 4.
"""
from __future__ import annotations

import itertools
import math

import numpy as np

EPS = np.float32(1e-5)

ROLE_A4 = 0
ROLE_A8 = 1
ROLE_A8_KMAJOR = 2

TILE_N = 16
TILE_K = 64
TILE_BYTES = 256


def absmean_beta(w: np.ndarray) -> np.float32:
    """beta = fp32(fp64(exact sum |w|) / (N*K)) for one weight tensor (not clamped)."""
    w = np.ascontiguousarray(w, dtype=np.float32).reshape(-1)
    n = w.size
    chunks = (np.abs(w[i : i + (1 << 22)]).astype(np.float64).tolist() for i in range(0, n, 1 << 22))
    total = math.fsum(itertools.chain.from_iterable(chunks))
    return np.float32(total / float(n))


def ternarize(w: np.ndarray, beta_clamped: np.float32) -> np.ndarray:
    """t = sign(w) * [2|w| > beta'] as int8 in {-1, 0, 1}."""
    w = np.ascontiguousarray(w, dtype=np.float32)
    keep = (np.abs(w) * np.float32(2.0)) > np.float32(beta_clamped)
    return (np.sign(w).astype(np.int8) * keep.astype(np.int8)).astype(np.int8)


def quantize_weights(w: np.ndarray):
    """Absmean ternary weights of one tensor: (t int8 [N][K], beta' float32)."""
    b = max(absmean_beta(w), EPS)
    b = np.float32(b)
    return ternarize(w, b), b


def code_offsets(role: int) -> np.ndarray:
    """offsets[i] = input offset (0..15) held by code i of a packed word."""
    i = np.arange(16)
    if role == ROLE_A4:
        return np.where(i % 2 == 1, 8, 0) + i // 2
    if role == ROLE_A8:
        return 4 * (i % 4) + i // 4
    raise ValueError(f"unknown role {role}")


def _pack_kmajor(t: np.ndarray) -> np.ndarray:
    N, K = t.shape
    code = (t.T.astype(np.int64) + 1).astype(np.uint64)  # [K][N], t + 1
    grp = code.reshape(K, N // 16, 16)  # [k][g][i], output n = 16g + i
    shifts = (2 * np.arange(16)).astype(np.uint64)
    words = (grp << shifts).sum(axis=-1).astype(np.uint32)  # [k][g]
    return np.ascontiguousarray(words).astype("<u4").view(np.uint8).reshape(-1)


def kmajor_rows(packed: np.ndarray, N: int, ks) -> np.ndarray:
    """Rows t[:, k] for the inputs ks of a K-major packed tensor: int8 [len(ks)][N].
    Only the N/4 bytes of each listed input are read."""
    packed = np.ascontiguousarray(packed, dtype=np.uint8)
    ks = np.asarray(ks, dtype=np.int64)
    row_bytes = N // 4
    rows = np.stack([packed[k * row_bytes : (k + 1) * row_bytes] for k in ks]) if ks.size else (
        np.zeros((0, row_bytes), np.uint8))
    words = rows.view("<u4").astype(np.uint64)  # [len][N/16]
    shifts = (2 * np.arange(16)).astype(np.uint64)
    code = ((words[..., None] >> shifts) & 3).astype(np.int8)  # [len][g][i]
    return (code - 1).reshape(len(ks), N)  # code 11 would decode as 2, never written


def pack(t: np.ndarray, role: int) -> np.ndarray:
    """Pack ternary int8 [N][K] into the layout of `role`; returns uint8 [N*K/4]."""
    t = np.asarray(t)
    N, K = t.shape
    if N % TILE_N or K % TILE_K:
        raise ValueError("N must be a multiple of 16 and K of 64")
    if role == ROLE_A8_KMAJOR:
        return _pack_kmajor(t)
    code = np.where(t == 1, 1, np.where(t == -1, 3, 0)).astype(np.uint64)
    # [nb][c][kb][j][off]
    c5 = code.reshape(N // TILE_N, TILE_N, K // TILE_K, 4, 16)
    held = c5[..., code_offsets(role)]  # [..., i] = code of the input held by code slot i
    shifts = (2 * np.arange(16)).astype(np.uint64)
    words = (held << shifts).sum(axis=-1).astype(np.uint32)  # [nb][c][kb][j]
    words = words.transpose(0, 2, 1, 3)  # [nb][kb][c][j]
    return np.ascontiguousarray(words).astype("<u4").view(np.uint8).reshape(-1)


def unpack(packed: np.ndarray, N: int, K: int, role: int) -> np.ndarray:
    """Inverse of pack: uint8 [N*K/4] -> int8 [N][K] (code 10 decodes as -2, never written;
    in the K-major layout code 11 decodes as 2, never written)."""
    if role == ROLE_A8_KMAJOR:
        return np.ascontiguousarray(kmajor_rows(packed, N, np.arange(K)).T)
    words = np.ascontiguousarray(packed, dtype=np.uint8).view("<u4").astype(np.uint64)
    words = words.reshape(N // TILE_N, K // TILE_K, TILE_N, 4).transpose(0, 2, 1, 3)
    shifts = (2 * np.arange(16)).astype(np.uint64)
    held = ((words[..., None] >> shifts) & 3).astype(np.int8)  # [nb][c][kb][j][i]
    val = np.where(held >= 2, held - 4, held).astype(np.int8)
    out = np.empty_like(val)
    out[..., code_offsets(role)] = val
    return out.reshape(N, K)
