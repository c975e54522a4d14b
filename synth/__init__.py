"""Seeded synthetic workloads for the W1.58A4 / W1.58A8 BitLinear path.

This module is shared by the CPU oracle's tests and by the GPU side (tests,
bench).  It draws random numbers and stores them as fp32 or bf16; it holds
none of the method's arithmetic (no scale, rounding to a code grid, top-k,
packing or contraction).

Every generator takes a seed and returns host numpy arrays.  bf16 tensors are
returned as ``Bf16`` pairs: the raw uint16 bit patterns (what a device buffer
holds) and the same values widened to float32 (exact), so that both sides see
identical numbers.

Workload shapes follow the 7B Llama-like model the BitNet a4.8 pages describe
(hidden 4096, FFN 11008, 32 heads of 128): the q/k/v/gate/up inputs are drawn
near-Gaussian and the out/down inputs heavy-tailed, as the toshoseti review of
BitNet a4.8 («Метод» paragraph) reports from the authors' activation
histograms; a few outlier channels stand in for the outlier dimensions named
in the BitNet a4.8 abstract.
"""
from __future__ import annotations

import dataclasses

import numpy as np

SEED_BASE = 20241107

HIDDEN = 4096
FFN = 11008
HEADS = 32
HEAD_DIM = 128


@dataclasses.dataclass
class Bf16:
    bits: np.ndarray  # uint16, the bf16 bit patterns
    f32: np.ndarray  # float32, the same values (exact widening)

    @property
    def shape(self):
        return self.bits.shape


def rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


def to_bf16(x: np.ndarray) -> Bf16:
    """Round float32 values to bf16 (round-half-to-even on the dropped 16 bits)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    hi = ((u + 0x7FFF + lsb) >> 16).astype(np.uint16)
    f = (hi.astype(np.uint32) << 16).view(np.float32)
    return Bf16(bits=hi, f32=f)


def normal(seed: int, shape, sigma: float = 1.0) -> np.ndarray:
    return (rng(seed).standard_normal(size=shape, dtype=np.float32) * np.float32(sigma)).astype(np.float32)


# ---------------------------------------------------------------------------
# Single BitLinear, M=16, K=N=256, fp32 activations and weights.
# ---------------------------------------------------------------------------
def small_bitlinear(seed: int = SEED_BASE + 0, M: int = 16, K: int = 256, N: int = 256):
    g = rng(seed)
    x = g.standard_normal(size=(M, K), dtype=np.float32)
    w = (g.standard_normal(size=(N, K), dtype=np.float32) * np.float32(0.02)).astype(np.float32)
    return x, w


# ---------------------------------------------------------------------------
# Decode activations: bf16 N(0,1), 0.1 % of channels scaled x20 for every token.
# ---------------------------------------------------------------------------
def outlier_channels(seed: int, K: int, frac: float = 0.001) -> np.ndarray:
    n = max(1, int(round(frac * K)))
    return np.sort(rng(seed + 7919).choice(K, size=n, replace=False))


def decode_activations(seed: int = SEED_BASE + 1, M: int = 1, K: int = HIDDEN) -> Bf16:
    x = rng(seed).standard_normal(size=(M, K), dtype=np.float32)
    x[:, outlier_channels(seed, K)] *= np.float32(20.0)
    return to_bf16(x)


def weight_tensor(seed: int, N: int, K: int, sigma: float = 0.02) -> np.ndarray:
    """One fp32 weight tensor [N][K] (nn.Linear out x in), N(0, sigma)."""
    return normal(seed, (N, K), sigma)


def fused_weights(seed: int, parts, K: int, sigma: float = 0.02):
    """A list of separately-drawn weight tensors that a fused projection concatenates along N
    (q,k,v: three HIDDEN x HIDDEN; gate,up: two FFN x HIDDEN)."""
    return [weight_tensor(seed + 101 * i, n, K, sigma) for i, n in enumerate(parts)]


QKV_PARTS = (HIDDEN, HIDDEN, HIDDEN)
GATE_UP_PARTS = (FFN, FFN)


# ---------------------------------------------------------------------------
# Prefill activations: bf16 N(0,1) [M][K].
# ---------------------------------------------------------------------------
def prefill_activations(seed: int = SEED_BASE + 2, M: int = 2048, K: int = HIDDEN) -> Bf16:
    return to_bf16(rng(seed).standard_normal(size=(M, K), dtype=np.float32))


# ---------------------------------------------------------------------------
# Sparse path inputs: gate, up bf16 N(0,1) [M][FFN]; out_proj input Student-t(3).
# ---------------------------------------------------------------------------
def gate_up(seed: int = SEED_BASE + 3, M: int = 2048, K: int = FFN):
    g = rng(seed)
    gate = g.standard_normal(size=(M, K), dtype=np.float32)
    up = g.standard_normal(size=(M, K), dtype=np.float32)
    return to_bf16(gate), to_bf16(up)


def heavy_tailed(seed: int = SEED_BASE + 13, M: int = 2048, K: int = HIDDEN, df: float = 3.0) -> Bf16:
    t = rng(seed).standard_t(df, size=(M, K)).astype(np.float32)
    return to_bf16(t)


# ---------------------------------------------------------------------------
# KV cache: bf16 N(0,1) [B][S][H][D] times a per-head LogNormal(0,0.5) scale;
# token 0 (bos) and a seeded ~1 % of positions (eos) are the special tokens.
# ---------------------------------------------------------------------------
def kv_tensor(seed: int, B: int = 8, S: int = 4096, H: int = HEADS, D: int = HEAD_DIM) -> Bf16:
    g = rng(seed)
    sigma_h = g.lognormal(mean=0.0, sigma=0.5, size=H).astype(np.float32)
    x = g.standard_normal(size=(B, S, H, D), dtype=np.float32)
    x *= sigma_h[None, None, :, None]
    return to_bf16(x)


def kv_special_slots(seed: int, B: int = 8, S: int = 4096, frac: float = 0.01):
    """slot_of[B][S] (int32): -1 for ordinary tokens, else the index of the token's
    side-slab slot.  Position 0 of every sequence is special, plus round(frac*S)
    distinct seeded positions drawn from [1, S) per sequence."""
    g = rng(seed + 104729)
    slot_of = np.full((B, S), -1, dtype=np.int32)
    n_extra = int(round(frac * S)) if S > 1 else 0
    n_extra = min(n_extra, max(S - 1, 0))
    nxt = 0
    for b in range(B):
        pos = [0]
        if n_extra:
            pos += sorted(int(p) for p in g.choice(np.arange(1, S), size=n_extra, replace=False))
        for p in pos:
            slot_of[b, p] = nxt
            nxt += 1
    return slot_of, nxt
