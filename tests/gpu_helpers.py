"""Helpers for the GPU parity tests: host<->device transfer and comparisons."""
from __future__ import annotations

import numpy as np
import torch

DEV = "cuda:0"


def bf16_dev(b) -> torch.Tensor:
    """synth.Bf16 -> torch.bfloat16 device tensor with identical bits."""
    return torch.from_numpy(np.ascontiguousarray(b.bits).view(np.int16)).to(DEV).view(torch.bfloat16)


def f32_dev(x: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(DEV)


def host(t: torch.Tensor) -> np.ndarray:
    torch.cuda.synchronize()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def assert_rel(y_gpu: np.ndarray, y_ref: np.ndarray, rtol: float = 1e-5, what: str = "y"):
    """|y_gpu - y_ref| <= rtol * |y_ref| elementwise (so y_ref == 0 demands an exact 0)."""
    y_gpu = np.asarray(y_gpu, dtype=np.float64)
    y_ref = np.asarray(y_ref, dtype=np.float64)
    err = np.abs(y_gpu - y_ref)
    bad = err > rtol * np.abs(y_ref)
    if bad.any():
        idx = np.argwhere(bad)[:5]
        raise AssertionError(
            f"{what}: {int(bad.sum())} of {bad.size} outside rtol={rtol}; first {idx.tolist()}: "
            f"gpu {[y_gpu[tuple(i)] for i in idx]} ref {[y_ref[tuple(i)] for i in idx]}"
        )


def assert_same(a: np.ndarray, b: np.ndarray, what: str):
    a = np.asarray(a)
    b = np.asarray(b)
    if a.shape != b.shape:
        raise AssertionError(f"{what}: shape {a.shape} vs {b.shape}")
    if not np.array_equal(a, b):
        bad = np.argwhere(a != b)
        raise AssertionError(
            f"{what}: {len(bad)} of {a.size} differ; first {bad[:5].tolist()}: "
            f"gpu {[a[tuple(i)] for i in bad[:5]]} ref {[b[tuple(i)] for i in bad[:5]]}"
        )


U = 2.0**-24


def gamma(n):
    return n * U / (1 - n * U)


def attn_bound(qd: np.ndarray, kd: np.ndarray, vd: np.ndarray, p: np.ndarray) -> np.ndarray:
    """First-order rounding bound [D] on one fp32 single-token attention output
    (fixed-point query, integer dot products, fp32 softmax and value sums) against
    the exact evaluation over the same dequantized cache.  qd [D], kd / vd [S][D]
    the dequantized keys / values (fp64), p [S] the exact softmax weights.  With
    u = 2^-24 and gamma_n = n u / (1 - n u):
      score error  E_z = max_s [gamma_D sum_d |q_d k_sd| + 2^-31 max|q| sum_d |k_sd|
                               + 2^-23 max|q| s_s] / sqrt(D) + 4u |z_s|
    (the second term is the query rounded to multiples of 2^-30 max|q| for the
    integer dot products, the third the two fp32 roundings of the exact integer
    sum at the position's scale s_s = max|k_s| / 3),
      weight error E_p = 2 E_z + gamma_S + 2u,
      |out_d - ref_d| <= (E_p + gamma_S + 2u) sum_s p_s |v_sd|  (+ 1e-30)."""
    S, D = kd.shape
    z = kd @ qd / np.sqrt(D)
    s_pos = np.abs(kd).max(axis=1) / 3.0 + 1e-30
    fixed = 2.0**-31 * np.abs(qd).max() * np.abs(kd).sum(axis=1) + 2.0**-23 * np.abs(qd).max() * s_pos
    e_z = np.max((gamma(D) * (np.abs(kd) @ np.abs(qd)) + fixed) / np.sqrt(D) + 4 * U * np.abs(z))
    e_p = 2 * e_z + gamma(S) + 2 * U
    return (e_p + gamma(S) + 2 * U) * (p @ np.abs(vd)) + 1e-30
