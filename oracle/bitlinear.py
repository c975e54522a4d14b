"""BitLinear contractions and the dequant epilogue (oracle; test infrastructure).

BitNet a4.8 abstract: ternary-weight layers multiply 4-bit activations (the
inputs of attention and FFN, INT4 or FP4 kernels) and 8-bit activations (the
sparsified intermediate states).  shd-paper.top summary, 方法详解: the same two
activation paths feed the same ternary layers.

Definitions:
* acc[m][n] = sum_k q[m][k] * t[n][k], an exact integer (INT4 and INT8 codes);
* for e2m1 codes the sum of e2m1(q) * t is a multiple of 1/2, computed here as
  an exact integer sum of doubled values, then halved;
* y[m][n] = acc[m][n] * s[m] * beta'[n] (reading: per-token scale times
  per-channel weight scale, evaluated here in fp64).
"""
from __future__ import annotations

import numpy as np

from . import act4, ternary


def _exact_int_matmul(a: np.ndarray, b_t: np.ndarray) -> np.ndarray:
    """a @ b_t^T for integer matrices, returned as int64.  Computed with an fp64
    matmul, which is exact whatever the summation order because every product
    and partial sum is an integer of magnitude at most max|a| * max|b| * K,
    checked here to stay below 2^53."""
    a = np.asarray(a)
    b_t = np.asarray(b_t)
    K = a.shape[1]
    bound = float(np.abs(a).max(initial=0)) * float(np.abs(b_t).max(initial=0)) * K
    if bound >= 2.0**53:
        raise ValueError("integer contraction too large for exact fp64 evaluation")
    return (a.astype(np.float64) @ b_t.astype(np.float64).T).astype(np.int64)


def contract(q: np.ndarray, t: np.ndarray) -> np.ndarray:
    """acc = q @ t^T as exact integers (q [M][K] ints, t [N][K] ternary), int64."""
    return _exact_int_matmul(q, t)


def contract_e2m1_doubled(codes: np.ndarray, t: np.ndarray) -> np.ndarray:
    """2 * sum_k e2m1(codes[m][k]) * t[n][k] as exact int64 (doubled values are integers)."""
    twice = np.rint(2.0 * act4.e2m1_decode(codes)).astype(np.int64)
    return _exact_int_matmul(twice, t)


def epilogue(acc: np.ndarray, s_x: np.ndarray, beta: np.ndarray) -> np.ndarray:
    """y = acc * s_x[m] * beta[n] in fp64."""
    return (
        np.asarray(acc, dtype=np.float64)
        * np.asarray(s_x, dtype=np.float64)[:, None]
        * np.asarray(beta, dtype=np.float64)[None, :]
    )


def bitlinear_a4_int4(x: np.ndarray, t: np.ndarray, beta: np.ndarray):
    """INT4 activations x ternary weights: returns (codes, s_x, acc, y)."""
    q, s = act4.quantize_int4(x)
    acc = contract(q, t)
    return q, s, acc, epilogue(acc, s, beta)


def bitlinear_a4_fp4(x: np.ndarray, t: np.ndarray, beta: np.ndarray):
    """e2m1 activations x ternary weights: returns (codes, s_x, acc (fp64, exact), y)."""
    c, s = act4.quantize_fp4(x)
    acc = contract_e2m1_doubled(c, t).astype(np.float64) / 2.0
    return c, s, acc, epilogue(acc, s, beta)


def contract_gather_kmajor(codes: np.ndarray, packed_kmajor: np.ndarray, N: int) -> np.ndarray:
    """acc[m][n] = sum over the inputs k with codes[m][k] != 0 of codes[m][k] * t[n][k],
    reading from the K-major packed weights only the rows of those inputs (the
    single-token decode product on sparsified 8-bit codes; BitNet a4.8 abstract,
    55 % of the parameters active).  Dropped inputs add nothing, so this equals
    contract(codes, t).  Returns int64 [M][N]."""
    codes = np.asarray(codes)
    M = codes.shape[0]
    acc = np.zeros((M, N), dtype=np.int64)
    for m in range(M):
        ks = np.flatnonzero(codes[m])
        rows = ternary.kmajor_rows(packed_kmajor, N, ks)  # [len][N]
        acc[m] = _exact_int_matmul(codes[m, ks][None, :], rows.T)[0]
    return acc
