"""Pins for the oracle's ReLU^2 gate, top-k and INT8 sparse quantizer."""
import json
import os
from fractions import Fraction

import numpy as np
import pytest

from oracle import sparse8

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _g():
    with open(os.path.join(GOLD, "topk_int8_worked.json")) as f:
        return json.load(f)


def test_topk_worked_examples():
    for case in _g()["topk_cases"]:
        h = np.array([case["h"]], dtype=np.float32)
        keep = sparse8.topk_mask(h, case["k"])
        assert sorted(np.flatnonzero(keep[0]).tolist()) == case["keep"]


def test_int8_worked_example():
    c = _g()["int8_case"]
    h = np.array([c["h"]], dtype=np.float32)
    keep = sparse8.topk_mask(h, c["k"])
    assert np.flatnonzero(keep[0]).tolist() == c["keep"]
    q, s = sparse8.quantize_int8(h, keep)
    assert s[0] == np.float32(c["scale"]) and q[0].tolist() == c["codes"]


def test_fp32_tie_in_scaling():
    c = _g()["fp32_tie_case"]
    inv = np.float32(127) / np.float32(c["a"])
    exact = Fraction(float(inv)) * 3
    assert exact == 127 - Fraction(1, 2**18)
    h = np.array([[c["x"], 1.0, -2.0, 0.5]], dtype=np.float32)
    keep = np.ones_like(h, dtype=bool)
    q, _ = sparse8.quantize_int8(h, keep)
    assert q[0, 0] == c["expected_code"]


def test_topk_invariants_vs_stable_sort():
    rs = np.random.default_rng(20)
    # heavy ties: small integer magnitudes
    h = rs.integers(-3, 4, size=(40, 96)).astype(np.float32)
    for k in [1, 17, 48, 95, 96]:
        keep = sparse8.topk_mask(h, k)
        assert np.all(keep.sum(axis=1) == k)
        for m in range(40):
            order = sorted(range(96), key=lambda i: (-abs(float(h[m, i])), i))
            assert set(np.flatnonzero(keep[m]).tolist()) == set(order[:k])
            kept = np.abs(h[m][keep[m]])
            dropped = np.abs(h[m][~keep[m]])
            if dropped.size:
                assert kept.min() >= dropped.max()


def test_relu2_exact_for_bf16_inputs():
    rs = np.random.default_rng(21)
    g = rs.standard_normal((8, 64)).astype(np.float32)
    u = rs.standard_normal((8, 64)).astype(np.float32)
    # truncate to bf16 values (8 significant bits)
    g = (g.view(np.uint32) & 0xFFFF0000).view(np.float32)
    u = (u.view(np.uint32) & 0xFFFF0000).view(np.float32)
    h = sparse8.relu2_gate(g, u)
    for m in range(8):
        for k in range(64):
            r = max(Fraction(float(g[m, k])), Fraction(0))
            assert Fraction(float(h[m, k])) == r * r * Fraction(float(u[m, k]))


def test_sparse_a8_invariants_gaussian():
    rs = np.random.default_rng(22)
    gate = rs.standard_normal((16, 1024)).astype(np.float32)
    up = rs.standard_normal((16, 1024)).astype(np.float32)
    h, keep, q, s = sparse8.sparse_a8(gate, up, 512)
    assert np.all(keep.sum(axis=1) == 512)
    assert np.all(q[~keep] == 0)
    assert q.min() >= -127 and q.max() <= 127
    err = np.abs(np.where(keep, h, 0).astype(np.float64) - q * s[:, None].astype(np.float64))
    assert np.all(err <= s[:, None] * (0.5 + 2.0**-19))
    # dropped entries never exceed survivors
    for m in range(16):
        assert np.abs(h[m][keep[m]]).min() >= np.abs(h[m][~keep[m]]).max()


def test_k_equals_K_is_plain_int8_absmax():
    rs = np.random.default_rng(23)
    x = rs.standard_t(3, size=(4, 256)).astype(np.float32)
    h, keep, q, s = sparse8.sparse_a8(x, None, 256)
    assert keep.all()
    assert np.array_equal(s, np.abs(x).max(axis=1) / np.float32(127))


def test_mask_words_bit_order():
    keep = np.zeros((1, 64), dtype=bool)
    keep[0, [0, 5, 31, 32, 63]] = True
    w = sparse8.mask_words(keep)
    assert w[0].tolist() == [(1 << 0) | (1 << 5) | (1 << 31), 1 | (1 << 31)]


def test_bad_k():
    with pytest.raises(ValueError):
        sparse8.topk_mask(np.zeros((1, 4), np.float32), 0)
