"""Pins for the oracle's contractions and epilogue."""
from fractions import Fraction

import numpy as np

from oracle import act4, bitlinear, ternary


def test_contract_brute_force_loops():
    rs = np.random.default_rng(10)
    q = rs.integers(-8, 8, size=(3, 20))
    t = rs.integers(-1, 2, size=(5, 20))
    acc = bitlinear.contract(q, t)
    for m in range(3):
        for n in range(5):
            s = 0
            for k in range(20):
                s += int(q[m, k]) * int(t[n, k])
            assert acc[m, n] == s


def test_contract_special_weights():
    rs = np.random.default_rng(11)
    q = rs.integers(-127, 128, size=(4, 64))
    ones = np.ones((3, 64), dtype=np.int8)
    assert np.array_equal(bitlinear.contract(q, ones), np.repeat(q.sum(axis=1)[:, None], 3, axis=1))
    assert np.all(bitlinear.contract(q, -ones) == -bitlinear.contract(q, ones))
    assert np.all(bitlinear.contract(q, np.zeros((3, 64), np.int8)) == 0)
    # additivity over disjoint supports
    t = rs.integers(-1, 2, size=(3, 64)).astype(np.int8)
    sel = rs.integers(0, 2, size=(3, 64)).astype(bool)
    t1 = np.where(sel, t, 0)
    t2 = np.where(sel, 0, t)
    assert np.array_equal(bitlinear.contract(q, t), bitlinear.contract(q, t1) + bitlinear.contract(q, t2))


def test_e2m1_contraction_exact_fractions():
    rs = np.random.default_rng(12)
    codes = rs.integers(0, 16, size=(2, 32)).astype(np.uint8)
    t = rs.integers(-1, 2, size=(3, 32))
    d = bitlinear.contract_e2m1_doubled(codes, t)
    table = {0: 0, 1: Fraction(1, 2), 2: 1, 3: Fraction(3, 2), 4: 2, 5: 3, 6: 4, 7: 6}
    for m in range(2):
        for n in range(3):
            s = Fraction(0)
            for k in range(32):
                c = int(codes[m, k])
                v = table[c & 7] * (-1 if c & 8 else 1)
                s += v * int(t[n, k])
            assert Fraction(int(d[m, n]), 2) == s


def test_epilogue_and_zero():
    acc = np.array([[0, 3], [-5, 7]])
    s = np.array([0.5, 2.0], dtype=np.float32)
    b = np.array([0.25, 4.0], dtype=np.float32)
    y = bitlinear.epilogue(acc, s, b)
    assert y.tolist() == [[0.0, 6.0], [-2.5, 56.0]]


def test_end_to_end_small_matches_float_reference():
    """Dequantized y approximates the float product x @ W^T (loose, statistical)."""
    rs = np.random.default_rng(13)
    x = rs.standard_normal((16, 256)).astype(np.float32)
    w = (rs.standard_normal((64, 256)) * 0.02).astype(np.float32)
    t, b = ternary.quantize_weights(w)
    _, _, acc, y = bitlinear.bitlinear_a4_int4(x, t, np.full(64, b, np.float32))
    ref = x.astype(np.float64) @ (t.astype(np.float64) * float(b)).T
    rel = np.linalg.norm(y - ref) / np.linalg.norm(ref)
    assert rel < 0.2
    # acc bound |acc| <= 7*K
    assert np.abs(acc).max() <= 7 * 256
    c, s, acc4, y4 = bitlinear.bitlinear_a4_fp4(x, t, np.full(64, b, np.float32))
    rel4 = np.linalg.norm(y4 - ref) / np.linalg.norm(ref)
    assert rel4 < 0.2
    assert np.all(acc4 * 2 == np.rint(acc4 * 2))
    q, _ = act4.quantize_int4(x)
    assert np.array_equal(bitlinear.contract(q, t), acc)


def test_gather_kmajor_matches_dense_and_brute_force():
    """The row-gather product over K-major weights equals the dense contraction
    (tiny case also by explicit loops), for sparse, empty and full code rows."""
    rs = np.random.default_rng(21)
    N, K = 32, 128
    t = rs.integers(-1, 2, size=(N, K)).astype(np.int8)
    q = rs.integers(-128, 128, size=(4, K)).astype(np.int64)
    q[0, rs.permutation(K)[: K // 2]] = 0  # half dropped
    q[1] = 0  # every input dropped
    q[2, ::3] = 0
    p = ternary.pack(t, ternary.ROLE_A8_KMAJOR)
    acc = bitlinear.contract_gather_kmajor(q, p, N)
    assert np.array_equal(acc, bitlinear.contract(q, t))
    assert not acc[1].any()
    for m in (0, 3):
        for n in (0, 7, 31):
            assert acc[m, n] == sum(int(q[m, k]) * int(t[n, k]) for k in range(K))
