"""Pins for the oracle's absmean ternary weights and the 2-bit packed layout."""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

from oracle import ternary

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def test_worked_example():
    with open(os.path.join(GOLD, "ternary_worked.json")) as f:
        g = json.load(f)
    w = np.array(g["w"], dtype=np.float32)
    t, b = ternary.quantize_weights(w)
    assert hex(np.float32(b).view(np.uint32)) == g["beta_f32_bits"]
    assert t.tolist() == g["codes"]


def test_beta_is_exact_mean_rounded():
    """beta equals the exact rational mean, rounded to fp64 then fp32 (Fraction arithmetic)."""
    rs = np.random.default_rng(5)
    for trial in range(5):
        w = (rs.standard_normal((16, 64)) * 10.0 ** rs.uniform(-6, 3, size=(16, 64))).astype(np.float32)
        exact = sum(Fraction(float(v)) for v in np.abs(w).ravel())
        s64 = float(exact)  # correctly rounded
        assert float(ternary.absmean_beta(w)) == float(np.float32(s64 / w.size))


def test_beta_cancellation_case():
    """A sum that naive fp32 accumulation gets wrong: one large value then many tiny ones."""
    w = np.full((16, 64), 2.0**-30, dtype=np.float32)
    w[0, 0] = 1.0
    exact = Fraction(1) + Fraction(1023, 2**30)
    assert float(ternary.absmean_beta(w)) == float(np.float32(float(exact) / 1024))


@pytest.mark.parametrize("j", [-10, -1, 4])
def test_beta_power_of_two_equivariance(j):
    rs = np.random.default_rng(6)
    w = (rs.standard_normal((32, 64)) * 0.02).astype(np.float32)
    t0, b0 = ternary.quantize_weights(w)
    t1, b1 = ternary.quantize_weights(w * np.float32(2.0**j))
    assert b1 == b0 * np.float32(2.0**j)
    assert np.array_equal(t0, t1)


def test_gaussian_zero_fraction_closed_form():
    """For W ~ N(0, sigma) the threshold beta/2 = sigma*sqrt(2/pi)/2, so
    P(t = 0) = 2*Phi(sqrt(2/pi)/2) - 1 = erf(1/(2*sqrt(pi))) ~ 0.3101."""
    rs = np.random.default_rng(7)
    w = (rs.standard_normal((1024, 1024)) * 0.02).astype(np.float32)
    t, _ = ternary.quantize_weights(w)
    p0 = math.erf(1.0 / (2.0 * math.sqrt(math.pi)))
    n = t.size
    frac0 = np.mean(t == 0)
    assert abs(frac0 - p0) < 5 * math.sqrt(p0 * (1 - p0) / n) + 1e-3
    assert abs(np.mean(t == 1) - np.mean(t == -1)) < 0.01
    assert set(np.unique(t).tolist()) <= {-1, 0, 1}


def test_all_equal_magnitude_gives_all_signs():
    w = np.where(np.arange(64 * 16).reshape(16, 64) % 3 == 0, -0.7, 0.7).astype(np.float32)
    t, b = ternary.quantize_weights(w)
    assert b == np.float32(0.7)
    assert np.array_equal(t, np.sign(w).astype(np.int8))


def test_zero_tensor():
    t, b = ternary.quantize_weights(np.zeros((16, 64), np.float32))
    assert b == np.float32(1e-5) and np.all(t == 0)


# The packed layout, restated as explicit tables (code slot -> input offset).
A4_TABLE = [0, 8, 1, 9, 2, 10, 3, 11, 4, 12, 5, 13, 6, 14, 7, 15]
A8_TABLE = [0, 4, 8, 12, 1, 5, 9, 13, 2, 6, 10, 14, 3, 7, 11, 15]


@pytest.mark.parametrize("role,table", [(ternary.ROLE_A4, A4_TABLE), (ternary.ROLE_A8, A8_TABLE)])
def test_pack_single_weight_positions(role, table):
    N, K = 32, 128
    for (n, k, v) in [(0, 0, 1), (0, 1, -1), (5, 17, 1), (16, 64, -1), (31, 127, 1), (7, 8, -1), (20, 100, 1)]:
        t = np.zeros((N, K), dtype=np.int8)
        t[n, k] = v
        p = ternary.pack(t, role)
        assert p.size == N * K // 4
        nb, c = divmod(n, 16)
        kb, r = divmod(k, 64)
        j, off = divmod(r, 16)
        slot = table.index(off)
        byte = (nb * (K // 64) + kb) * 256 + c * 16 + j * 4 + (2 * slot) // 8
        bit = (2 * slot) % 8
        expect = np.zeros_like(p)
        expect[byte] = (1 if v == 1 else 3) << bit
        assert np.array_equal(p, expect), (n, k, v)


@pytest.mark.parametrize("role", [ternary.ROLE_A4, ternary.ROLE_A8])
def test_pack_roundtrip(role):
    rs = np.random.default_rng(8)
    t = rs.integers(-1, 2, size=(48, 192)).astype(np.int8)
    p = ternary.pack(t, role)
    assert np.array_equal(ternary.unpack(p, 48, 192, role), t)
    # code 10 is never written
    b = p
    for sh in (0, 2, 4, 6):
        assert not np.any(((b >> sh) & 3) == 2)


def test_pack_kmajor_single_weight_positions():
    """K-major layout written out by hand: input k owns N/4 bytes, output n sits in
    word n // 16 at bits 2 * (n % 16), code t + 1 (so a zero weight is 01)."""
    N, K = 48, 128
    for (n, k, v) in [(0, 0, 1), (0, 1, -1), (5, 17, 1), (16, 64, -1), (47, 127, 1), (31, 8, -1), (20, 100, 0)]:
        t = np.zeros((N, K), dtype=np.int8)
        t[n, k] = v
        p = ternary.pack(t, ternary.ROLE_A8_KMAJOR)
        assert p.size == N * K // 4
        expect = np.full(N * K // 4, 0x55, dtype=np.uint8)  # every code 01 (t = 0)
        byte = k * (N // 4) + 4 * (n // 16) + (2 * (n % 16)) // 8
        bit = (2 * (n % 16)) % 8
        expect[byte] = (0x55 & ~(3 << bit)) | ((v + 1) << bit)
        assert np.array_equal(p, expect), (n, k, v)


def test_pack_kmajor_roundtrip_and_rows():
    rs = np.random.default_rng(18)
    t = rs.integers(-1, 2, size=(80, 192)).astype(np.int8)
    p = ternary.pack(t, ternary.ROLE_A8_KMAJOR)
    assert np.array_equal(ternary.unpack(p, 80, 192, ternary.ROLE_A8_KMAJOR), t)
    ks = [191, 0, 77, 77, 3]
    assert np.array_equal(ternary.kmajor_rows(p, 80, ks), t[:, ks].T)
    # code 11 is never written
    for sh in (0, 2, 4, 6):
        assert not np.any(((p >> sh) & 3) == 3)
