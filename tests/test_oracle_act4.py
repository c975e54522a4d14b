"""Pins for the oracle's 4-bit activation quantizers (INT4 absmax, FP4 e2m1)."""
import json
import os
from fractions import Fraction

import numpy as np
import pytest

from oracle import act4

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


def test_int4_worked_example():
    g = _load("int4_worked.json")
    x = np.array([g["x"]], dtype=np.float32)
    q, s = act4.quantize_int4(x)
    assert s[0] == np.float32(g["scale"])
    assert q[0].tolist() == g["codes"]
    assert act4.pack_nibbles(q)[0].tolist() == g["bytes"]


def test_int4_invariants_random():
    rs = np.random.default_rng(1)
    x = rs.standard_normal((64, 256)).astype(np.float32) * rs.lognormal(0, 2, size=(64, 1)).astype(np.float32)
    q, s = act4.quantize_int4(x)
    assert q.min() >= -7 and q.max() <= 7  # absmax never reaches -8
    # the row maximum maps to +/-7
    am = np.argmax(np.abs(x), axis=1)
    assert np.all(np.abs(q[np.arange(64), am]) == 7)
    # the code is the nearest integer to x/s: error <= s/2 (tiny slack for the rounding of inv and s)
    err = np.abs(x.astype(np.float64) - q.astype(np.float64) * s[:, None].astype(np.float64))
    assert np.all(err <= s[:, None].astype(np.float64) * (0.5 + 2.0**-19))
    # nibbles round-trip
    assert np.array_equal(act4.unpack_nibbles(act4.pack_nibbles(q), signed=True), q)


@pytest.mark.parametrize("j", [-10, -3, 1, 5, 30])  # row max stays above the 1e-5 clamp
def test_int4_power_of_two_equivariance(j):
    rs = np.random.default_rng(2)
    x = rs.standard_normal((8, 128)).astype(np.float32)
    q0, s0 = act4.quantize_int4(x)
    q1, s1 = act4.quantize_int4(x * np.float32(2.0**j))
    assert np.array_equal(q0, q1)
    assert np.array_equal(s1, s0 * np.float32(2.0**j))


def test_int4_zero_row_and_constant_row():
    x = np.zeros((2, 64), dtype=np.float32)
    x[1, :] = -3.25
    q, s = act4.quantize_int4(x)
    assert np.all(q[0] == 0) and s[0] == np.float32(1e-5) / np.float32(7)
    assert np.all(q[1] == -7)


def test_int4_exact_rational_nearest():
    """Against exact rational arithmetic: with inv = fl(7/a'), fl(x*inv) is the
    correctly-rounded product, and q is its nearest integer (ties to even)."""
    rs = np.random.default_rng(3)
    x = rs.standard_normal((4, 64)).astype(np.float32)
    q, s = act4.quantize_int4(x)
    a = np.abs(x).max(axis=1)
    for m in range(4):
        inv = np.float32(7) / a[m]
        for k in range(64):
            exact = Fraction(float(x[m, k])) * Fraction(float(inv))
            t = float(np.float32(float(exact)))  # one correct fp32 rounding (float64 is exact here)
            assert abs(Fraction(t) - exact) <= abs(Fraction(float(np.spacing(np.float32(t))))) / 2
            assert q[m, k] == round(t)  # Python round: half to even


def test_fp4_worked_example():
    g = _load("fp4_worked.json")
    x = np.array([g["x"]], dtype=np.float32)
    c, s = act4.quantize_fp4(x)
    assert s[0] == np.float32(g["scale"])
    assert c[0].tolist() == g["codes"]


def _fp4_by_thresholds(t):
    """Independent formulation: count the midpoints that |t| passes; at a midpoint the
    lower neighbour wins when it has the even code, the upper one otherwise."""
    mag = np.abs(t.astype(np.float64))
    mids = [(0.25, False), (0.75, True), (1.25, False), (1.75, True), (2.5, False), (3.5, True), (5.0, False)]
    code = np.zeros(t.shape, dtype=np.int32)
    for mid, upper_even in mids:
        code += (mag >= mid) if upper_even else (mag > mid)
    return (code | (np.signbit(t).astype(np.int32) << 3)).astype(np.uint8)


def test_fp4_all_bf16_patterns_and_near_midpoints():
    bits = np.arange(1 << 16, dtype=np.uint32) << 16
    t = bits.view(np.float32)
    t = t[np.isfinite(t)]
    assert np.array_equal(act4.e2m1_encode(t), _fp4_by_thresholds(t))
    near = []
    for mid in [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0, 0.0]:
        c = np.float32(mid).view(np.int32)
        near.append((np.arange(-64, 65, dtype=np.int32) + c).view(np.float32))
    t2 = np.concatenate(near)
    t2 = np.concatenate([t2, -t2])
    t2 = t2[np.isfinite(t2)]
    assert np.array_equal(act4.e2m1_encode(t2), _fp4_by_thresholds(t2))


def test_fp4_dense_sweep_of_fp32_range():
    # every 97th fp32 bit pattern in [0, 8): ~11k values per binade
    lo = np.float32(0).view(np.uint32)
    hi = np.float32(8).view(np.uint32)
    t = np.arange(lo, hi, 97, dtype=np.uint32).view(np.float32)
    t = np.concatenate([t, -t])
    assert np.array_equal(act4.e2m1_encode(t), _fp4_by_thresholds(t))


def test_fp4_decode_and_error_bound():
    rs = np.random.default_rng(4)
    x = rs.standard_normal((32, 128)).astype(np.float32)
    c, s = act4.quantize_fp4(x)
    v = act4.e2m1_decode(c)
    assert np.all(np.abs(v) <= 6)
    am = np.argmax(np.abs(x), axis=1)
    assert np.all(np.abs(v[np.arange(32), am]) == 6)
    # grid spacing near t is at most 2 (between 4 and 6): |t - v| <= half the local gap
    t = (x * (np.float32(6) / np.abs(x).max(axis=1))[:, None]).astype(np.float64)
    gap = np.where(np.abs(t) < 2, 0.5, np.where(np.abs(t) < 4, 1.0, 2.0))
    assert np.all(np.abs(t - v) <= gap / 2 + 1e-12)


# ---- INT4 values stored as e2m3 fields (operand of the fp6 matrix instructions)

def test_e2m3_worked_group():
    g = _load("int4_e2m3_worked.json")
    q = np.zeros((1, 64), dtype=np.int8)
    for k, v in g["q_nonzero"].items():
        q[0, int(k)] = v
    want = np.zeros(48, dtype=np.uint8)
    for k, v in g["bytes_nonzero"].items():
        want[int(k)] = v
    assert act4.pack_int4_e2m3(q)[0].tolist() == want.tolist()
    assert np.array_equal(act4.unpack_int4_e2m3(act4.pack_int4_e2m3(q), 64), q)


def test_e2m3_value_table():
    """The 32 magnitudes of e2m3 (OCP Microscaling): 0 .. 7/8 in steps of 1/8
    (subnormal), then 1 .. 15/8, 2 .. 3.75 by 1/4, 4 .. 7.5 by 1/2."""
    want = [m / 8 for m in range(8)] + [1 + m / 8 for m in range(8)] + [2 + m / 4 for m in range(8)] + \
        [4 + m / 2 for m in range(8)]
    assert act4.e2m3_value(np.arange(32)).tolist() == want
    assert act4.e2m3_value(np.arange(32, 64)).tolist() == [-w for w in want]
    # |q| <= 15 written as the 5-bit magnitude reads as q / 8: the subnormals and
    # the first normal binade are spaced by 1/8
    q = np.arange(-15, 16)
    assert np.array_equal(act4.e2m3_value(act4.e2m3_fields(q)) * 8, q.astype(np.float64))


def _pack_e2m3_by_ints(q):
    """Independent packer: each 32-value stream as one Python integer."""
    M, K = q.shape
    out = bytearray()
    for m in range(M):
        for g in range(K // 64):
            streams = []
            for h in range(2):
                v = 0
                for j in range(32):
                    x = int(q[m, 64 * g + 32 * h + j])
                    v |= ((32 if x < 0 else 0) | abs(x)) << (6 * j)
                streams.append(v.to_bytes(24, "little"))
            out += streams[0][:16] + streams[1][:16] + streams[0][16:] + streams[1][16:]
    return np.frombuffer(bytes(out), dtype=np.uint8).reshape(M, K // 64 * 48)


def test_e2m3_pack_matches_integer_streams_and_round_trips():
    rs = np.random.default_rng(7)
    q = rs.integers(-8, 8, size=(5, 192)).astype(np.int8)
    q[0, :16] = np.arange(-8, 8)
    p = act4.pack_int4_e2m3(q)
    assert p.shape == (5, 144)
    assert np.array_equal(p, _pack_e2m3_by_ints(q))
    assert np.array_equal(act4.unpack_int4_e2m3(p, 192), q)
    # a quantized row: the storage holds exactly the INT4 codes
    x = rs.standard_normal((3, 256)).astype(np.float32)
    qi, _ = act4.quantize_int4(x)
    assert np.array_equal(act4.unpack_int4_e2m3(act4.pack_int4_e2m3(qi), 256), qi)
