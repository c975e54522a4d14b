"""Pins for the oracle's 3-bit KV codec."""
import json
import os

import numpy as np

from oracle import kv3

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _g():
    with open(os.path.join(GOLD, "kv_worked.json")) as f:
        return json.load(f)


def test_worked_example():
    g = _g()
    x = np.array(g["x"], dtype=np.float32)
    q3, s3 = kv3.quantize(x, 3, -4, 3)
    assert q3.tolist() == g["codes3"] and s3 == np.float32(g["scale3"])
    q4, s4 = kv3.quantize(x, 7, -8, 7)
    assert q4.tolist() == g["codes4"] and hex(np.float32(s4).view(np.uint32)) == g["scale4_f32_bits"]


# Bit positions (word, bit) of the three bits of field u_j (j = code index mod 8)
# inside byte i = (code index mod 32) // 8 of each word, written out per field.
FIELD_BITS = {
    0: [(0, 0), (0, 1), (0, 2)], 1: [(0, 3), (0, 4), (0, 5)],
    2: [(1, 0), (1, 1), (1, 2)], 3: [(1, 3), (1, 4), (1, 5)],
    4: [(2, 0), (2, 1), (2, 2)], 5: [(2, 3), (2, 4), (2, 5)],
    6: [(0, 6), (0, 7), (1, 6)], 7: [(1, 7), (2, 6), (2, 7)],
}


def _scatter(q):
    """Reference placement of every code by the per-bit table (bit k of u = q + 4)."""
    D = q.size
    words = np.zeros((D // 32, 3), dtype=np.uint32)
    for c in range(D):
        g, r = divmod(c, 32)
        i, j = divmod(r, 8)
        u = int(q[c]) + 4
        for k, (w, b) in enumerate(FIELD_BITS[j]):
            if (u >> k) & 1:
                words[g, w] |= np.uint32(1 << (8 * i + b))
    return words.reshape(-1)


def test_plane_layout_single_codes():
    D = 64
    for pos, code in [(0, 1), (0, -1), (6, -4), (7, 3), (31, -4), (32, 3), (45, -2), (62, 2), (63, -3)]:
        q = np.zeros(D, dtype=np.int8)
        q[pos] = code
        p = kv3.planes_encode(q)
        assert p.size == 3 * D // 8
        assert np.array_equal(p.view("<u4"), _scatter(q)), (pos, code)
        assert np.array_equal(kv3.planes_decode(p, D), q)


def test_plane_layout_all_codes():
    rs = np.random.default_rng(5)
    for D in (32, 128):
        q = rs.integers(-4, 4, size=D).astype(np.int8)
        p = kv3.planes_encode(q)
        assert np.array_equal(p.view("<u4"), _scatter(q))
        assert np.array_equal(kv3.planes_decode(p, D), q)


def _case(seed, B=2, S=9, H=3, D=64):
    rs = np.random.default_rng(seed)
    x = (rs.standard_normal((B, S, H, D)) * rs.lognormal(0, 0.5, size=(1, 1, H, 1))).astype(np.float32)
    slot_of = np.full((B, S), -1, dtype=np.int32)
    slot_of[0, 0], slot_of[0, 4], slot_of[1, 0] = 0, 1, 2
    return x, slot_of, 3


def test_roundtrip_error_bounds_and_specials():
    x, slot_of, ns = _case(30)
    p3, s3, p4, s4 = kv3.kv_pack3(x, slot_of, ns)
    y = kv3.kv_unpack3(p3, s3, p4, s4, slot_of, x.shape[-1])
    a = np.abs(x).max(axis=-1)
    err = np.abs(y.astype(np.float64) - x)
    special = slot_of >= 0
    bound3 = (a / 3)[..., None] * (0.5 + 2.0**-19)
    bound4 = (a / 7)[..., None] * (0.5 + 2.0**-19)
    assert np.all(err[~special] <= bound3[~special])
    assert np.all(err[special] <= bound4[special])
    q3 = kv3.planes_decode(p3, x.shape[-1])
    assert q3.min() >= -3 and q3.max() <= 3
    q4 = kv3.nibbles_decode(p4)
    assert q4.min() >= -7 and q4.max() <= 7
    # special positions are strictly better than their 3-bit codes would be on average
    y3 = q3.astype(np.float32) * s3[..., None]
    assert np.abs(y3[special] - x[special]).mean() > err[special].mean()


def test_idempotence():
    x, slot_of, ns = _case(31)
    p3, s3, p4, s4 = kv3.kv_pack3(x, slot_of, ns)
    y = kv3.kv_unpack3(p3, s3, p4, s4, slot_of, x.shape[-1])
    p3b, s3b, p4b, s4b = kv3.kv_pack3(y, slot_of, ns)
    # ordinary positions: the 3-bit codes reproduce exactly
    ordinary = slot_of < 0
    assert np.array_equal(p3b[ordinary], p3[ordinary])
    assert np.array_equal(p4b, p4)


def test_zero_vector():
    x = np.zeros((1, 1, 1, 32), dtype=np.float32)
    p3, s3, p4, s4 = kv3.kv_pack3(x, np.full((1, 1), -1, np.int32), 0)
    # every field holds u = 0 + 4: bytes 0x24 (W0), 0x64 (W1), 0xA4 (W2)
    assert p3.reshape(-1).tolist() == [0x24] * 4 + [0x64] * 4 + [0xA4] * 4
    assert s3[0, 0, 0] == np.float32(1e-5) / np.float32(3)


def test_slot_values_beyond_n_special_are_ordinary_tokens():
    """Only slot_of values in [0, n_special) name a side slot; larger values (and
    negative ones) mark ordinary tokens: 3-bit codes only, side slab untouched."""
    x, slot_of, ns = _case(32)
    odd = slot_of.copy()
    odd[1, 3] = ns  # one past the last slot
    odd[0, 7] = ns + 40
    odd[1, 8] = -7
    p3, s3, p4, s4 = kv3.kv_pack3(x, odd, ns)
    r3, rs3, r4, rs4 = kv3.kv_pack3(x, slot_of, ns)  # same positions marked -1 there
    assert np.array_equal(p3, r3) and np.array_equal(s3, rs3)
    assert np.array_equal(p4, r4) and np.array_equal(s4, rs4)
    y = kv3.kv_unpack3(p3, s3, p4, s4, odd, x.shape[-1])
    q3 = kv3.planes_decode(p3, x.shape[-1]).astype(np.float32) * s3[..., None]
    for b, s in ((1, 3), (0, 7), (1, 8)):
        assert np.array_equal(y[b, s], q3[b, s])
    assert kv3.is_special(odd, ns).sum() == (slot_of >= 0).sum()


def _bf16_rne_exact(bits32: int) -> int:
    """bf16 bit pattern of the fp32 value with these bits, rounded half-to-even,
    by exact rational arithmetic: bf16 keeps 8 significant bits, exponents down to
    -126 (below that a fixed quantum of 2^-133), and overflows to infinity."""
    from fractions import Fraction

    sign = (bits32 >> 31) << 15
    v = Fraction(float(np.array([bits32], dtype=np.uint32).view(np.float32)[0]))
    a = abs(v)
    if a == 0:
        return sign
    e = a.numerator.bit_length() - a.denominator.bit_length()  # 2^e <= a < 2^(e+2)
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    ulp = Fraction(2) ** (max(e, -126) - 7)
    n = a.numerator * ulp.denominator // (a.denominator * ulp.numerator)
    r = a / ulp - n
    if r > Fraction(1, 2) or (r == Fraction(1, 2) and n % 2 == 1):
        n += 1
    val = n * ulp
    if val >= Fraction(2) ** 128:
        return sign | 0x7F80
    b = int(np.array([float(val)], dtype=np.float32).view(np.uint32)[0])
    assert b & 0xFFFF == 0  # representable in bf16
    return sign | (b >> 16)


def test_bf16_rounding_hand_cases():
    """RNE of fp32 to bf16: exact ties go to the even bf16 pattern, a carry moves
    into the exponent, signed zeros and subnormals keep their sign, the largest
    finite fp32 overflows to infinity."""
    cases = {
        0x3F800000: 0x3F80,  # 1.0 exact
        0x3F808000: 0x3F80,  # tie, 0x3F80 even: stays
        0x3F818000: 0x3F82,  # tie, 0x3F81 odd: up to even
        0x3F808001: 0x3F81,  # just above the tie
        0x3F807FFF: 0x3F80,  # just below the tie
        0x3FFF8000: 0x4000,  # tie up from an odd pattern carries into the exponent
        0xBFFF8000: 0xC000,  # same, negative
        0xBF818000: 0xBF82,
        0x00000000: 0x0000,  # +0
        0x80000000: 0x8000,  # -0
        0x00008000: 0x0000,  # subnormal tie to even (0)
        0x00018000: 0x0002,  # subnormal tie up from odd
        0x80018000: 0x8002,
        0x00000001: 0x0000,  # smallest subnormal
        0x007FFFFF: 0x0080,  # largest subnormal rounds to the smallest normal
        0x7F7F7FFF: 0x7F7F,  # below the top tie
        0x7F7F8000: 0x7F80,  # tie from odd 0x7F7F: rounds to infinity
        0x7F7FFFFF: 0x7F80,  # largest finite fp32: infinity
        0xFF7FFFFF: 0xFF80,
    }
    bits = np.array(list(cases), dtype=np.uint32)
    got = kv3.to_bf16_bits(bits.view(np.float32))
    for b, g in zip(cases, got.tolist()):
        assert g == cases[b], (hex(b), hex(g), hex(cases[b]))
        assert _bf16_rne_exact(b) == cases[b], hex(b)


def test_bf16_rounding_sweep_against_exact_rationals():
    """Random finite fp32 patterns, weighted towards the cases that decide the
    rounding (low halves 0x7FFF, 0x8000, 0x8001, 0xFFFF, 0x0000) and towards
    subnormals and the top binade, against the exact-rational rounding."""
    rs = np.random.default_rng(77)
    n = 6000
    hi = rs.integers(0, 1 << 16, size=n, dtype=np.uint32)
    hi = np.where((hi & 0x7F80) == 0x7F80, hi & 0xFF7F, hi)  # no inf/nan inputs
    lo = rs.integers(0, 1 << 16, size=n, dtype=np.uint32)
    pick = rs.integers(0, 6, size=n)
    special_lo = np.array([0x7FFF, 0x8000, 0x8001, 0xFFFF, 0x0000], dtype=np.uint32)
    lo = np.where(pick < 5, special_lo[np.minimum(pick, 4)], lo)
    hi[:400] = (hi[:400] & 0x8000) | (hi[:400] & 0x007F)  # subnormals
    hi[400:800] = (hi[400:800] & 0x8000) | 0x7F00 | (hi[400:800] & 0x007F)  # top binade
    bits = (hi << 16) | lo
    got = kv3.to_bf16_bits(bits.view(np.float32))
    for b, g in zip(bits.tolist(), got.tolist()):
        assert g == _bf16_rne_exact(b), hex(b)
