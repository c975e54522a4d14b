"""Pins for the oracle's single-token attention over the 3-bit KV cache."""
import math

import numpy as np

from oracle import attn3, kv3


def _brute_dequant(p3, s3, p4, s4, slot_of, b, s, h, D):
    """Dequantize one vector by reading the bit planes / nibbles directly (pure Python)."""
    slot = int(slot_of[b, s])
    if slot >= 0:
        out = []
        for d in range(D):
            byte = int(p4[slot, h, d // 2])
            c = (byte >> (4 * (d % 2))) & 0xF
            c = c - 16 if c >= 8 else c
            out.append(float(np.float32(np.float32(c) * s4[slot, h])))
        return out
    words = [int.from_bytes(bytes(p3[b, s, h, 4 * i : 4 * i + 4]), "little") for i in range(3 * D // 32)]
    # (word, bit within the byte) of bits 0, 1, 2 of field u = code + 4, by code index mod 8
    field_bits = [[(0, 0), (0, 1), (0, 2)], [(0, 3), (0, 4), (0, 5)], [(1, 0), (1, 1), (1, 2)],
                  [(1, 3), (1, 4), (1, 5)], [(2, 0), (2, 1), (2, 2)], [(2, 3), (2, 4), (2, 5)],
                  [(0, 6), (0, 7), (1, 6)], [(1, 7), (2, 6), (2, 7)]]
    out = []
    for d in range(D):
        g, r = divmod(d, 32)
        i, j = divmod(r, 8)
        u = sum(((words[3 * g + w] >> (8 * i + bit)) & 1) << k for k, (w, bit) in enumerate(field_bits[j]))
        out.append(float(np.float32(np.float32(u - 4) * s3[b, s, h])))
    return out


def _pack(x, slot_of, n_special):
    return kv3.kv_pack3(x, slot_of, n_special)


def test_brute_force_loops():
    """Tiny case against explicit Python loops (own dequantization, math.exp)."""
    rs = np.random.default_rng(31)
    B, S, H, D = 2, 7, 2, 64
    k = rs.standard_normal((B, S, H, D)).astype(np.float32)
    v = rs.standard_normal((B, S, H, D)).astype(np.float32)
    q = rs.standard_normal((B, H, D)).astype(np.float32)
    slot_of = np.full((B, S), -1, np.int32)
    slot_of[0, 0], slot_of[1, 4] = 0, 1
    kp, vp = _pack(k, slot_of, 2), _pack(v, slot_of, 2)
    out, p = attn3.decode_attention(q, kp, vp, slot_of, D)
    for b in range(B):
        for h in range(H):
            ks = [_brute_dequant(*kp, slot_of, b, s, h, D) for s in range(S)]
            vs = [_brute_dequant(*vp, slot_of, b, s, h, D) for s in range(S)]
            z = [sum(float(q[b, h, d]) * ks[s][d] for d in range(D)) / math.sqrt(D) for s in range(S)]
            mx = max(z)
            e = [math.exp(t - mx) for t in z]
            tot = sum(e)
            for s in range(S):
                assert abs(p[b, h, s] - e[s] / tot) < 1e-12
            for d in range(D):
                ref = sum(e[s] / tot * vs[s][d] for s in range(S))
                assert abs(out[b, h, d] - ref) < 1e-12 * (1 + abs(ref))


def test_equal_keys_average_values():
    """All keys equal -> uniform weights -> out is the plain mean of the value vectors."""
    rs = np.random.default_rng(32)
    B, S, H, D = 1, 9, 3, 32
    k = np.broadcast_to(rs.standard_normal((1, 1, H, D)), (B, S, H, D)).astype(np.float32)
    v = rs.standard_normal((B, S, H, D)).astype(np.float32)
    q = rs.standard_normal((B, H, D)).astype(np.float32)
    slot_of = np.full((B, S), -1, np.int32)
    vp = _pack(v, slot_of, 0)
    out, p = attn3.decode_attention(q, _pack(k, slot_of, 0), vp, slot_of, D)
    assert np.allclose(p, 1.0 / S, rtol=0, atol=1e-15)
    vd = kv3.kv_unpack3(*vp, slot_of, D).astype(np.float64)
    assert np.allclose(out[0], vd[0].mean(axis=0), rtol=1e-13, atol=1e-15)


def test_dominant_key_selects_its_value_and_special_slot_is_used():
    """One key aligned with a large query dominates the softmax, so out equals that
    position's value, read from its 4-bit slot (not its 3-bit codes)."""
    B, S, H, D = 1, 6, 1, 32
    rs = np.random.default_rng(33)
    k = (rs.standard_normal((B, S, H, D)) * 0.01).astype(np.float32)
    k[0, 3, 0] = 1.0
    q = np.full((B, H, D), 400.0, np.float32)
    v = rs.standard_normal((B, S, H, D)).astype(np.float32)
    slot_of = np.full((B, S), -1, np.int32)
    slot_of[0, 3] = 0
    vp = _pack(v, slot_of, 1)
    out, p = attn3.decode_attention(q, _pack(k, slot_of, 1), vp, slot_of, D)
    assert p[0, 0, 3] > 1 - 1e-12
    # dequantized values are fl(code * scale) in fp32
    four = (kv3.nibbles_decode(vp[2][0, 0]).astype(np.float32) * vp[3][0, 0]).astype(np.float64)
    three = (kv3.planes_decode(vp[0][0, 3, 0], D).astype(np.float32) * vp[1][0, 3, 0]).astype(np.float64)
    assert not np.allclose(four, three)
    assert np.allclose(out[0, 0], four, rtol=1e-10, atol=1e-12)
