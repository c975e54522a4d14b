"""Pins for the oracle's decoder layer (composition of the pinned pieces)."""
import numpy as np

from oracle import block, kv3, ternary


def _layer(rs, HD, F, zero_out=False):
    w = lambda n, k: (rs.standard_normal((n, k)) * 0.02).astype(np.float32)
    ts, bs = [], []
    for n, k in ((HD, HD), (HD, HD), (HD, HD)):  # q, k, v ternarized separately
        t, b = ternary.quantize_weights(w(n, k))
        ts.append(t)
        bs.append(np.full(n, b, np.float32))
    t_qkv, b_qkv = np.concatenate(ts), np.concatenate(bs)
    t_o, bo = ternary.quantize_weights(w(HD, HD))
    tg, bg = ternary.quantize_weights(w(F, HD))
    tu, bu = ternary.quantize_weights(w(F, HD))
    t_d, bd = ternary.quantize_weights(w(HD, F))
    if zero_out:
        t_o = np.zeros_like(t_o)
        t_d = np.zeros_like(t_d)
    return (t_qkv, b_qkv, t_o, np.full(HD, bo, np.float32), np.concatenate([tg, tu]),
            np.concatenate([np.full(F, bg, np.float32), np.full(F, bu, np.float32)]), t_d,
            np.full(HD, bd, np.float32))


def _cache(rs, B, S, H, D):
    slot_of = np.full((B, S), -1, np.int32)
    slot_of[:, 0] = np.arange(B)
    slot_of[0, 5] = B
    kv = [(rs.standard_normal((B, S, H, D))).astype(np.float32) for _ in range(2)]
    return [kv3.kv_pack3(t, slot_of, B + 1) for t in kv], slot_of, B + 1


def test_zero_output_weights_pass_the_residual_through():
    """With W_o = W_down = 0 both branches add exactly 0, so x_out == x bit for bit,
    and the cache gains exactly the codec's packing of the new k, v."""
    rs = np.random.default_rng(41)
    B, H, D, F, S, pos = 2, 2, 64, 128, 9, 5
    HD = H * D
    (kp, vp), slot_of, ns = _cache(rs, B, S, H, D)
    x = rs.standard_normal((B, HD)).astype(np.float32)
    w = _layer(rs, HD, F, zero_out=True)
    x_out, kp2, vp2, mid = block.decode_block(x, *w, kp, vp, slot_of, ns, pos, H)
    assert np.array_equal(x_out, x)
    assert not mid["y_o"].any() and not mid["y_d"].any()
    for pack, new, cols in ((kp2, mid["y_qkv"], slice(HD, 2 * HD)), (vp2, mid["y_qkv"], slice(2 * HD, 3 * HD))):
        q3, s3, q4, s4 = kv3.kv_pack3(new[:, cols].reshape(B, 1, H, D), slot_of[:, pos : pos + 1], ns)
        assert np.array_equal(pack[0][:, pos], q3[:, 0]) and np.array_equal(pack[1][:, pos], s3[:, 0])
        assert np.array_equal(pack[2][B], q4[B]) and np.array_equal(pack[3][B], s4[B])  # pos 5 of seq 0 is special
    # positions other than pos are untouched
    assert np.array_equal(np.delete(kp2[0], pos, axis=1), np.delete(kp[0], pos, axis=1))


def test_positions_after_pos_do_not_matter():
    """Attention covers positions 0..pos only: changing the cache beyond pos leaves
    every output unchanged."""
    rs = np.random.default_rng(42)
    B, H, D, F, S, pos = 2, 2, 64, 128, 12, 6
    HD = H * D
    (kp, vp), slot_of, ns = _cache(rs, B, S, H, D)
    x = rs.standard_normal((B, HD)).astype(np.float32)
    w = _layer(rs, HD, F)
    out1, *_ = block.decode_block(x, *w, kp, vp, slot_of, ns, pos, H)
    kp_alt = (kp[0].copy(), kp[1].copy(), kp[2], kp[3])
    kp_alt[0][:, pos + 1 :] ^= 0x5A
    kp_alt[1][:, pos + 1 :] *= 3
    out2, *_ = block.decode_block(x, *w, kp_alt, vp, slot_of, ns, pos, H)
    assert np.array_equal(out1, out2)


def test_handoff_is_the_fp32_epilogue():
    """fp32_handoff rounds twice in fp32, matching fl(fl(acc*s)*beta) written out per element."""
    rs = np.random.default_rng(43)
    acc = rs.integers(-30000, 30000, size=(3, 5))
    s = rs.uniform(0.01, 2, size=3).astype(np.float32)
    b = rs.uniform(0.001, 0.05, size=5).astype(np.float32)
    y = block.fp32_handoff(acc, s, b)
    for m in range(3):
        for n in range(5):
            assert y[m, n] == np.float32(np.float32(np.float32(acc[m, n]) * s[m]) * b[n])
