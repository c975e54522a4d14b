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


def _run(w, seed=44, B=3, H=2, D=64, F=256, S=11, pos=7):
    rs = np.random.default_rng(seed)
    (kp, vp), slot_of, ns = _cache(rs, B, S, H, D)
    x = rs.standard_normal((B, H * D)).astype(np.float32)
    return block.decode_block(x, *w, kp, vp, slot_of, ns, pos, H), (kp, vp, slot_of, ns, x)


def test_up_rows_enter_linearly_gate_rows_through_relu2():
    """W_gate_up holds gate rows [0, F) and up rows [F, 2F).  The up branch enters
    h linearly: negating the up rows negates h, keeps the same top-k survivors
    (|h| unchanged), negates every INT8 code and so negates the down projection
    exactly, x1 untouched.  The gate goes through ReLU^2: negating the gate rows
    zeroes h where g was positive and opens it where g was negative, so the down
    projection changes.  With gate and up swapped the first identity fails."""
    rs = np.random.default_rng(45)
    HD, F = 128, 256
    w = list(_layer(rs, HD, F))
    (x_out, _, _, mid), _ = _run(w)
    w_up = list(w)
    w_up[4] = np.concatenate([w[4][:F], -w[4][F:]])
    (x_out2, _, _, mid2), _ = _run(w_up)
    assert np.array_equal(mid2["x1"], mid["x1"])
    assert np.array_equal(mid2["h_d"], -mid["h_d"])
    assert np.array_equal(mid2["keep_d"], mid["keep_d"])
    assert np.array_equal(mid2["q8d"], -mid["q8d"])
    assert np.array_equal(mid2["y_d"], -mid["y_d"])
    w_gate = list(w)
    w_gate[4] = np.concatenate([-w[4][:F], w[4][F:]])
    (_, _, _, mid3), _ = _run(w_gate)
    assert np.array_equal(mid3["x1"], mid["x1"])
    assert not np.array_equal(np.abs(mid3["y_d"]), np.abs(mid["y_d"]))
    # h is zero exactly where the gate is not positive
    assert np.array_equal(mid["h_d"] == 0, (mid["g"] <= 0) | (mid["u"] == 0))


def test_zero_gate_rows_leave_x1():
    """Gate rows all zero: g = 0, ReLU^2 gives 0, h = 0, every INT8 code is 0 and
    x_out == x1 bit for bit."""
    rs = np.random.default_rng(46)
    HD, F = 128, 256
    w = list(_layer(rs, HD, F))
    w[4] = np.concatenate([np.zeros_like(w[4][:F]), w[4][F:]])
    (x_out, _, _, mid), _ = _run(w)
    assert not mid["q8d"].any() and not mid["y_d"].any()
    assert np.array_equal(x_out, mid["x1"])


def test_top_k_keeps_half_of_each_input():
    """Exactly HD/2 of the out_proj inputs and F/2 of the down_proj inputs survive per
    token, and every survivor's magnitude is at least every dropped one's."""
    rs = np.random.default_rng(47)
    HD, F = 128, 256
    (_, _, _, mid), _ = _run(_layer(rs, HD, F))
    for keep, h, k in ((mid["keep_o"], mid["att"], HD // 2), (mid["keep_d"], mid["h_d"], F // 2)):
        assert (keep.sum(axis=1) == k).all()
        for m in range(keep.shape[0]):
            assert np.abs(h[m][keep[m]]).min() >= np.abs(h[m][~keep[m]]).max()
        assert not np.any(np.where(keep, 0, 1) * (mid["q8"] if h is mid["att"] else mid["q8d"]))


def test_query_is_the_first_slice():
    """With the q rows of W_qkv zero every score is 0, so the attention output is
    the plain mean of the dequantized values over positions 0..pos (the softmax of
    equal scores is uniform).  Taking q from another slice would not give it."""
    rs = np.random.default_rng(48)
    HD, F, H, D, pos = 128, 256, 2, 64, 7
    w = list(_layer(rs, HD, F))
    w[0] = np.concatenate([np.zeros_like(w[0][:HD]), w[0][HD:]])
    (_, _, vp2, mid), (kp, vp, slot_of, ns, x) = _run(w, H=H, D=D, pos=pos)
    vd = kv3.kv_unpack3(vp2[0][:, : pos + 1], vp2[1][:, : pos + 1], vp2[2], vp2[3], slot_of[:, : pos + 1], D)
    mean = vd.astype(np.float64).mean(axis=1).reshape(x.shape[0], HD)
    assert np.allclose(mid["att"], mean, rtol=1e-6, atol=1e-7 * np.abs(mean).max())


def test_key_and_value_slices_feed_their_caches():
    """Zeroing the v rows of W_qkv (columns 2HD..3HD of y_qkv) writes all-zero codes at
    pos into the V cache and leaves the K cache's new entry nonzero; zeroing the k
    rows does the opposite."""
    rs = np.random.default_rng(49)
    HD, F, D, pos = 128, 256, 64, 7
    base = list(_layer(rs, HD, F))
    for zero_rows, zero_cache in ((slice(2 * HD, 3 * HD), 1), (slice(HD, 2 * HD), 0)):
        w = list(base)
        t = w[0].copy()
        t[zero_rows] = 0
        w[0] = t
        (_, kp2, vp2, _), _ = _run(w, D=D, pos=pos)
        caches = (kp2, vp2)
        q_zero = kv3.planes_decode(caches[zero_cache][0][:, pos], D)
        q_other = kv3.planes_decode(caches[1 - zero_cache][0][:, pos], D)
        assert not q_zero.any() and q_other.any()
