"""GPU parity: one decoder layer for one new token per sequence (bw_block_decode).

The layer is checked stage by stage.  Next to bw_block_decode the test runs the
same layer as a chain of separate C-ABI calls (bw_quantize, bw_bitlinear_a4,
bw_kv_pack3, bw_attn_decode_kv3, bw_quantize_sparse_a8, bw_bitlinear_sparse_a8,
with the two residual adds and the gate/up split done by the test in torch fp32),
and demands:

* the layer's x_out and its whole KV cache (3-bit slabs, scales, 4-bit slots)
  bit-identical to the chain's, as the layer's contract promises;
* every stage of the chain equal to the oracle fed with the chain's previous
  stage: INT4 and INT8 codes, scales, survivor masks and int32 accumulators bit
  for bit, every BitLinear output bit-exact against the fp32 hand-off
  fl(fl(acc * s) * beta) and within 1e-5 relative of the fp64 epilogue, the
  appended cache entries bit for bit against the oracle codec, and the attention
  output within the rounding bound derived from its fp32 arithmetic
  (gpu_helpers.attn_bound).

Cases: small ragged shapes, the 7B layer shapes, the largest batch at the cache's
last position, and the benchmark's configuration (8 sequences, 32 heads of 128,
FFN 11008, a 4096-position cache, new token at position 4095).  A guard test
checks that the layer writes nothing past the workspace size it asks for."""
import numpy as np
import pytest
import torch

import synth
import ternary_weight_bit_amd as bw
from oracle import act4, attn3, bitlinear, block, kv3, sparse8, ternary
from tests.gpu_helpers import assert_rel, assert_same, attn_bound, bf16_dev, f32_dev, host

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def packed(parts, role):
    """Pack tensors separately into one concatenated buffer (GPU) and ternarize them (oracle)."""
    N = sum(p.shape[0] for p in parts)
    K = parts[0].shape[1]
    wp = torch.empty(N * K // 4, dtype=torch.uint8, device=DEV)
    bp = torch.empty(N, dtype=torch.float32, device=DEV)
    ts, bs = [], []
    off = 0
    for w in parts:
        n = w.shape[0]
        bw.bw_pack_ternary(f32_dev(w), role, wp[off * K // 4 : (off + n) * K // 4], bp[off : off + n])
        t, b = ternary.quantize_weights(w)
        ts.append(t)
        bs.append(np.full(n, b, np.float32))
        off += n
    return (wp, bp), (np.concatenate(ts), np.concatenate(bs))


def bits(a):
    return np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)


def check_bitlinear(label, codes_ref, t, beta, s_x, acc_gpu, y_gpu):
    """acc bit-exact; y bit-exact against the fp32 hand-off and within 1e-5 of fp64."""
    acc_ref = bitlinear.contract(codes_ref, t)
    assert_same(acc_gpu, acc_ref.astype(np.int32), f"{label} acc")
    assert_same(bits(y_gpu), bits(block.fp32_handoff(acc_ref, s_x, beta)), f"{label} y (fp32 hand-off)")
    assert_rel(y_gpu, bitlinear.epilogue(acc_ref, s_x, beta), 1e-5, f"{label} y")


def check_int4(label, x_host, codes_gpu, s_gpu):
    q, s = act4.quantize_int4(x_host)
    assert_same(codes_gpu, act4.pack_nibbles(q), f"{label} INT4 codes")
    assert_same(bits(s_gpu), bits(s), f"{label} INT4 scales")
    return q, s


def check_sparse(label, h_in, up, k, codes_gpu, s_gpu, mask_gpu):
    _, keep, q, s = sparse8.sparse_a8(h_in, up, k)
    assert_same(mask_gpu.view(np.uint32), sparse8.mask_words(keep), f"{label} survivors")
    assert (keep.sum(axis=1) == k).all()
    assert_same(codes_gpu, q, f"{label} INT8 codes")
    assert_same(bits(s_gpu), bits(s), f"{label} INT8 scales")
    return q, s


def clone_pack(p):
    return tuple(t.clone() for t in p)


def run_layer(seed, B, H, D, F, S_cap, pos, pairs=None):
    """pairs: (b, h) attention outputs checked against the oracle (default: all)."""
    HD = H * D
    print(f"case layer B={B} H={H} D={D} F={F} S_cap={S_cap} pos={pos}", flush=True)
    wt = lambda i, n, k: synth.weight_tensor(seed + i, n, k)
    (gq, (t_qkv, b_qkv)) = packed([wt(1, HD, HD), wt(2, HD, HD), wt(3, HD, HD)], bw.BW_ROLE_A4)
    (go, (t_o, b_o)) = packed([wt(4, HD, HD)], bw.BW_ROLE_A8)
    (ggu, (t_gu, b_gu)) = packed([wt(5, F, HD), wt(6, F, HD)], bw.BW_ROLE_A4)
    (gd, (t_d, b_d)) = packed([wt(7, HD, F)], bw.BW_ROLE_A8)
    k = synth.kv_tensor(seed + 8, B, S_cap, H, D)
    v = synth.kv_tensor(seed + 9, B, S_cap, H, D)
    slot_of, ns = synth.kv_special_slots(seed + 8, B, S_cap)
    if slot_of[0, pos] < 0:  # make the new position of sequence 0 special (a fresh slot)
        slot_of[0, pos] = ns
        ns += 1
    sl = torch.from_numpy(slot_of).to(DEV)
    kp0 = bw.bw_kv_pack3(bf16_dev(k), sl, ns)
    vp0 = bw.bw_kv_pack3(bf16_dev(v), sl, ns)
    del k, v
    x = synth.normal(seed + 10, (B, HD))
    xd = f32_dev(x)
    print("  inputs ready", flush=True)

    # the layer in one call
    kp_l, vp_l = clone_pack(kp0), clone_pack(vp0)
    out = host(bw.bw_block_decode(xd, (*gq, *go, *ggu, *gd), kp_l, vp_l, sl, ns, pos, H))
    assert np.isfinite(out).all()

    # the same layer as separate calls, each stage against the oracle
    kp_c, vp_c = clone_pack(kp0), clone_pack(vp0)
    i32 = lambda n: torch.empty((B, n), dtype=torch.int32, device=DEV)
    c4, s4 = bw.bw_quantize(xd, bw.BW_ACT_INT4)
    q4, sx = check_int4("x", x, host(c4), host(s4))
    acc = i32(3 * HD)
    y_qkv = bw.bw_bitlinear_a4(c4, s4, bw.BW_ACT_INT4, *gq, acc_dbg=acc)
    check_bitlinear("q/k/v", q4, t_qkv, b_qkv, sx, host(acc), host(y_qkv))
    y_qkv_h = host(y_qkv)
    col = sl[:, pos : pos + 1].contiguous()
    for name, cache, lo in (("K", kp_c, HD), ("V", vp_c, 2 * HD)):
        new = y_qkv[:, lo : lo + HD].reshape(B, 1, H, D).contiguous()
        p3n, s3n, _, _ = bw.bw_kv_pack3(new, col, ns, p4=cache[2], s4=cache[3])
        cache[0][:, pos] = p3n[:, 0]
        cache[1][:, pos] = s3n[:, 0]
        r3, rs3, r4, rs4 = kv3.kv_pack3(y_qkv_h[:, lo : lo + HD].reshape(B, 1, H, D), slot_of[:, pos : pos + 1], ns)
        assert_same(host(p3n), r3, f"{name} appended codes")
        assert_same(bits(host(s3n)), bits(rs3), f"{name} appended scales")
        for b in range(B):
            sl_b = int(slot_of[b, pos])
            if 0 <= sl_b < ns:
                assert_same(host(cache[2])[sl_b], r4[sl_b], f"{name} appended 4-bit slot")
                assert_same(bits(host(cache[3])[sl_b]), bits(rs4[sl_b]), f"{name} appended 4-bit scales")
    upto = lambda p: (p[0][:, : pos + 1].contiguous(), p[1][:, : pos + 1].contiguous(), p[2], p[3])
    q_att = y_qkv[:, :HD].reshape(B, H, D).contiguous()
    att = bw.bw_attn_decode_kv3(q_att, upto(kp_c), upto(vp_c), sl[:, : pos + 1].contiguous(), ns)
    att_h = host(att)
    kc = [host(t) for t in kp_c]
    vc = [host(t) for t in vp_c]
    so = slot_of[:, : pos + 1]
    if pairs is None:
        pairs = [(b, h) for b in range(B) for h in range(H)]
    for b, h in pairs:
        sub = lambda c: (c[0][b : b + 1, : pos + 1, h : h + 1], c[1][b : b + 1, : pos + 1, h : h + 1],
                         c[2][:, h : h + 1], c[3][:, h : h + 1])
        ref, p = attn3.decode_attention(y_qkv_h[b : b + 1, h * D : (h + 1) * D].reshape(1, 1, D), sub(kc), sub(vc),
                                        so[b : b + 1], D, ns)
        kd = kv3.kv_unpack3(*sub(kc), so[b : b + 1], D, ns)[0, :, 0].astype(np.float64)
        vd = kv3.kv_unpack3(*sub(vc), so[b : b + 1], D, ns)[0, :, 0].astype(np.float64)
        bound = attn_bound(y_qkv_h[b, h * D : (h + 1) * D].astype(np.float64), kd, vd, p[0, 0])
        err = np.abs(att_h[b, h].astype(np.float64) - ref[0, 0])
        assert (err <= bound).all(), f"attention (b={b}, h={h}): worst err/bound {float((err / bound).max()):.3g}"
    print(f"  attention checked on {len(pairs)} (batch, head) pairs", flush=True)
    a32 = att.reshape(B, HD)
    mask = torch.empty((B, HD // 32), dtype=torch.int32, device=DEV)
    c8, s8 = bw.bw_quantize_sparse_a8(a32, None, HD // 2, mask_dbg=mask)
    q8, sx8 = check_sparse("out_proj input", att_h.reshape(B, HD), None, HD // 2, host(c8), host(s8), host(mask))
    acc = i32(HD)
    y_o = bw.bw_bitlinear_sparse_a8(c8, s8, *go, acc_dbg=acc)
    check_bitlinear("out_proj", q8, t_o, b_o, sx8, host(acc), host(y_o))
    x1 = xd + y_o
    x1_h = host(x1)
    assert_same(bits(x1_h), bits((x + host(y_o)).astype(np.float32)), "x1")
    c4b, s4b = bw.bw_quantize(x1, bw.BW_ACT_INT4)
    q4b, sxb = check_int4("x1", x1_h, host(c4b), host(s4b))
    acc = i32(2 * F)
    y_gu = bw.bw_bitlinear_a4(c4b, s4b, bw.BW_ACT_INT4, *ggu, acc_dbg=acc)
    check_bitlinear("gate/up", q4b, t_gu, b_gu, sxb, host(acc), host(y_gu))
    g = y_gu[:, :F].contiguous()
    u = y_gu[:, F:].contiguous()
    mask = torch.empty((B, F // 32), dtype=torch.int32, device=DEV)
    c8d, s8d = bw.bw_quantize_sparse_a8(g, u, F // 2, mask_dbg=mask)
    q8d, sx8d = check_sparse("down_proj input", host(g), host(u), F // 2, host(c8d), host(s8d), host(mask))
    acc = i32(HD)
    y_d = bw.bw_bitlinear_sparse_a8(c8d, s8d, *gd, acc_dbg=acc)
    check_bitlinear("down_proj", q8d, t_d, b_d, sx8d, host(acc), host(y_d))
    x_chain = host(x1 + y_d)
    print("  every stage of the chain matches the oracle", flush=True)

    # the layer equals the chain bit for bit, output and cache
    assert_same(bits(out), bits(x_chain), "x_out (layer vs separate calls)")
    for name, a, c in (("K", kp_l, kp_c), ("V", vp_l, vp_c)):
        for part, ta, tc in zip(("p3", "s3", "p4", "s4"), a, c):
            ha, hc = host(ta), host(tc)
            if ha.dtype == np.float32:
                ha, hc = bits(ha), bits(hc)
            assert_same(ha, hc, f"{name} cache {part} (layer vs separate calls)")
    # positions other than pos are as packed
    assert_same(np.delete(host(kp_l[0]), pos, axis=1), np.delete(host(kp0[0]), pos, axis=1), "K p3 elsewhere")
    assert_same(np.delete(host(vp_l[0]), pos, axis=1), np.delete(host(vp0[0]), pos, axis=1), "V p3 elsewhere")


def test_small_layer():
    run_layer(synth.SEED_BASE + 90, B=2, H=2, D=128, F=512, S_cap=64, pos=37)


def test_small_layer_d64():
    run_layer(synth.SEED_BASE + 91, B=3, H=4, D=64, F=256, S_cap=40, pos=0)


def test_7b_layer_shapes():
    """7B shapes: hidden 4096 (32 heads x 128), FFN 11008, 8 sequences, a 512-position cache."""
    run_layer(synth.SEED_BASE + 92, B=8, H=32, D=128, F=11008, S_cap=512, pos=300,
              pairs=[(b, h) for b in range(8) for h in (0, 13, 31)])


def test_max_batch_last_position():
    """The largest batch the layer takes (16 sequences) writing the cache's last position."""
    run_layer(synth.SEED_BASE + 93, B=16, H=2, D=64, F=192, S_cap=33, pos=32)


def test_benchmark_layer_configuration():
    """The decoder-layer configuration the benchmark times: 8 sequences, 32 heads of
    128, FFN 11008, a 4096-position cache, the new token at position 4095."""
    run_layer(synth.SEED_BASE + 94, B=8, H=32, D=128, F=11008, S_cap=4096, pos=4095,
              pairs=[(0, 0), (7, 31), (3, 17), (5, 2), (1, 30), (6, 9), (2, 23), (4, 4)])


def test_workspace_guard_bytes_untouched():
    """One sequence at position 1278 of a 2048-position cache with 32 heads of 128:
    the attention launch there has the most chunks; the layer must write nothing
    beyond the workspace size it asks for."""
    B, H, D, F, S_cap, pos = 1, 32, 128, 256, 2048, 1278
    HD = H * D
    print(f"case guard B={B} H={H} D={D} F={F} S_cap={S_cap} pos={pos}", flush=True)
    seed = synth.SEED_BASE + 95
    wt = lambda i, n, k: synth.weight_tensor(seed + i, n, k)
    (gq, _) = packed([wt(1, 3 * HD, HD)], bw.BW_ROLE_A4)
    (go, _) = packed([wt(2, HD, HD)], bw.BW_ROLE_A8)
    (ggu, _) = packed([wt(3, 2 * F, HD)], bw.BW_ROLE_A4)
    (gd, _) = packed([wt(4, HD, F)], bw.BW_ROLE_A8)
    slot_of, ns = synth.kv_special_slots(seed, B, S_cap)
    sl = torch.from_numpy(slot_of).to(DEV)
    kp = bw.bw_kv_pack3(bf16_dev(synth.kv_tensor(seed + 5, B, S_cap, H, D)), sl, ns)
    vp = bw.bw_kv_pack3(bf16_dev(synth.kv_tensor(seed + 6, B, S_cap, H, D)), sl, ns)
    need = bw.bw_block_decode_workspace_bytes(B, S_cap, H, D, F)
    guard = 1 << 20
    buf = torch.full((need + guard,), 0xA5, dtype=torch.uint8, device=DEV)
    x = f32_dev(synth.normal(seed + 7, (B, HD)))
    ref = bw.bw_block_decode(x, (*gq, *go, *ggu, *gd), clone_pack(kp), clone_pack(vp), sl, ns, pos, H)
    out = bw.bw_block_decode(x, (*gq, *go, *ggu, *gd), kp, vp, sl, ns, pos, H, workspace=buf[:need])
    tail = host(buf[need:])
    assert (tail == 0xA5).all(), f"{int((tail != 0xA5).sum())} guard bytes written"
    assert_same(bits(host(out)), bits(host(ref)), "x_out with an exact-size workspace")
