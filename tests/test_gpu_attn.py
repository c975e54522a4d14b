"""GPU parity: single-token attention over the 3-bit KV cache (bw_attn_decode_kv3) vs
the oracle (oracle.attn3, fp64 after the codec's dequantization).

Both sides quantize the same bf16 K/V themselves (GPU: bw_kv_pack3, pinned bit-exact
to the oracle codec elsewhere; oracle: kv3.kv_pack3).  The GPU computes in fp32, so
each output is held to a first-order rounding bound derived from the arithmetic:
with u = 2^-24 and gamma_n = n u / (1 - n u),
  score error  E_z   = max_s [gamma_D * sum_d |q_d k_sd| + 2^-31 max|q| sum_d |k_sd|
                            + 2^-23 max|q| s_s] / sqrt(D) + 4u |z_s|
(the second term is the kernel's fixed-point query, q rounded to multiples of
2^-30 max|q|, for its integer dot products; the third covers the two fp32
roundings of the exact integer sum, whose low part is below 2^31 units of
2^-30 max|q| times the scale s_s)
  weight error E_p   = 2 E_z + gamma_S + 2u      (exp, normalization, max shift)
  |out_d - ref_d| <= (E_p + gamma_S + 2u) * sum_s p_s |v_sd|  (+ 1e-30)
A wrong index, sign, scale or a missed special position costs O(1) of that sum."""
import numpy as np
import pytest
import torch

import synth
import ternary_weight_bit_amd as bw
from oracle import attn3, kv3
from tests.gpu_helpers import attn_bound, bf16_dev, f32_dev, host

pytestmark = pytest.mark.gpu


def check_attention(q32, k16, v16, slot_of, n_special, label, pairs=None):
    """q32 fp32 [B][H][D]; k16/v16 synth.Bf16 [B][S][H][D]; compares the (b, h) pairs
    given (default: all) against the oracle."""
    B, S, H, D = k16.f32.shape
    print(f"case {label}: B={B} S={S} H={H} D={D} specials={int((slot_of >= 0).sum())}", flush=True)
    sl = torch.from_numpy(slot_of).to("cuda:0")
    ns = n_special
    kp = bw.bw_kv_pack3(bf16_dev(k16), sl, ns)
    vp = bw.bw_kv_pack3(bf16_dev(v16), sl, ns)
    if ns == 0:
        kp = (kp[0], kp[1], None, None)
        vp = (vp[0], vp[1], None, None)
    ws = torch.full((max(bw.bw_attn_decode_kv3_workspace_bytes(B, S, H, D), 16),), 0x7F, dtype=torch.uint8,
                    device="cuda:0")  # contents on entry are ignored
    out = host(bw.bw_attn_decode_kv3(f32_dev(q32), kp, vp, sl, ns, workspace=ws))
    assert np.isfinite(out).all()
    okp = kv3.kv_pack3(k16.f32, slot_of, ns)
    ovp = kv3.kv_pack3(v16.f32, slot_of, ns)
    if pairs is None:
        pairs = [(b, h) for b in range(B) for h in range(H)]
    for b, h in pairs:
        sub = lambda pk: (pk[0][b : b + 1, :, h : h + 1], pk[1][b : b + 1, :, h : h + 1],
                          pk[2][:, h : h + 1], pk[3][:, h : h + 1])
        so = slot_of[b : b + 1]
        ref, p = attn3.decode_attention(q32[b : b + 1, h : h + 1], sub(okp), sub(ovp), so, D)
        kd = kv3.kv_unpack3(*sub(okp), so, D)[0, :, 0].astype(np.float64)  # [S][D]
        vd = kv3.kv_unpack3(*sub(ovp), so, D)[0, :, 0].astype(np.float64)
        bound = attn_bound(q32[b, h].astype(np.float64), kd, vd, p[0, 0])
        err = np.abs(out[b, h].astype(np.float64) - ref[0, 0])
        bad = err > bound
        assert not bad.any(), (f"{label} (b={b}, h={h}): {int(bad.sum())} dims outside the bound; "
                               f"worst err/bound {float((err / bound).max()):.3g}")


def qkv(seed, B, S, H, D):
    k = synth.kv_tensor(seed, B, S, H, D)
    v = synth.kv_tensor(seed + 1, B, S, H, D)
    q = synth.normal(seed + 2, (B, H, D))
    slot_of, ns = synth.kv_special_slots(seed, B, S)
    return q, k, v, slot_of, ns


@pytest.mark.parametrize("B,S,H,D", [(2, 100, 3, 128), (1, 130, 2, 64), (3, 257, 1, 128), (2, 1, 2, 128),
                                     (1, 33, 4, 64), (2, 90, 40, 128), (1, 70, 70, 64), (4, 999, 5, 128)])
def test_small_ragged(B, S, H, D):
    q, k, v, slot_of, ns = qkv(synth.SEED_BASE + 70 + S, B, S, H, D)
    check_attention(q, k, v, slot_of, ns, f"ragged {B}x{S}x{H}x{D}")


def test_no_special_positions():
    B, S, H, D = 2, 300, 2, 128
    q, k, v, _, _ = qkv(synth.SEED_BASE + 80, B, S, H, D)
    check_attention(q, k, v, np.full((B, S), -1, np.int32), 0, "no specials")


def test_many_special_positions():
    """A third of the positions special (all in the 4-bit side slab)."""
    B, S, H, D = 2, 384, 2, 128
    q, k, v, _, _ = qkv(synth.SEED_BASE + 81, B, S, H, D)
    slot_of = np.full((B, S), -1, np.int32)
    pos = np.arange(0, S, 3)
    slot_of[0, pos] = np.arange(len(pos))
    slot_of[1, pos + 1] = len(pos) + np.arange(len(pos))
    check_attention(q, k, v, slot_of, 2 * len(pos), "many specials")


def test_peaked_scores():
    """A query 40x larger than the keys: the softmax concentrates on a few positions."""
    B, S, H, D = 1, 512, 2, 128
    q, k, v, slot_of, ns = qkv(synth.SEED_BASE + 82, B, S, H, D)
    check_attention((q * np.float32(40.0)).astype(np.float32), k, v, slot_of, ns, "peaked")


def test_decode_kv_shape_sampled():
    """The decode KV shape, 8 x 4096 x 32 x 128 (special: bos plus 1 % per sequence);
    eight (batch, head) pairs checked against the oracle."""
    B, S, H, D = 8, 4096, 32, 128
    q, k, v, slot_of, ns = qkv(synth.SEED_BASE + 83, B, S, H, D)
    pairs = [(0, 0), (7, 31), (3, 17), (5, 2), (1, 30), (6, 9), (2, 23), (4, 4)]
    check_attention(q, k, v, slot_of, ns, "decode 8x4096x32x128", pairs=pairs)


def test_longest_sequence():
    B, S, H, D = 1, 16384, 2, 64
    q, k, v, slot_of, ns = qkv(synth.SEED_BASE + 84, B, S, H, D)
    check_attention(q, k, v, slot_of, ns, "S=16384")


def test_query_with_one_huge_entry():
    """max|q| far above the rest: the fixed-point query's step (2^-30 max|q|) is the
    largest error term, and the result must still meet the bound."""
    B, S, H, D = 1, 200, 2, 128
    q, k, v, slot_of, ns = qkv(synth.SEED_BASE + 85, B, S, H, D)
    q = q.copy()
    q[0, :, 5] = np.float32(3.0e4)
    check_attention(q, k, v, slot_of, ns, "huge q entry")


def test_chunk_at_lds_cap_sampled():
    """128 heads of 64 dims over 8 x 4096 positions: the chunk is cut to the largest
    one whose scores fit the LDS budget (124 positions, 34 chunks instead of 32), so
    the workgroup holds its largest score array beside the phase-sum buffer.  The
    oracle packs only the sampled heads (the codec works per vector)."""
    B, S, H, D = 8, 4096, 128, 64
    assert bw.bw_attn_decode_kv3_workspace_bytes(B, S, H, D) == B * 34 * H * (D + 4) * 4
    seed = synth.SEED_BASE + 86
    k16 = synth.kv_tensor(seed, B, S, H, D)
    v16 = synth.kv_tensor(seed + 1, B, S, H, D)
    q32 = synth.normal(seed + 2, (B, H, D))
    slot_of, ns = synth.kv_special_slots(seed, B, S)
    print(f"case LDS cap: B={B} S={S} H={H} D={D} specials={int((slot_of >= 0).sum())}", flush=True)
    sl = torch.from_numpy(slot_of).to("cuda:0")
    kp = bw.bw_kv_pack3(bf16_dev(k16), sl, ns)
    vp = bw.bw_kv_pack3(bf16_dev(v16), sl, ns)
    out = host(bw.bw_attn_decode_kv3(f32_dev(q32), kp, vp, sl, ns))
    assert np.isfinite(out).all()
    for b, h in [(0, 0), (7, 127), (3, 64), (5, 1), (2, 126), (6, 77)]:
        so = slot_of[b : b + 1]
        okp = kv3.kv_pack3(k16.f32[b : b + 1, :, h : h + 1], so, ns)
        ovp = kv3.kv_pack3(v16.f32[b : b + 1, :, h : h + 1], so, ns)
        ref, p = attn3.decode_attention(q32[b : b + 1, h : h + 1], okp, ovp, so, D)
        kd = kv3.kv_unpack3(*okp, so, D)[0, :, 0].astype(np.float64)
        vd = kv3.kv_unpack3(*ovp, so, D)[0, :, 0].astype(np.float64)
        bound = attn_bound(q32[b, h].astype(np.float64), kd, vd, p[0, 0])
        err = np.abs(out[b, h].astype(np.float64) - ref[0, 0])
        assert not (err > bound).any(), f"LDS cap (b={b}, h={h}): worst err/bound {float((err / bound).max()):.3g}"
