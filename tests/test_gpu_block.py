"""GPU parity: one decoder layer for one new token per sequence (bw_block_decode) vs
the oracle's composition (oracle.block), both starting from the same synthetic
weights, cache contents and input.

The appended cache entries (codes, scales, 4-bit slot) must be bit-exact: they
depend only on the q/k/v projection, which both sides compute exactly.  The layer
output goes through attention, which the GPU evaluates in fp32 and the oracle in
fp64; the next top-k/INT8 step can then, rarely, flip a code or swap two entries
of nearly equal magnitude, so x_out is checked statistically: the median error is
at fp32 rounding level, almost every element is within 1e-4 of the layer's
output scale, and none is off by more than 2 % of it (a wiring mistake -- a wrong
weight slice, sign or position -- moves x_out by O(1) of that scale)."""
import numpy as np
import pytest
import torch

import synth
import ternary_weight_bit_amd as bw
from oracle import block, kv3, ternary
from tests.gpu_helpers import assert_same, bf16_dev, f32_dev, host

pytestmark = pytest.mark.gpu


def packed(parts, role):
    """Pack tensors separately into one concatenated buffer (GPU) and ternarize them (oracle)."""
    N = sum(p.shape[0] for p in parts)
    K = parts[0].shape[1]
    wp = torch.empty(N * K // 4, dtype=torch.uint8, device="cuda:0")
    bp = torch.empty(N, dtype=torch.float32, device="cuda:0")
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


def run_layer(seed, B, H, D, F, S_cap, pos):
    HD = H * D
    print(f"case layer B={B} H={H} D={D} F={F} S_cap={S_cap} pos={pos}", flush=True)
    wt = lambda i, n, k: synth.weight_tensor(seed + i, n, k)
    (gq, oq) = packed([wt(1, HD, HD), wt(2, HD, HD), wt(3, HD, HD)], bw.BW_ROLE_A4)
    (go, oo) = packed([wt(4, HD, HD)], bw.BW_ROLE_A8)
    (ggu, ogu) = packed([wt(5, F, HD), wt(6, F, HD)], bw.BW_ROLE_A4)
    (gd, od) = packed([wt(7, HD, F)], bw.BW_ROLE_A8)
    k = synth.kv_tensor(seed + 8, B, S_cap, H, D)
    v = synth.kv_tensor(seed + 9, B, S_cap, H, D)
    slot_of, ns = synth.kv_special_slots(seed + 8, B, S_cap)
    if slot_of[0, pos] < 0:  # make the new position of sequence 0 special (a fresh slot)
        slot_of[0, pos] = ns
        ns += 1
    sl = torch.from_numpy(slot_of).to("cuda:0")
    kp = bw.bw_kv_pack3(bf16_dev(k), sl, ns)
    vp = bw.bw_kv_pack3(bf16_dev(v), sl, ns)
    kp0 = [host(t).copy() for t in kp]
    x = synth.normal(seed + 10, (B, HD))
    out = host(bw.bw_block_decode(f32_dev(x), (*gq, *go, *ggu, *gd), kp, vp, sl, ns, pos, H))
    ref, okp, ovp, mid = block.decode_block(x, *oq, *oo, *ogu, *od, kv3.kv_pack3(k.f32, slot_of, ns),
                                            kv3.kv_pack3(v.f32, slot_of, ns), slot_of, ns, pos, H)
    # cache: position pos bit-exact, the 4-bit slot of sequence 0 too, other positions untouched
    for name, gpack, opack in (("K", kp, okp), ("V", vp, ovp)):
        g3, g_s3 = host(gpack[0]), host(gpack[1])
        assert_same(g3[:, pos], opack[0][:, pos], f"{name} p3 at pos")
        assert_same(g_s3[:, pos].view(np.uint32), opack[1][:, pos].view(np.uint32), f"{name} s3 at pos")
        s0 = int(slot_of[0, pos])
        assert_same(host(gpack[2])[s0], opack[2][s0], f"{name} p4 slot")
        assert_same(host(gpack[3])[s0].view(np.uint32), opack[3][s0].view(np.uint32), f"{name} s4 slot")
    assert_same(np.delete(host(kp[0]), pos, axis=1), np.delete(kp0[0], pos, axis=1), "K p3 elsewhere")
    # layer output
    d = np.abs(out.astype(np.float64) - ref.astype(np.float64))
    scale = float(np.abs(ref - x).max())
    print(f"  x_out: scale {scale:.4g}  median err {np.median(d):.3g}  max err {d.max():.3g}  "
          f"frac > 1e-4 scale {np.mean(d > 1e-4 * scale):.4f}", flush=True)
    assert np.isfinite(out).all()
    assert np.median(d) <= 1e-6 * scale + 1e-30
    assert np.mean(d > 1e-4 * scale) < 0.02
    assert d.max() <= 2e-2 * scale
    return out, ref


def test_small_layer():
    run_layer(synth.SEED_BASE + 90, B=2, H=2, D=128, F=512, S_cap=64, pos=37)


def test_small_layer_d64():
    run_layer(synth.SEED_BASE + 91, B=3, H=4, D=64, F=256, S_cap=40, pos=0)


def test_7b_layer_shapes():
    """7B shapes: hidden 4096 (32 heads x 128), FFN 11008, 8 sequences, a 512-position cache."""
    run_layer(synth.SEED_BASE + 92, B=8, H=32, D=128, F=11008, S_cap=512, pos=300)


def test_max_batch_last_position():
    """The largest batch the layer takes (16 sequences) writing the cache's last position."""
    run_layer(synth.SEED_BASE + 93, B=16, H=2, D=64, F=192, S_cap=33, pos=32)
