"""GPU parity: 3-bit KV codec (bw_kv_pack3 / bw_kv_unpack3) vs the oracle, bit-exact."""
import numpy as np
import pytest
import torch

import synth
import ternary_weight_bit_amd as bw
from oracle import kv3
from tests.gpu_helpers import assert_same, bf16_dev, f32_dev, host

pytestmark = pytest.mark.gpu


def check_pack(kv_dev, x32, slot_of, ns, label):
    sd = torch.from_numpy(slot_of).to("cuda:0")
    p3, s3, p4, s4 = bw.bw_kv_pack3(kv_dev, sd, ns)
    r3, rs3, r4, rs4 = kv3.kv_pack3(x32, slot_of, ns)
    assert_same(host(p3), r3, f"{label} p3")
    assert_same(host(s3).view(np.uint32), rs3.view(np.uint32), f"{label} s3")
    if ns:
        assert_same(host(p4)[:ns], r4, f"{label} p4")
        assert_same(host(s4)[:ns].view(np.uint32), rs4.view(np.uint32), f"{label} s4")
    return (p3, s3, p4, s4), (r3, rs3, r4, rs4), sd


@pytest.mark.parametrize("D", [32, 64, 128, 256, 512])
@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_pack_unpack_small(D, dt):
    B, S, H = 2, 48, 4
    x = synth.kv_tensor(seed=D, B=B, S=S, H=H, D=D)
    slot_of, ns = synth.kv_special_slots(seed=D, B=B, S=S, frac=0.05)
    dev = bf16_dev(x) if dt == "bf16" else f32_dev(x.f32)
    gpu, ref, sd = check_pack(dev, x.f32, slot_of, ns, f"D={D} {dt}")
    out = bw.bw_kv_unpack3(*gpu, sd, ns, out_dtype=torch.float32)
    rout = kv3.kv_unpack3(*ref, slot_of, D)
    assert_same(host(out).view(np.uint32), rout.view(np.uint32), f"D={D} unpack f32")
    outb = bw.bw_kv_unpack3(*gpu, sd, ns, out_dtype=torch.bfloat16)
    assert_same(host(outb), kv3.to_bf16_bits(rout), f"D={D} unpack bf16")


def test_unpack_from_oracle_bytes():
    """The GPU decoder reads bytes written by the oracle's encoder."""
    B, S, H, D = 1, 16, 2, 128
    x = synth.kv_tensor(seed=77, B=B, S=S, H=H, D=D)
    slot_of, ns = synth.kv_special_slots(seed=77, B=B, S=S, frac=0.1)
    r3, rs3, r4, rs4 = kv3.kv_pack3(x.f32, slot_of, ns)
    dev = [torch.from_numpy(a).to("cuda:0") for a in (r3, rs3, r4, rs4)]
    out = bw.bw_kv_unpack3(*dev, torch.from_numpy(slot_of).to("cuda:0"), ns)
    assert_same(host(out).view(np.uint32), kv3.kv_unpack3(r3, rs3, r4, rs4, slot_of, D).view(np.uint32), "decode")


def test_no_special_tokens_and_out_of_range_slots():
    B, S, H, D = 2, 8, 3, 64
    x = synth.kv_tensor(seed=5, B=B, S=S, H=H, D=D)
    slot_of = np.full((B, S), -1, np.int32)
    slot_of[0, 3] = 7  # out of [0, n_special): ordinary
    gpu, ref, sd = check_pack(bf16_dev(x), x.f32, np.where(slot_of >= 0, -1, slot_of).astype(np.int32), 0, "no specials")
    sd2 = torch.from_numpy(slot_of).to("cuda:0")
    p3, s3, p4, s4 = bw.bw_kv_pack3(bf16_dev(x), sd2, 0)
    assert_same(host(p3), ref[0], "out-of-range slot ignored")


def test_full_layer_shape_sampled():
    """One 7B layer: B=8, S=4096, H=32, D=128 bf16 (the benchmark's launch); 512 sampled
    positions checked bit-exact, plus every special position."""
    B, S, H, D = 8, 4096, 32, 128
    x = synth.kv_tensor(seed=synth.SEED_BASE + 5, B=B, S=S, H=H, D=D)
    slot_of, ns = synth.kv_special_slots(seed=synth.SEED_BASE + 5, B=B, S=S)
    sd = torch.from_numpy(slot_of).to("cuda:0")
    xd = bf16_dev(x)
    p3, s3, p4, s4 = bw.bw_kv_pack3(xd, sd, ns)
    out = bw.bw_kv_unpack3(p3, s3, p4, s4, sd, ns, out_dtype=torch.bfloat16)
    hp3, hs3, hp4, hs4, hout = host(p3), host(s3), host(p4), host(s4), host(out)
    rs = np.random.default_rng(1)
    bs = [(int(b), int(s)) for b, s in zip(rs.integers(0, B, 512), rs.integers(0, S, 512))]
    bs += [tuple(map(int, p)) for p in np.argwhere(slot_of >= 0)]
    bi = np.array([p[0] for p in bs])
    si = np.array([p[1] for p in bs])
    sub = x.f32[bi, si][None]  # [1][n][H][D]
    sub_slots = np.where(slot_of[bi, si] >= 0, np.arange(len(bs)), -1).astype(np.int32)[None]
    r3, rs3, r4, rs4 = kv3.kv_pack3(sub, sub_slots, len(bs))
    assert_same(hp3[bi, si], r3[0], "full p3")
    assert_same(hs3[bi, si].view(np.uint32), rs3[0].view(np.uint32), "full s3")
    sp = slot_of[bi, si]
    special = sp >= 0
    assert_same(hp4[sp[special]], r4[np.arange(len(bs))[special]], "full p4")
    assert_same(hs4[sp[special]].view(np.uint32), rs4[np.arange(len(bs))[special]].view(np.uint32), "full s4")
    rout = kv3.kv_unpack3(r3, rs3, r4, rs4, sub_slots, D)[0]
    assert_same(hout[bi, si], kv3.to_bf16_bits(rout), "full unpack bf16")


def test_slot_ids_beyond_n_special_against_the_oracle():
    """slot_of values >= n_special (and negative ones other than -1) mark ordinary
    tokens on both sides: pack and unpack (fp32, bf16) bit-exact against the oracle
    fed the same slot ids."""
    B, S, H, D = 2, 40, 3, 128
    x = synth.kv_tensor(seed=6, B=B, S=S, H=H, D=D)
    slot_of, ns = synth.kv_special_slots(seed=6, B=B, S=S, frac=0.05)
    slot_of[0, 5] = ns  # one past the last slot
    slot_of[1, 9] = ns + 100
    slot_of[1, 11] = -3
    gpu, ref, sd = check_pack(bf16_dev(x), x.f32, slot_of, ns, "slot ids beyond n_special")
    out = bw.bw_kv_unpack3(*gpu, sd, ns, out_dtype=torch.float32)
    rout = kv3.kv_unpack3(*ref, slot_of, D)
    assert_same(host(out).view(np.uint32), rout.view(np.uint32), "unpack f32")
    outb = bw.bw_kv_unpack3(*gpu, sd, ns, out_dtype=torch.bfloat16)
    assert_same(host(outb), kv3.to_bf16_bits(rout), "unpack bf16")
