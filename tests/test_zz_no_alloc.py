"""GPU test: the allocation-free decoder layer (bw_block_decode_noalloc, whose
workspace is the library's static per-GPU array) gives bit for bit what
bw_block_decode gives with a caller workspace (x_out and the whole KV cache), on
two calls in a row, the second with smaller shapes, so that a stale first call in
the shared array would show."""
import numpy as np
import pytest
import torch

import synth
import ternary_weight_bit_amd as bw
from tests.gpu_helpers import assert_same, bf16_dev, f32_dev, host

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _weights(seed, H, D, F):
    HD = H * D
    out = []
    for i, (n, k, role) in enumerate(((3 * HD, HD, bw.BW_ROLE_A4), (HD, HD, bw.BW_ROLE_A8),
                                      (2 * F, HD, bw.BW_ROLE_A4), (HD, F, bw.BW_ROLE_A8))):
        out += list(bw.bw_pack_ternary(f32_dev(synth.weight_tensor(seed + i, n, k)), role))
    return tuple(out)


def _bits(t):
    a = host(t)
    return a.view(np.uint32) if a.dtype == np.float32 else a


def _compare(seed, B, H, D, F, S_cap, pos):
    HD = H * D
    print(f"case no-alloc layer B={B} H={H} D={D} F={F} S_cap={S_cap} pos={pos}", flush=True)
    w = _weights(seed, H, D, F)
    slot_of, ns = synth.kv_special_slots(seed, B, S_cap)
    sl = torch.from_numpy(slot_of).to(DEV)
    kp = bw.bw_kv_pack3(bf16_dev(synth.kv_tensor(seed + 10, B, S_cap, H, D)), sl, ns)
    vp = bw.bw_kv_pack3(bf16_dev(synth.kv_tensor(seed + 11, B, S_cap, H, D)), sl, ns)
    x = f32_dev(synth.normal(seed + 12, (B, HD)))
    kp_ref, vp_ref = tuple(t.clone() for t in kp), tuple(t.clone() for t in vp)
    ref = bw.bw_block_decode(x, w, kp_ref, vp_ref, sl, ns, pos, H)
    out = torch.empty_like(x)
    bw.bw_block_decode_noalloc(x, w, kp, vp, sl, ns, pos, H, out)
    assert_same(_bits(out), _bits(ref), "x_out (no-alloc vs caller workspace)")
    for name, a, b in (("K", kp, kp_ref), ("V", vp, vp_ref)):
        for part, ta, tb in zip(("p3", "s3", "p4", "s4"), a, b):
            assert_same(_bits(ta), _bits(tb), f"{name} cache {part}")


def test_no_alloc_matches_caller_workspace_two_calls():
    # 7B attention shape (32 heads of 128, FFN 11008), 8 sequences, 1024-position cache
    _compare(synth.SEED_BASE + 120, B=8, H=32, D=128, F=11008, S_cap=1024, pos=1000)
    # then a smaller layer: fewer sequences, heads, positions and a narrower FFN
    _compare(synth.SEED_BASE + 121, B=3, H=2, D=64, F=256, S_cap=40, pos=5)
