"""GPU: the calls on empty inputs (no token rows, no sequences, no positions, no bytes)
return OK without touching any output that has elements (checked against sentinel
bytes), and a call on real data right after still matches the oracle."""
import numpy as np
import pytest
import torch

import synth
import ternary_weight_bit_amd as bw
from oracle import act4, bitlinear, ternary
from tests.gpu_helpers import assert_rel, assert_same, bf16_dev, f32_dev, host

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def packed(role, N=32, K=128, seed=3):
    w = synth.weight_tensor(seed, N, K)
    return bw.bw_pack_ternary(f32_dev(w), role), w


def test_bitlinear_a4_no_rows():
    (p, b), _ = packed(bw.BW_ROLE_A4)
    for fmt in (bw.BW_ACT_INT4, bw.BW_ACT_FP4_E2M1):
        codes = torch.empty((0, 64), dtype=torch.uint8, device=DEV)
        scales = torch.empty(0, dtype=torch.float32, device=DEV)
        y = bw.bw_bitlinear_a4(codes, scales, fmt, p, b)
        assert y.shape == (0, 32)


def test_sparse_a8_front_end_and_products_no_rows():
    (p, b), _ = packed(bw.BW_ROLE_A8)
    (pk, bk), _ = packed(bw.BW_ROLE_A8_KMAJOR)
    for dt in (torch.bfloat16, torch.float32):
        g = torch.empty((0, 128), dtype=dt, device=DEV)
        for up in (None, torch.empty((0, 128), dtype=dt, device=DEV)):
            codes, scales = bw.bw_quantize_sparse_a8(g, up)
            assert codes.shape == (0, 128) and scales.shape == (0,)
    codes = torch.empty((0, 128), dtype=torch.int8, device=DEV)
    scales = torch.empty(0, dtype=torch.float32, device=DEV)
    assert bw.bw_bitlinear_sparse_a8(codes, scales, p, b).shape == (0, 32)
    ws = torch.empty(max(bw.bw_bitlinear_sparse_a8_gather_workspace_bytes(1, 128, 32), 16), dtype=torch.uint8,
                     device=DEV)
    y = torch.empty((0, 32), dtype=torch.float32, device=DEV)
    assert bw.bw_bitlinear_sparse_a8_gather(codes, scales, pk, bk, ws, y).shape == (0, 32)


@pytest.mark.parametrize("B,S", [(0, 16), (2, 0)])
def test_kv_codec_no_vectors(B, S):
    """No sequences or no positions: the 4-bit side slab (which has elements) keeps its bytes."""
    H, D, n_special = 2, 64, 3
    kv = torch.empty((B, S, H, D), dtype=torch.bfloat16, device=DEV)
    slot = torch.empty((B, S), dtype=torch.int32, device=DEV)
    p3 = torch.empty((B, S, H, 3 * D // 8), dtype=torch.uint8, device=DEV)
    s3 = torch.empty((B, S, H), dtype=torch.float32, device=DEV)
    p4 = torch.full((n_special, H, D // 2), 0xA5, dtype=torch.uint8, device=DEV)
    s4 = torch.full((n_special, H), 7.0, dtype=torch.float32, device=DEV)
    bw.bw_kv_pack3(kv, slot, n_special, p3, s3, p4, s4)
    out = bw.bw_kv_unpack3(p3, s3, p4, s4, slot, n_special, out_dtype=torch.float32)
    assert out.shape == (B, S, H, D)
    torch.cuda.synchronize()
    assert bool((p4 == 0xA5).all()) and bool((s4 == 7.0).all())


def test_attention_no_sequences():
    H, D, S = 2, 64, 8
    q = torch.empty((0, H, D), dtype=torch.float32, device=DEV)
    pack = (torch.empty((0, S, H, 3 * D // 8), dtype=torch.uint8, device=DEV),
            torch.empty((0, S, H), dtype=torch.float32, device=DEV), None, None)
    slot = torch.empty((0, S), dtype=torch.int32, device=DEV)
    ws = torch.empty(16, dtype=torch.uint8, device=DEV)
    out = bw.bw_attn_decode_kv3(q, pack, pack, slot, 0, workspace=ws)
    assert out.shape == (0, H, D)


def test_stream_read_no_bytes():
    sink = torch.full((8,), 0x5A5A5A5A, dtype=torch.int32, device=DEV)
    bw.bw_stream_read(torch.empty(0, dtype=torch.uint8, device=DEV), sink)
    torch.cuda.synchronize()
    assert bool((sink == 0x5A5A5A5A).all())


def test_real_call_after_empty_calls():
    """A quantizer + GEMV call on real rows right after the empty calls matches the oracle."""
    (p, b), w = packed(bw.BW_ROLE_A4, N=48, K=256, seed=9)
    bw.bw_bitlinear_a4(torch.empty((0, 128), dtype=torch.uint8, device=DEV),
                       torch.empty(0, dtype=torch.float32, device=DEV), bw.BW_ACT_INT4, p, b)
    x = synth.to_bf16(synth.normal(41, (3, 256)))
    y, codes, scales = bw.bw_quantize_bitlinear_a4(bf16_dev(x), bw.BW_ACT_INT4, p, b)
    q, s = act4.quantize_int4(x.f32)
    assert_same(host(codes), act4.pack_nibbles(q), "codes")
    t, beta = ternary.quantize_weights(w)
    ref = bitlinear.epilogue(bitlinear.contract(q, t), s, np.full(48, beta, np.float32))
    assert_rel(host(y), ref, 1e-5, "y after empty calls")
