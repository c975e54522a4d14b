"""GPU parity: 4-bit activation quantizer (bw_quantize) vs the oracle, bit-exact."""
import numpy as np
import pytest
import torch

import synth
import ternary_weight_bit_amd as bw
from oracle import act4
from tests.gpu_helpers import assert_same, bf16_dev, f32_dev, host

pytestmark = pytest.mark.gpu

FMTS = [(bw.BW_ACT_INT4, "int4"), (bw.BW_ACT_FP4_E2M1, "fp4")]


def oracle_codes(x32, fmt):
    if fmt == bw.BW_ACT_INT4:
        q, s = act4.quantize_int4(x32)
    else:
        q, s = act4.quantize_fp4(x32)
    return act4.pack_nibbles(q), s


def check(x_dev, x32, fmt, label):
    codes, scales = bw.bw_quantize(x_dev, fmt)
    ref_c, ref_s = oracle_codes(x32, fmt)
    assert_same(host(scales).view(np.uint32), ref_s.view(np.uint32), f"{label} scales")
    assert_same(host(codes), ref_c, f"{label} codes")


@pytest.mark.parametrize("fmt,name", FMTS)
def test_small_bitlinear_inputs_fp32(fmt, name):
    x, _ = synth.small_bitlinear()
    check(f32_dev(x), x, fmt, f"fp32 16x256 {name}")


@pytest.mark.parametrize("fmt,name", FMTS)
@pytest.mark.parametrize("M", [1, 2, 4, 8])
def test_decode_bf16_outliers(fmt, name, M):
    x = synth.decode_activations(seed=synth.SEED_BASE + 1 + M, M=M)
    check(bf16_dev(x), x.f32, fmt, f"decode M={M} {name}")


@pytest.mark.parametrize("fmt,name", FMTS)
@pytest.mark.parametrize("M,K", [(37, 64), (3, 320), (130, 4096), (5, 12288), (2, 131072)])
def test_ragged_and_large_rows(fmt, name, M, K):
    x = synth.to_bf16(synth.normal(7 + M + K, (M, K)) * np.float32(3.0))
    check(bf16_dev(x), x.f32, fmt, f"bf16 {M}x{K} {name}")


@pytest.mark.parametrize("fmt,name", FMTS)
def test_edge_rows(fmt, name):
    K = 128
    rows = [
        np.zeros(K),                                  # all-zero row: scale from the 1e-5 floor
        np.full(K, -2.5),                             # constant row
        np.where(np.arange(K) % 2, 1e-30, -1e-30),    # tiny magnitudes
        np.where(np.arange(K) % 3 == 0, 3e30, 1.0),   # huge magnitudes
        np.linspace(-7, 7, K),                        # many exact halfway cases for INT4
        np.tile([6, 0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0], K // 8) * np.where(np.arange(K) % 2, 1, -1),
        np.r_[[-0.0] * (K // 2), [1e-5] * (K // 2)],  # negative zeros, row max at the floor
        np.r_[[7.0], np.full(K - 1, 3.5)],
        np.where(np.arange(K) % 2, 1e-44, -1e-44),    # fp32 subnormal inputs and products, both signs
    ]
    x = np.array(rows, dtype=np.float32)
    check(f32_dev(x), x, fmt, f"edge rows {name}")


@pytest.mark.parametrize("fmt,name", FMTS)
@pytest.mark.parametrize("M,K", [(1024, 64), (1027, 1088), (1030, 2048), (1025, 2112), (1029, 4096)])
def test_many_rows(fmt, name, M, K):
    """Over a thousand rows of up to 4096 entries (ragged chunk counts per thread),
    bf16 and fp32 inputs."""
    x = synth.to_bf16(synth.normal(17 + M + K, (M, K)) * np.float32(2.5))
    check(bf16_dev(x), x.f32, fmt, f"bf16 {M}x{K} {name}")
    check(f32_dev(x.f32), x.f32, fmt, f"fp32 {M}x{K} {name}")


@pytest.mark.parametrize("fmt,name", FMTS)
def test_edge_rows_many(fmt, name):
    """The edge rows repeated over 1161 rows."""
    K = 128
    base = np.array([
        np.zeros(K), np.full(K, -2.5), np.where(np.arange(K) % 2, 1e-30, -1e-30),
        np.where(np.arange(K) % 3 == 0, 3e30, 1.0), np.linspace(-7, 7, K),
        np.tile([6, 0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0], K // 8) * np.where(np.arange(K) % 2, 1, -1),
        np.r_[[-0.0] * (K // 2), [1e-5] * (K // 2)], np.r_[[7.0], np.full(K - 1, 3.5)],
        np.where(np.arange(K) % 2, 1e-44, -1e-44),
    ], dtype=np.float32)
    x = np.tile(base, (129, 1))
    check(f32_dev(x), x, fmt, f"edge rows x129 {name}")


def test_full_prefill_shape_sampled():
    """2048 x 4096 bf16: all scales, codes of 64 sampled rows."""
    x = synth.prefill_activations()
    xd = bf16_dev(x)
    for fmt, name in FMTS:
        codes, scales = bw.bw_quantize(xd, fmt)
        rows = np.random.default_rng(99).choice(2048, size=64, replace=False)
        ref_c, ref_s = oracle_codes(x.f32[rows], fmt)
        assert_same(host(codes)[rows], ref_c, f"prefill {name} codes")
        assert_same(host(scales)[rows].view(np.uint32), ref_s.view(np.uint32), f"prefill {name} scales")


def test_determinism():
    x = synth.prefill_activations(M=256)
    xd = bf16_dev(x)
    a, sa = bw.bw_quantize(xd, bw.BW_ACT_FP4_E2M1)
    b, sb = bw.bw_quantize(xd, bw.BW_ACT_FP4_E2M1)
    torch.cuda.synchronize()
    assert torch.equal(a, b) and torch.equal(sa, sb)


def test_empty_batch():
    x = torch.empty((0, 256), dtype=torch.bfloat16, device="cuda:0")
    codes, scales = bw.bw_quantize(x, bw.BW_ACT_INT4)
    assert codes.shape == (0, 128)
