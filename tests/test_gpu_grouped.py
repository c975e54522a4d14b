"""GPU parity: several BitLinear products over one set of codes in one call.

Each product of a grouped call must equal the single-product call bit for bit
(y and accumulators), and the single-product calls are pinned to the oracle by
test_gpu_bitlinear.py; one small case per path is also checked against the
oracle directly.  Shapes cover the one-launch grid (M > 16, K % 128 == 0: the
256-k kernel, the 128-k kernel at K = 384 and 1152, the INT8 kernel), products
of different and ragged N, one to four products, the per-product fallback
(M <= 16, and K % 128 != 0), no tokens, and the prefill shapes of the bench
(M = 2048, K = 4096, N = 11008 and 4096)."""
import numpy as np
import pytest
import torch

import synth
import ternary_weight_bit_amd as bw
from oracle import act4, bitlinear, sparse8, ternary
from tests.gpu_helpers import assert_rel, assert_same, bf16_dev, host

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def a4_products(M, K, Ns, fmt, seed):
    x = synth.to_bf16(synth.normal(seed, (M, K)))
    codes, scales = bw.bw_quantize(bf16_dev(x), fmt)
    ws = [synth.to_bf16(synth.normal(seed + 7 * i + N, (N, K), 0.02)) for i, N in enumerate(Ns)]
    packed = [bw.bw_pack_ternary(bf16_dev(w), bw.BW_ROLE_A4) for w in ws]
    return x, ws, codes, scales, packed


def oracle_a4(x32, w32, fmt):
    t, b = ternary.quantize_weights(w32)
    beta = np.full(w32.shape[0], b, np.float32)
    if fmt == bw.BW_ACT_INT4:
        _, _, acc, y = bitlinear.bitlinear_a4_int4(x32, t, beta)
    else:
        _, _, acc, y = bitlinear.bitlinear_a4_fp4(x32, t, beta)
    return acc, y


def acc_like(M, N, fmt):
    return torch.empty((M, N), dtype=torch.int32 if fmt == bw.BW_ACT_INT4 else torch.float32, device=DEV)


@pytest.mark.parametrize("fmt", [bw.BW_ACT_INT4, bw.BW_ACT_FP4_E2M1])
@pytest.mark.parametrize("M,K,Ns", [(300, 1024, (272, 4096)), (130, 256, (208, 144, 512)),
                                    (40, 384, (96, 256, 16, 4112)), (33, 1152, (272,)),
                                    (17, 4096, (4096, 11008)), (16, 4096, (4096, 272)), (300, 320, (208, 96)),
                                    (8, 11008, (64, 128))])
def test_a4_grouped_equals_single_calls(fmt, M, K, Ns):
    _, _, codes, scales, packed = a4_products(M, K, Ns, fmt, seed=M + K)
    accs = [acc_like(M, N, fmt) for N in Ns]
    ys = bw.bw_bitlinear_a4_grouped(codes, scales, fmt, packed, accs=accs)
    for i, ((p, b), N) in enumerate(zip(packed, Ns)):
        acc1 = acc_like(M, N, fmt)
        y1 = bw.bw_bitlinear_a4(codes, scales, fmt, p, b, acc_dbg=acc1)
        assert_same(host(accs[i]), host(acc1), f"grouped acc {i} {M}x{K}x{N}")
        assert_same(host(ys[i]).view(np.uint32), host(y1).view(np.uint32), f"grouped y {i} {M}x{K}x{N}")


@pytest.mark.parametrize("fmt", [bw.BW_ACT_INT4, bw.BW_ACT_FP4_E2M1])
def test_a4_grouped_vs_oracle(fmt):
    M, K, Ns = 70, 512, (144, 48)
    x, ws, codes, scales, packed = a4_products(M, K, Ns, fmt, seed=11)
    accs = [acc_like(M, N, fmt) for N in Ns]
    ys = bw.bw_bitlinear_a4_grouped(codes, scales, fmt, packed, accs=accs)
    for i, w in enumerate(ws):
        ref_acc, ref_y = oracle_a4(x.f32, w.f32, fmt)
        dt = np.int32 if fmt == bw.BW_ACT_INT4 else np.float32
        assert_same(host(accs[i]), ref_acc.astype(dt), f"grouped acc {i} vs oracle")
        assert_rel(host(ys[i]), ref_y)


@pytest.mark.parametrize("M,K,Ns", [(300, 4096, (272, 4096)), (130, 11008, (208, 144, 512)),
                                    (260, 384, (96, 16, 4112)), (9, 4096, (208, 96))])
def test_a8_grouped_equals_single_calls(M, K, Ns):
    x = synth.prefill_activations(seed=M + K, M=M, K=K)
    codes, scales = bw.bw_quantize_sparse_a8(bf16_dev(x), None, K)
    ws = [synth.to_bf16(synth.normal(3 * i + N + K, (N, K), 0.02)) for i, N in enumerate(Ns)]
    packed = [bw.bw_pack_ternary(bf16_dev(w), bw.BW_ROLE_A8) for w in ws]
    accs = [torch.empty((M, N), dtype=torch.int32, device=DEV) for N in Ns]
    ys = bw.bw_bitlinear_sparse_a8_grouped(codes, scales, packed, accs=accs)
    for i, ((p, b), N) in enumerate(zip(packed, Ns)):
        acc1 = torch.empty((M, N), dtype=torch.int32, device=DEV)
        y1 = bw.bw_bitlinear_sparse_a8(codes, scales, p, b, acc_dbg=acc1)
        assert_same(host(accs[i]), host(acc1), f"grouped a8 acc {i} {M}x{K}x{N}")
        assert_same(host(ys[i]).view(np.uint32), host(y1).view(np.uint32), f"grouped a8 y {i} {M}x{K}x{N}")
    if M == 130:  # one case straight against the oracle
        _, _, q, s = sparse8.sparse_a8(x.f32, None, K)
        for i, w in enumerate(ws):
            t, b = ternary.quantize_weights(w.f32)
            ra = bitlinear.contract(q, t)
            assert_same(host(accs[i]), ra.astype(np.int32), f"grouped a8 acc {i} vs oracle")
            assert_rel(host(ys[i]), bitlinear.epilogue(ra, s, np.full(Ns[i], b, np.float32)))


def test_grouped_no_tokens():
    K, Ns = 256, (16, 32)
    ws = [bw.bw_pack_ternary(bf16_dev(synth.to_bf16(synth.normal(N, (N, K), 0.02))), bw.BW_ROLE_A4) for N in Ns]
    ys = [torch.full((0, N), 7.0, device=DEV) for N in Ns]
    codes = torch.empty((0, K // 2), dtype=torch.uint8, device=DEV)
    scales = torch.empty(0, dtype=torch.float32, device=DEV)
    out = bw.bw_bitlinear_a4_grouped(codes, scales, bw.BW_ACT_INT4, ws, ys=ys)
    assert [tuple(o.shape) for o in out] == [(0, 16), (0, 32)]


def test_a4_grouped_bench_shapes():
    """The prefill pair of the bench (M = 2048, K = 4096, N = 11008 and 4096) in one launch:
    equal to the single calls everywhere (compared on the GPU), and sampled rows against
    the oracle."""
    M, K, Ns = 2048, 4096, (11008, 4096)
    fmt = bw.BW_ACT_INT4
    x, ws, codes, scales, packed = a4_products(M, K, Ns, fmt, seed=5)
    ys = bw.bw_bitlinear_a4_grouped(codes, scales, fmt, packed)
    for i, ((p, b), N) in enumerate(zip(packed, Ns)):
        y1 = bw.bw_bitlinear_a4(codes, scales, fmt, p, b)
        assert torch.equal(ys[i].view(torch.int32), y1.view(torch.int32)), f"bench-shape product {i}"
    rows = np.array([0, 1, 127, 128, 1000, 2047])
    q, s = act4.quantize_int4(x.f32[rows])
    for i, w in enumerate(ws):
        t, b = ternary.quantize_weights(w.f32)
        ref = bitlinear.epilogue(bitlinear.contract(q, t), s, np.full(Ns[i], b, np.float32))
        assert_rel(host(ys[i])[rows], ref)
