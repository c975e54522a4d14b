"""GPU parity: W1.58A4 and W1.58A8 contractions vs the oracle.

acc (int32, or fp32 for e2m1 codes) must be bit-exact; y within 1e-5 relative.
The GPU contraction is fed the GPU quantizer's codes and packer's bytes, which
the quantizer/packer tests pin bit-exact to the oracle; the oracle side runs
from the raw activations and weights."""
import numpy as np
import pytest
import torch

import synth
import ternary_weight_bit_amd as bw
from oracle import act4, bitlinear, sparse8, ternary
from tests.gpu_helpers import assert_rel, assert_same, bf16_dev, f32_dev, host

pytestmark = pytest.mark.gpu


def run_a4(x_dev, w_dev, fmt, with_acc=True):
    codes, scales = bw.bw_quantize(x_dev, fmt)
    packed, beta = bw.bw_pack_ternary(w_dev, bw.BW_ROLE_A4)
    M = x_dev.shape[0]
    N = w_dev.shape[0]
    acc = None
    if with_acc:
        acc = torch.empty((M, N), dtype=torch.int32 if fmt == bw.BW_ACT_INT4 else torch.float32, device="cuda:0")
    y = bw.bw_bitlinear_a4(codes, scales, fmt, packed, beta, acc_dbg=acc)
    return y, acc


def oracle_a4(x32, w32, fmt):
    t, b = ternary.quantize_weights(w32)
    beta = np.full(w32.shape[0], b, np.float32)
    if fmt == bw.BW_ACT_INT4:
        _, _, acc, y = bitlinear.bitlinear_a4_int4(x32, t, beta)
    else:
        _, _, acc, y = bitlinear.bitlinear_a4_fp4(x32, t, beta)
    return acc, y


@pytest.mark.parametrize("fmt", [bw.BW_ACT_INT4, bw.BW_ACT_FP4_E2M1])
def test_small_bitlinear_m16_k256_n256(fmt):
    x, w = synth.small_bitlinear()
    y, acc = run_a4(f32_dev(x), f32_dev(w), fmt)
    ref_acc, ref_y = oracle_a4(x, w, fmt)
    if fmt == bw.BW_ACT_INT4:
        assert_same(host(acc), ref_acc.astype(np.int32), "acc int4")
    else:
        assert_same(host(acc), ref_acc.astype(np.float32), "acc fp4")
    assert_rel(host(y), ref_y)


@pytest.mark.parametrize("fmt", [bw.BW_ACT_INT4, bw.BW_ACT_FP4_E2M1])
@pytest.mark.parametrize("M,K,N", [(1, 64, 16), (37, 320, 208), (130, 1024, 144), (200, 256, 400), (8, 4096, 512),
                                   (9, 320, 48), (16, 1088, 32), (17, 512, 64), (3, 11008, 64), (300, 11008, 272),
                                   (40, 384, 96), (33, 1152, 272)])
def test_ragged_shapes(fmt, M, K, N):
    """K = 320 takes the register-staged kernel, K = 384 and 1152 the 128-k LDS kernel,
    other multiples of 256 the 256-k one (an odd stage count at K = 11008); M <= 16 the GEMV."""
    x = synth.to_bf16(synth.normal(M + 3 * K + N, (M, K)))
    w = synth.to_bf16(synth.normal(N + 5 * K, (N, K), 0.02))
    y, acc = run_a4(bf16_dev(x), bf16_dev(w), fmt)
    ref_acc, ref_y = oracle_a4(x.f32, w.f32, fmt)
    dt = np.int32 if fmt == bw.BW_ACT_INT4 else np.float32
    assert_same(host(acc), ref_acc.astype(dt), f"acc {M}x{K}x{N}")
    assert_rel(host(y), ref_y)


@pytest.mark.parametrize("fmt", [bw.BW_ACT_INT4, bw.BW_ACT_FP4_E2M1])
def test_extreme_codes(fmt):
    """Saturated codes (+-7 / +-6) against all-+1 and all--1 weights: largest |acc|."""
    M, K, N = 32, 4096, 32
    x = np.where(np.arange(K) % 2, 1.0, -1.0).astype(np.float32) * np.ones((M, 1), np.float32)
    x[1::2] = np.abs(x[1::2])
    w = np.ones((N, K), np.float32)
    w[N // 2 :] = -1.0
    y, acc = run_a4(f32_dev(x), f32_dev(w), fmt)
    ref_acc, ref_y = oracle_a4(x, w, fmt)
    dt = np.int32 if fmt == bw.BW_ACT_INT4 else np.float32
    assert_same(host(acc), ref_acc.astype(dt), "extreme acc")
    assert_rel(host(y), ref_y)


def test_decode_qkv_shape():
    """M in 1..8 at the fused q/k/v shape K=4096, N=3*4096 (all columns)."""
    ws = synth.fused_weights(synth.SEED_BASE + 21, synth.QKV_PARTS, synth.HIDDEN)
    N = sum(synth.QKV_PARTS)
    packed = torch.empty(N * synth.HIDDEN // 4, dtype=torch.uint8, device="cuda:0")
    beta = torch.empty(N, dtype=torch.float32, device="cuda:0")
    ts, bs = [], []
    off = 0
    for w in ws:
        n = w.shape[0]
        bw.bw_pack_ternary(f32_dev(w), bw.BW_ROLE_A4, packed[off * synth.HIDDEN // 4 : (off + n) * synth.HIDDEN // 4],
                           beta[off : off + n])
        t, b = ternary.quantize_weights(w)
        ts.append(t)
        bs.append(np.full(n, b, np.float32))
        off += n
    t = np.concatenate(ts)
    bref = np.concatenate(bs)
    assert_same(host(beta).view(np.uint32), bref.view(np.uint32), "qkv beta")
    for M in (1, 2, 4, 8):
        x = synth.decode_activations(seed=synth.SEED_BASE + 40 + M, M=M)
        for fmt in (bw.BW_ACT_INT4, bw.BW_ACT_FP4_E2M1):
            codes, scales = bw.bw_quantize(bf16_dev(x), fmt)
            acc = torch.empty((M, N), dtype=torch.int32 if fmt == bw.BW_ACT_INT4 else torch.float32, device="cuda:0")
            y = bw.bw_bitlinear_a4(codes, scales, fmt, packed, beta, acc_dbg=acc)
            if fmt == bw.BW_ACT_INT4:
                q, s = act4.quantize_int4(x.f32)
                ra = bitlinear.contract(q, t)
                assert_same(host(acc), ra.astype(np.int32), f"decode M={M} int4 acc")
            else:
                c, s = act4.quantize_fp4(x.f32)
                ra = bitlinear.contract_e2m1_doubled(c, t) / 2.0
                assert_same(host(acc), ra.astype(np.float32), f"decode M={M} fp4 acc")
            assert_rel(host(y), bitlinear.epilogue(ra, s, bref))


def test_prefill_full_shape_sampled():
    """M=2048, K=4096, N=11008, in the launch configuration the benchmark times;
    checked on 96 sampled rows (all columns) against the oracle."""
    M, K, N = 2048, 4096, 11008
    x = synth.prefill_activations(M=M, K=K)
    w = synth.weight_tensor(synth.SEED_BASE + 12, N, K)
    t, b = ternary.quantize_weights(w)
    rows = np.sort(np.random.default_rng(5).choice(M, size=96, replace=False))
    xd, wd = bf16_dev(x), f32_dev(w)
    packed, beta = bw.bw_pack_ternary(wd, bw.BW_ROLE_A4)
    del wd
    for fmt in (bw.BW_ACT_INT4, bw.BW_ACT_FP4_E2M1):
        codes, scales = bw.bw_quantize(xd, fmt)
        acc = torch.empty((M, N), dtype=torch.int32 if fmt == bw.BW_ACT_INT4 else torch.float32, device="cuda:0")
        y = bw.bw_bitlinear_a4(codes, scales, fmt, packed, beta, acc_dbg=acc)
        ga, gy = host(acc)[rows], host(y)[rows]
        if fmt == bw.BW_ACT_INT4:
            q, s = act4.quantize_int4(x.f32[rows])
            ra = bitlinear.contract(q, t)
            assert_same(ga, ra.astype(np.int32), "prefill int4 acc")
        else:
            c, s = act4.quantize_fp4(x.f32[rows])
            ra = bitlinear.contract_e2m1_doubled(c, t) / 2.0
            assert_same(ga, ra.astype(np.float32), "prefill fp4 acc")
        assert_rel(gy, bitlinear.epilogue(ra, s, np.full(N, b, np.float32)))


# ---------------------------------------------------------------- W1.58A8
@pytest.mark.parametrize("M,K,N", [(16, 256, 256), (37, 320, 208), (64, 11008, 256), (130, 4096, 144),
                                   (1, 11008, 4096), (8, 11008, 512), (5, 4096, 208)])
def test_a8_small(M, K, N):
    g, u = synth.gate_up(seed=M + K, M=M, K=K)
    w = synth.to_bf16(synth.normal(N + K, (N, K), 0.02))
    codes, scales = bw.bw_quantize_sparse_a8(bf16_dev(g), bf16_dev(u), K // 2)
    packed, beta = bw.bw_pack_ternary(bf16_dev(w), bw.BW_ROLE_A8)
    acc = torch.empty((M, N), dtype=torch.int32, device="cuda:0")
    y = bw.bw_bitlinear_sparse_a8(codes, scales, packed, beta, acc_dbg=acc)
    _, _, q, s = sparse8.sparse_a8(g.f32, u.f32, K // 2)
    t, b = ternary.quantize_weights(w.f32)
    ra = bitlinear.contract(q, t)
    assert_same(host(acc), ra.astype(np.int32), f"a8 acc {M}x{K}x{N}")
    assert_rel(host(y), bitlinear.epilogue(ra, s, np.full(N, b, np.float32)))


def test_a8_extreme_codes():
    M, K, N = 32, 11008, 32
    h = np.where(np.arange(K) % 2, 5.0, -5.0).astype(np.float32) * np.ones((M, 1), np.float32)
    w = np.ones((N, K), np.float32)
    w[::2] = -1.0
    codes, scales = bw.bw_quantize_sparse_a8(f32_dev(h), None, K)
    packed, beta = bw.bw_pack_ternary(f32_dev(w), bw.BW_ROLE_A8)
    acc = torch.empty((M, N), dtype=torch.int32, device="cuda:0")
    bw.bw_bitlinear_sparse_a8(codes, scales, packed, beta, acc_dbg=acc)
    _, _, q, _ = sparse8.sparse_a8(h, None, K)
    t, _ = ternary.quantize_weights(w)
    assert_same(host(acc), bitlinear.contract(q, t).astype(np.int32), "a8 extreme acc")


# ---------------------------------------------------------------- b1.58 baseline path
@pytest.mark.parametrize("M,K,N", [(37, 4096, 208), (5, 16384, 144), (130, 4096, 272), (260, 4096, 144)])
def test_b158_int8_keep_all(M, K, N):
    """BitNet b1.58's activation path, which a4.8 is compared against: INT8 absmax of every
    entry (the sparse front end with k = K, no top-k), then the W1.58A8 contraction.  260
    rows of 4096 take the one-wave-per-row front end, the other shapes a workgroup per row."""
    x = synth.prefill_activations(seed=M + K + N, M=M, K=K)
    w = synth.to_bf16(synth.normal(N + 3 * K, (N, K), 0.02))
    codes, scales = bw.bw_quantize_sparse_a8(bf16_dev(x), None, K)
    packed, beta = bw.bw_pack_ternary(bf16_dev(w), bw.BW_ROLE_A8)
    acc = torch.empty((M, N), dtype=torch.int32, device="cuda:0")
    y = bw.bw_bitlinear_sparse_a8(codes, scales, packed, beta, acc_dbg=acc)
    _, keep, q, s = sparse8.sparse_a8(x.f32, None, K)
    assert keep.all()
    assert_same(host(codes), q, f"b1.58 int8 codes {M}x{K}")
    assert_same(host(scales).view(np.uint32), s.view(np.uint32), f"b1.58 int8 scales {M}x{K}")
    t, b = ternary.quantize_weights(w.f32)
    ra = bitlinear.contract(q, t)
    assert_same(host(acc), ra.astype(np.int32), f"b1.58 acc {M}x{K}x{N}")
    assert_rel(host(y), bitlinear.epilogue(ra, s, np.full(N, b, np.float32)))
