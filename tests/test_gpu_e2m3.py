"""GPU parity: INT4 activations stored as e2m3 (fp6) fields (BW_ACT_INT4_E2M3).

The quantizer's bytes equal the oracle's e2m3 storage of its INT4 codes (bit
for bit), and the products over them - the fp6 x fp4 matrix instruction -
equal the INT4 nibble path bit for bit (accumulators and y), which
test_gpu_bitlinear.py pins to the oracle; small cases are also checked
against the oracle directly.  Shapes cover K that is not a multiple of 256
(the last 256-k stage partly used), one to 300 tokens, ragged N, grouped
launches, the fused quantize + product call, and the prefill shapes of the
bench (M = 2048, K = 4096, N = 11008 and 4096)."""
import numpy as np
import pytest
import torch

import synth
import ternary_weight_bit_amd as bw
from oracle import act4, bitlinear, ternary
from tests.gpu_helpers import assert_rel, assert_same, bf16_dev, f32_dev, host

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
E6 = bw.BW_ACT_INT4_E2M3
I4 = bw.BW_ACT_INT4


@pytest.mark.parametrize("M,K", [(1, 64), (3, 192), (130, 1024), (7, 4096), (5, 8192), (4, 16384), (2, 131072)])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_quantize_e2m3_vs_oracle(M, K, dtype):
    x = synth.to_bf16(synth.normal(M * 7 + K, (M, K)) * np.float32(3.0))
    x32 = x.f32
    if M > 1:
        x32 = x32.copy()
        x32[1, ::7] *= np.float32(40.0)  # an outlier row
        x32[0, :] = np.float32(0.0)      # a zero row (every code 0)
        x = synth.to_bf16(x32) if dtype == "bf16" else None
        x32 = x.f32 if x is not None else x32
    dev = bf16_dev(x) if dtype == "bf16" else f32_dev(x32)
    codes, scales = bw.bw_quantize(dev, E6)
    assert tuple(codes.shape) == (M, K // 4 * 3)
    q, s = act4.quantize_int4(x32)
    assert_same(host(scales).view(np.uint32), s.view(np.uint32), f"e2m3 scales {M}x{K}")
    assert_same(host(codes), act4.pack_int4_e2m3(q), f"e2m3 codes {M}x{K}")


def e2m3_edge_rows(K: int) -> np.ndarray:
    """Rows whose scale is exactly 1 (row maximum 7), so that t = x: every halfway
    case of rne(t) of both signs, the values around -0.5 (the last t whose field is
    +0 and the first that is -1), negative zeros, fp32 subnormals of both signs;
    plus a zero row, a constant negative row, tiny and huge magnitudes."""
    halves = np.array([k + 0.5 for k in range(7)], np.float32)
    around = np.array([-0.5, np.nextafter(np.float32(-0.5), np.float32(-1)), np.nextafter(np.float32(-0.5), np.float32(0)),
                       -0.0, 0.0, 0.5, -1e-44, 1e-44, -0.25, -1.0, 1.0, -7.0], np.float32)
    ties = np.concatenate([[7.0], halves, -halves, around]).astype(np.float32)
    rows = [
        np.resize(ties, K),
        np.resize(ties[::-1], K),
        np.zeros(K),
        np.full(K, -2.5),
        np.where(np.arange(K) % 2, 1e-30, -1e-30),
        np.where(np.arange(K) % 3 == 0, 3e30, -1.0),
    ]
    return np.array(rows, dtype=np.float32)


@pytest.mark.parametrize("K", [64, 192, 4096, 16384])
def test_quantize_e2m3_edge_rows(K):
    """Ties, signs of zero fields and subnormals on the row kernel (K <= 8192) and
    the one-wave-per-row kernel (longer rows), bit for bit against the oracle."""
    x32 = e2m3_edge_rows(K)
    codes, scales = bw.bw_quantize(f32_dev(x32), E6)
    q, s = act4.quantize_int4(x32)
    assert_same(host(scales).view(np.uint32), s.view(np.uint32), f"e2m3 edge scales K={K}")
    assert_same(host(codes), act4.pack_int4_e2m3(q), f"e2m3 edge codes K={K}")


def a4_pair(M, K, N, seed):
    x = synth.to_bf16(synth.normal(seed, (M, K)))
    w = synth.to_bf16(synth.normal(seed + 1, (N, K), 0.02))
    packed, beta = bw.bw_pack_ternary(bf16_dev(w), bw.BW_ROLE_A4)
    c6, s6 = bw.bw_quantize(bf16_dev(x), E6)
    c4, s4 = bw.bw_quantize(bf16_dev(x), I4)
    return x, w, packed, beta, (c6, s6), (c4, s4)


SHAPES = [(1, 64, 16), (5, 192, 48), (17, 320, 272), (40, 384, 96), (33, 704, 208), (64, 1088, 96),
          (130, 1024, 4112), (300, 4096, 256), (129, 256, 16), (256, 11008, 144)]


@pytest.mark.parametrize("M,K,N", SHAPES)
def test_bitlinear_e2m3_equals_int4(M, K, N):
    _, _, packed, beta, (c6, s6), (c4, s4) = a4_pair(M, K, N, seed=M + K + N)
    acc6 = torch.empty((M, N), dtype=torch.int32, device=DEV)
    acc4 = torch.empty((M, N), dtype=torch.int32, device=DEV)
    y6 = bw.bw_bitlinear_a4(c6, s6, E6, packed, beta, acc_dbg=acc6)
    y4 = bw.bw_bitlinear_a4(c4, s4, I4, packed, beta, acc_dbg=acc4)
    assert_same(host(acc6), host(acc4), f"acc {M}x{K}x{N}")
    assert_same(host(y6).view(np.uint32), host(y4).view(np.uint32), f"y {M}x{K}x{N}")


@pytest.mark.parametrize("M,K,N", [(70, 512, 144), (9, 320, 48)])
def test_bitlinear_e2m3_vs_oracle(M, K, N):
    x, w, packed, beta, (c6, s6), _ = a4_pair(M, K, N, seed=3 * M + K)
    acc = torch.empty((M, N), dtype=torch.int32, device=DEV)
    y = bw.bw_bitlinear_a4(c6, s6, E6, packed, beta, acc_dbg=acc)
    t, b = ternary.quantize_weights(w.f32)
    _, _, ref_acc, ref_y = bitlinear.bitlinear_a4_int4(x.f32, t, np.full(N, b, np.float32))
    assert_same(host(acc), ref_acc.astype(np.int32), "acc vs oracle")
    assert_rel(host(y), ref_y)


def test_bitlinear_e2m3_extreme_codes():
    """Codes written directly (not by the quantizer): every value -8..7 in every
    position of a 64-k group, including -8, which absmax quantization never makes."""
    M, K, N = 48, 512, 64
    rs = np.random.default_rng(5)
    q = rs.integers(-8, 8, size=(M, K)).astype(np.int8)
    q[:16, :16] = np.arange(-8, 8)[None, :]
    q[16] = -8
    q[17] = 7
    c6 = torch.from_numpy(act4.pack_int4_e2m3(q)).to(DEV)
    c4 = torch.from_numpy(act4.pack_nibbles(q)).to(DEV)
    sx = f32_dev(rs.uniform(0.5, 2.0, M).astype(np.float32))
    w = synth.to_bf16(synth.normal(9, (N, K), 0.02))
    packed, beta = bw.bw_pack_ternary(bf16_dev(w), bw.BW_ROLE_A4)
    acc6 = torch.empty((M, N), dtype=torch.int32, device=DEV)
    acc4 = torch.empty((M, N), dtype=torch.int32, device=DEV)
    y6 = bw.bw_bitlinear_a4(c6, sx, E6, packed, beta, acc_dbg=acc6)
    y4 = bw.bw_bitlinear_a4(c4, sx, I4, packed, beta, acc_dbg=acc4)
    t, _ = ternary.quantize_weights(w.f32)
    assert_same(host(acc6), bitlinear.contract(q, t).astype(np.int32), "acc vs oracle contraction")
    assert_same(host(acc6), host(acc4), "acc e2m3 vs nibbles")
    assert_same(host(y6).view(np.uint32), host(y4).view(np.uint32), "y e2m3 vs nibbles")


def test_grouped_e2m3_equals_single_and_int4():
    M, K, Ns = 300, 1088, (272, 4096, 16)
    x = synth.to_bf16(synth.normal(21, (M, K)))
    ws = [bw.bw_pack_ternary(bf16_dev(synth.to_bf16(synth.normal(30 + N, (N, K), 0.02))), bw.BW_ROLE_A4) for N in Ns]
    c6, s6 = bw.bw_quantize(bf16_dev(x), E6)
    c4, s4 = bw.bw_quantize(bf16_dev(x), I4)
    accs = [torch.empty((M, N), dtype=torch.int32, device=DEV) for N in Ns]
    ys = bw.bw_bitlinear_a4_grouped(c6, s6, E6, ws, accs=accs)
    ys4 = bw.bw_bitlinear_a4_grouped(c4, s4, I4, ws)
    for i, ((p, b), N) in enumerate(zip(ws, Ns)):
        acc1 = torch.empty((M, N), dtype=torch.int32, device=DEV)
        y1 = bw.bw_bitlinear_a4(c6, s6, E6, p, b, acc_dbg=acc1)
        assert_same(host(accs[i]), host(acc1), f"grouped acc {i}")
        assert_same(host(ys[i]).view(np.uint32), host(y1).view(np.uint32), f"grouped y {i}")
        assert_same(host(ys[i]).view(np.uint32), host(ys4[i]).view(np.uint32), f"grouped y {i} vs INT4")


@pytest.mark.parametrize("M", [1, 2, 24])
def test_quantize_bitlinear_e2m3(M):
    K, N = 4096, 272
    x = synth.to_bf16(synth.normal(40 + M, (M, K)))
    w = synth.to_bf16(synth.normal(41, (N, K), 0.02))
    packed, beta = bw.bw_pack_ternary(bf16_dev(w), bw.BW_ROLE_A4)
    y6, c6, s6 = bw.bw_quantize_bitlinear_a4(bf16_dev(x), E6, packed, beta)
    y4, _, s4 = bw.bw_quantize_bitlinear_a4(bf16_dev(x), I4, packed, beta)
    q, s = act4.quantize_int4(x.f32)
    assert_same(host(c6), act4.pack_int4_e2m3(q), "fused e2m3 codes")
    assert_same(host(s6).view(np.uint32), host(s4).view(np.uint32), "fused scales")
    assert_same(host(y6).view(np.uint32), host(y4).view(np.uint32), "fused y vs INT4")


def test_e2m3_bench_shapes():
    """The prefill pair of the bench (M = 2048, K = 4096, N = 11008 and 4096) in one
    grouped launch: equal to the INT4 nibble path everywhere (compared on the GPU)."""
    M, K, Ns = 2048, 4096, (11008, 4096)
    x = synth.prefill_activations(seed=5, M=M, K=K)
    ws = [bw.bw_pack_ternary(bf16_dev(synth.to_bf16(synth.normal(50 + N, (N, K), 0.02))), bw.BW_ROLE_A4)
          for N in Ns]
    c6, s6 = bw.bw_quantize(bf16_dev(x), E6)
    c4, s4 = bw.bw_quantize(bf16_dev(x), I4)
    accs6 = [torch.empty((M, N), dtype=torch.int32, device=DEV) for N in Ns]
    accs4 = [torch.empty((M, N), dtype=torch.int32, device=DEV) for N in Ns]
    ys6 = bw.bw_bitlinear_a4_grouped(c6, s6, E6, ws, accs=accs6)
    ys4 = bw.bw_bitlinear_a4_grouped(c4, s4, I4, ws, accs=accs4)
    for i in range(2):
        assert torch.equal(accs6[i], accs4[i]), f"bench-shape acc {i}"
        assert torch.equal(ys6[i].view(torch.int32), ys4[i].view(torch.int32)), f"bench-shape y {i}"
    # sampled rows of the codes against the oracle
    rows = np.array([0, 1, 1000, 2047])
    q, _ = act4.quantize_int4(x.f32[rows])
    assert_same(host(c6)[rows], act4.pack_int4_e2m3(q), "bench-shape codes")


@pytest.mark.parametrize("M", [1, 8, 16])
@pytest.mark.parametrize("K,N", [(4096, 12288), (4096, 22016), (4160, 48), (11008, 4096)])
def test_e2m3_decode_gemv_equals_int4(M, K, N):
    """Decode shapes (M <= 16 tokens, the weight-streaming GEMV on the fp6 x fp4
    instruction): fused q/k/v and gate/up widths at K = 4096 with outlier channels,
    a K whose 65 tiles split unevenly over the waves, and K = 11008; accumulators
    and y equal the INT4 nibble path bit for bit."""
    x = synth.decode_activations(seed=700 + M + K, M=M, K=K)
    w = synth.weight_tensor(701 + N, N, K)
    packed, beta = bw.bw_pack_ternary(f32_dev(w), bw.BW_ROLE_A4)
    c6, s6 = bw.bw_quantize(bf16_dev(x), E6)
    c4, s4 = bw.bw_quantize(bf16_dev(x), I4)
    acc6 = torch.empty((M, N), dtype=torch.int32, device=DEV)
    acc4 = torch.empty((M, N), dtype=torch.int32, device=DEV)
    y6 = bw.bw_bitlinear_a4(c6, s6, E6, packed, beta, acc_dbg=acc6)
    y4 = bw.bw_bitlinear_a4(c4, s4, I4, packed, beta, acc_dbg=acc4)
    assert torch.equal(acc6, acc4), f"decode acc {M}x{K}x{N}"
    assert torch.equal(y6.view(torch.int32), y4.view(torch.int32)), f"decode y {M}x{K}x{N}"
    if N <= 4096:  # and the oracle on a few columns
        q, s = act4.quantize_int4(x.f32)
        t, b = ternary.quantize_weights(w)
        cols = np.array([0, 1, N // 2, N - 1])
        ref = bitlinear.contract(q, t[cols])
        assert_same(host(acc6)[:, cols], ref.astype(np.int32), f"decode acc vs oracle {M}x{K}x{N}")
