"""GPU parity: the 4-bit quantizer and W1.58A4 BitLinear in one call
(bw_quantize_bitlinear_a4) vs the oracle.

For one or two tokens (K <= 8192) every workgroup of the single launch
quantizes the tokens itself; otherwise the call makes the two launches of the
separate calls.  Either way: codes and scales bit-exact against the oracle's
quantizer, acc (int32, or fp32 for e2m1) bit-exact against the oracle's exact
contraction, y within 1e-5 relative of the fp64 epilogue, and y, codes and
scales bit-identical to bw_quantize followed by bw_bitlinear_a4."""
import numpy as np
import pytest
import torch

import synth
import ternary_weight_bit_amd as bw
from oracle import act4, bitlinear, ternary
from tests.gpu_helpers import assert_rel, assert_same, bf16_dev, f32_dev, host

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def packed_weights(seed, N, K):
    w = synth.weight_tensor(seed, N, K)
    p, b = bw.bw_pack_ternary(f32_dev(w), bw.BW_ROLE_A4)
    t, beta = ternary.quantize_weights(w)
    return (p, b), t, np.full(N, beta, np.float32)


def check(x_dev, x32, fmt, wts, label):
    (p, b), t, beta = wts
    M = x32.shape[0]
    N = t.shape[0]
    print(f"case {label}: M={M} K={x32.shape[1]} N={N} fmt={fmt} dtype={x_dev.dtype}", flush=True)
    acc = torch.empty((M, N), dtype=torch.int32 if fmt == bw.BW_ACT_INT4 else torch.float32, device=DEV)
    y, codes, scales = bw.bw_quantize_bitlinear_a4(x_dev, fmt, p, b, acc_dbg=acc)
    if fmt == bw.BW_ACT_INT4:
        q, s = act4.quantize_int4(x32)
        ra = bitlinear.contract(q, t)
        rdt = np.int32
    else:
        q, s = act4.quantize_fp4(x32)
        ra = bitlinear.contract_e2m1_doubled(q, t) / 2.0
        rdt = np.float32
    assert_same(host(codes), act4.pack_nibbles(q), f"{label} codes")
    assert_same(host(scales).view(np.uint32), s.view(np.uint32), f"{label} scales")
    assert_same(host(acc), ra.astype(rdt), f"{label} acc")
    assert_rel(host(y), bitlinear.epilogue(ra, s, beta), 1e-5, f"{label} y")
    # the separate calls give the same bytes
    c2, s2 = bw.bw_quantize(x_dev, fmt)
    y2 = bw.bw_bitlinear_a4(c2, s2, fmt, p, b)
    assert_same(host(y).view(np.uint32), host(y2).view(np.uint32), f"{label} y vs separate calls")


FMTS = [bw.BW_ACT_INT4, bw.BW_ACT_FP4_E2M1]


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("M,K,N", [(1, 64, 16), (2, 64, 48), (1, 320, 32), (2, 2048, 64), (1, 2112, 80),
                                   (2, 4160, 32), (1, 6144, 16), (2, 8192, 48), (1, 8256, 32), (3, 4096, 64),
                                   (16, 1024, 32), (17, 512, 16)])
def test_ragged_shapes_bf16(fmt, M, K, N):
    """One launch for M <= 2 and K <= 8192 (1 to 4 chunks of 2048 per thread and
    ragged chunk counts), two launches beyond (K = 8256, M = 3, 16, 17)."""
    x = synth.to_bf16(synth.normal(11 * M + K + N, (M, K)) * np.float32(2.0))
    check(bf16_dev(x), x.f32, fmt, packed_weights(K + N, N, K), f"bf16 {M}x{K}x{N}")


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("M,K", [(1, 4096), (2, 4096), (2, 192), (5, 4096)])
def test_fp32_input(fmt, M, K):
    x = synth.normal(3 * M + K, (M, K))
    check(f32_dev(x), x, fmt, packed_weights(K + 1, 128, K), f"fp32 {M}x{K}")


@pytest.mark.parametrize("fmt", FMTS)
def test_edge_rows(fmt):
    """Rows whose scale or codes sit on an edge, two at a time through the single
    launch: zeros (the 1e-5 floor), a constant, tiny and huge magnitudes, exact
    INT4 halves, the e2m1 tie table, negative zeros."""
    K = 128
    rows = [
        np.zeros(K),
        np.full(K, -2.5),
        np.where(np.arange(K) % 2, 1e-30, -1e-30),
        np.where(np.arange(K) % 3 == 0, 3e30, 1.0),
        np.linspace(-7, 7, K),
        np.tile([6, 0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0], K // 8) * np.where(np.arange(K) % 2, 1, -1),
        np.r_[[-0.0] * (K // 2), [1e-5] * (K // 2)],
        np.r_[[7.0], np.full(K - 1, 3.5)],
    ]
    x = np.array(rows, dtype=np.float32)
    wts = packed_weights(5, 32, K)
    for i in range(0, len(rows), 2):
        check(f32_dev(x[i : i + 2]), x[i : i + 2], fmt, wts, f"edge rows {i}-{i + 1}")


@pytest.mark.parametrize("parts", [synth.QKV_PARTS, synth.GATE_UP_PARTS])
@pytest.mark.parametrize("M", [1, 2])
def test_decode_shapes(parts, M):
    """The fused q/k/v (N = 12288) and gate/up (N = 22016) shapes at K = 4096 with
    the outlier-channel decode activations, INT4 and e2m1."""
    N = sum(parts)
    K = synth.HIDDEN
    ws = synth.fused_weights(synth.SEED_BASE + 21, parts, K)
    p = torch.empty(N * K // 4, dtype=torch.uint8, device=DEV)
    b = torch.empty(N, dtype=torch.float32, device=DEV)
    ts, bs = [], []
    off = 0
    for w in ws:
        n = w.shape[0]
        bw.bw_pack_ternary(f32_dev(w), bw.BW_ROLE_A4, p[off * K // 4 : (off + n) * K // 4], b[off : off + n])
        t, beta = ternary.quantize_weights(w)
        ts.append(t)
        bs.append(np.full(n, beta, np.float32))
        off += n
    x = synth.decode_activations(seed=synth.SEED_BASE + 60 + M, M=M)
    for fmt in FMTS:
        check(bf16_dev(x), x.f32, fmt, ((p, b), np.concatenate(ts), np.concatenate(bs)), f"decode N={N}")


def test_empty_batch():
    (p, b), _, _ = packed_weights(1, 16, 64)
    x = torch.empty((0, 64), dtype=torch.bfloat16, device=DEV)
    y, codes, scales = bw.bw_quantize_bitlinear_a4(x, bw.BW_ACT_INT4, p, b)
    assert y.shape == (0, 16) and codes.shape == (0, 32)
