"""GPU parity at the benchmark's full shapes, in the launch configurations bench.py
times, on sampled outputs the oracle computes row by row: the N = 4096 prefill GEMM,
the W1.58A8 down_proj and out_proj GEMMs fed by the top-k front end, and the fused
gate/up decode GEMV.  Integer accumulators bit-exact, y within 1e-5 relative."""
import numpy as np
import pytest
import torch

import synth
import ternary_weight_bit_amd as bw
from oracle import act4, bitlinear, sparse8, ternary
from tests.gpu_helpers import assert_rel, assert_same, bf16_dev, f32_dev, host

pytestmark = pytest.mark.gpu


def sample_rows(M, n, seed):
    return np.sort(np.random.default_rng(seed).choice(M, size=n, replace=False))


def test_prefill_n4096_full_shape_sampled():
    M, K, N = 2048, synth.HIDDEN, synth.HIDDEN
    x = synth.prefill_activations(seed=synth.SEED_BASE + 70, M=M, K=K)
    w = synth.weight_tensor(synth.SEED_BASE + 71, N, K)
    t, b = ternary.quantize_weights(w)
    rows = sample_rows(M, 96, 71)
    packed, beta = bw.bw_pack_ternary(f32_dev(w), bw.BW_ROLE_A4)
    xd = bf16_dev(x)
    for fmt in (bw.BW_ACT_INT4, bw.BW_ACT_FP4_E2M1):
        codes, scales = bw.bw_quantize(xd, fmt)
        acc = torch.empty((M, N), dtype=torch.int32 if fmt == bw.BW_ACT_INT4 else torch.float32, device="cuda:0")
        y = bw.bw_bitlinear_a4(codes, scales, fmt, packed, beta, acc_dbg=acc)
        ga, gy = host(acc)[rows], host(y)[rows]
        if fmt == bw.BW_ACT_INT4:
            q, s = act4.quantize_int4(x.f32[rows])
            ra = bitlinear.contract(q, t)
            assert_same(ga, ra.astype(np.int32), "prefill N=4096 int4 acc")
        else:
            c, s = act4.quantize_fp4(x.f32[rows])
            ra = bitlinear.contract_e2m1_doubled(c, t) / 2.0
            assert_same(ga, ra.astype(np.float32), "prefill N=4096 fp4 acc")
        assert_rel(gy, bitlinear.epilogue(ra, s, np.full(N, b, np.float32)))


@pytest.mark.parametrize("name", ["down_proj", "out_proj"])
def test_a8_full_shapes_sampled(name):
    """down_proj: ReLU^2(gate) * up, 2048 x 11008, top-k 5504, W [4096][11008];
    out_proj: Student-t(3) input, 2048 x 4096, top-k 2048, W [4096][4096]."""
    M, N = 2048, synth.HIDDEN
    if name == "down_proj":
        K = synth.FFN
        g, u = synth.gate_up(seed=synth.SEED_BASE + 72, M=M, K=K)
        gd, ud, g32, u32 = bf16_dev(g), bf16_dev(u), g.f32, u.f32
    else:
        K = synth.HIDDEN
        x = synth.heavy_tailed(seed=synth.SEED_BASE + 73, M=M, K=K)
        gd, ud, g32, u32 = bf16_dev(x), None, x.f32, None
    w = synth.weight_tensor(synth.SEED_BASE + 74 + K, N, K)
    t, b = ternary.quantize_weights(w)
    codes, scales = bw.bw_quantize_sparse_a8(gd, ud, K // 2)
    packed, beta = bw.bw_pack_ternary(f32_dev(w), bw.BW_ROLE_A8)
    acc = torch.empty((M, N), dtype=torch.int32, device="cuda:0")
    y = bw.bw_bitlinear_sparse_a8(codes, scales, packed, beta, acc_dbg=acc)
    rows = sample_rows(M, 64, K)
    _, _, q, s = sparse8.sparse_a8(g32[rows], None if u32 is None else u32[rows], K // 2)
    assert_same(host(codes)[rows], q, f"{name} codes")
    ra = bitlinear.contract(q, t)
    assert_same(host(acc)[rows], ra.astype(np.int32), f"{name} acc")
    assert_rel(host(y)[rows], bitlinear.epilogue(ra, s, np.full(N, b, np.float32)))


@pytest.mark.parametrize("M", [1, 8])
def test_decode_gate_up_shape(M):
    """Fused gate/up GEMV, K = 4096, N = 2 * 11008 (all columns), INT4 codes."""
    ws = synth.fused_weights(synth.SEED_BASE + 75, synth.GATE_UP_PARTS, synth.HIDDEN)
    N = sum(synth.GATE_UP_PARTS)
    packed = torch.empty(N * synth.HIDDEN // 4, dtype=torch.uint8, device="cuda:0")
    beta = torch.empty(N, dtype=torch.float32, device="cuda:0")
    ts, bs = [], []
    off = 0
    for w in ws:
        n = w.shape[0]
        bw.bw_pack_ternary(f32_dev(w), bw.BW_ROLE_A4, packed[off * synth.HIDDEN // 4 : (off + n) * synth.HIDDEN // 4],
                           beta[off : off + n])
        tt, bb = ternary.quantize_weights(w)
        ts.append(tt)
        bs.append(np.full(n, bb, np.float32))
        off += n
    t, bref = np.concatenate(ts), np.concatenate(bs)
    x = synth.decode_activations(seed=synth.SEED_BASE + 76 + M, M=M)
    codes, scales = bw.bw_quantize(bf16_dev(x), bw.BW_ACT_INT4)
    acc = torch.empty((M, N), dtype=torch.int32, device="cuda:0")
    y = bw.bw_bitlinear_a4(codes, scales, bw.BW_ACT_INT4, packed, beta, acc_dbg=acc)
    q, s = act4.quantize_int4(x.f32)
    ra = bitlinear.contract(q, t)
    assert_same(host(acc), ra.astype(np.int32), f"gate/up M={M} acc")
    assert_rel(host(y), bitlinear.epilogue(ra, s, bref))
