"""GPU parity: the single-token gather product over K-major weights
(bw_bitlinear_sparse_a8_gather) vs the oracle's row-gather contraction.

acc (int32) bit-exact; y within 1e-5 relative of the fp64 epilogue, and
bit-identical to the tiled W1.58A8 path's y on the same codes (both round
fl(fl(acc * s) * beta) from the same exact acc).  Codes come from the GPU
sparsifier (pinned bit-exact to the oracle elsewhere) or are drawn directly;
weights are packed by the GPU packer in both layouts."""
import numpy as np
import pytest
import torch

import synth
import ternary_weight_bit_amd as bw
from oracle import bitlinear, ternary
from tests.gpu_helpers import assert_rel, assert_same, bf16_dev, f32_dev, host

pytestmark = pytest.mark.gpu


def workspace(M, K, N, fill=0):
    """Workspace for one call; filled with garbage on purpose (its contents on entry are ignored)."""
    return torch.full((bw.bw_bitlinear_sparse_a8_gather_workspace_bytes(M, K, N),), fill, dtype=torch.uint8,
                      device="cuda:0")


def gather(codes, scales, wk, beta, ws):
    M, _ = codes.shape
    N = beta.shape[0]
    acc = torch.empty((M, N), dtype=torch.int32, device="cuda:0")
    y = bw.bw_bitlinear_sparse_a8_gather(codes, scales, wk, beta, ws, acc_dbg=acc)
    return y, acc


def check(codes_h, scales_h, w32, label, ws=None, w_dev=None):
    """Run the gather product on codes_h [M][K] int8 and weights w32 [N][K]; compare with the
    oracle (acc exact, y to 1e-5) and with the tiled W1.58A8 path (y, acc identical)."""
    M, K = codes_h.shape
    N = w32.shape[0]
    wd = f32_dev(w32) if w_dev is None else w_dev
    wk, beta = bw.bw_pack_ternary(wd, bw.BW_ROLE_A8_KMAJOR)
    wt, _ = bw.bw_pack_ternary(wd, bw.BW_ROLE_A8)
    codes = torch.from_numpy(np.ascontiguousarray(codes_h)).to("cuda:0")
    scales = f32_dev(scales_h)
    ws = workspace(M, K, N, 0xA5) if ws is None else ws
    print(f"case {label}: M={M} K={K} N={N}", flush=True)
    y, acc = gather(codes, scales, wk, beta, ws)
    t, b = ternary.quantize_weights(w32)
    ra = bitlinear.contract_gather_kmajor(codes_h, ternary.pack(t, ternary.ROLE_A8_KMAJOR), N)
    assert_same(host(acc), ra.astype(np.int32), f"{label} acc")
    assert_rel(host(y), bitlinear.epilogue(ra, scales_h, np.full(N, b, np.float32)), what=f"{label} y")
    acc_t = torch.empty((M, N), dtype=torch.int32, device="cuda:0")
    y_t = bw.bw_bitlinear_sparse_a8(codes, scales, wt, beta, acc_dbg=acc_t)
    assert_same(host(y).view(np.uint32), host(y_t).view(np.uint32), f"{label} y vs tiled path")
    return y


def half_sparse_codes(seed, M, K, keep=0.5):
    r = synth.rng(seed)
    q = r.integers(-128, 128, size=(M, K)).astype(np.int8)
    for m in range(M):
        q[m, r.permutation(K)[: K - int(K * keep)]] = 0
    s = (r.uniform(0.5, 2.0, size=M) / 127).astype(np.float32)
    return q, s


@pytest.mark.parametrize("M,K,N", [(1, 256, 256), (1, 64, 16), (1, 320, 208), (1, 4096, 4096), (2, 1024, 528),
                                   (3, 11008, 1040), (1, 16384, 64), (1, 131072, 16)])
def test_ragged_shapes(M, K, N):
    q, s = half_sparse_codes(M * 7 + K + N, M, K)
    w = synth.weight_tensor(synth.SEED_BASE + 40 + N, N, K)
    check(q, s, w, f"ragged {M}x{K}x{N}")


def test_down_proj_decode_from_sparsifier():
    """The decode down_proj: ReLU^2(gate)*up of one token, top-k 50 %, INT8 (GPU
    sparsifier), then the gather product with the 4096 x 11008 down weights."""
    M, K, N = 1, 11008, 4096
    g, u = synth.gate_up(seed=synth.SEED_BASE + 41, M=M, K=K)
    codes, scales = bw.bw_quantize_sparse_a8(bf16_dev(g), bf16_dev(u), K // 2)
    q = host(codes)
    assert 0 < np.count_nonzero(q) <= K // 2
    w = synth.weight_tensor(synth.SEED_BASE + 42, N, K)
    check(q, host(scales), w, "down_proj decode")


def test_empty_and_full_rows():
    """All codes zero (y = 0 exactly, no rows read), every code nonzero, and rows at the
    code extremes, in one batch of tokens."""
    M, K, N = 4, 2048, 512
    q = np.zeros((M, K), np.int8)
    q[1] = np.where(np.arange(K) % 3 == 0, -128, 127)
    q[2, ::5] = -128
    q[3] = synth.rng(43).integers(1, 128, size=K).astype(np.int8)
    s = np.full(M, 1.0 / 127, np.float32)
    w = synth.weight_tensor(synth.SEED_BASE + 44, N, K)
    y = check(q, s, w, "empty/full")
    assert not y[0].any().item()


def test_field_bound_worst_case():
    """The largest segment (1024 inputs, 64 rows per row group) with every code -128: with
    every weight +1 the 16-bit accumulator fields reach -16384, the most negative they can
    be; with every weight -1 they stay 0 and the whole sum comes from the -sum(q) term."""
    M, K, N = 16, 16384, 16
    q = np.full((M, K), -128, np.int8)
    s = np.full(M, 1.0 / 127, np.float32)
    for sign in (1.0, -1.0):
        w = np.full((N, K), sign, np.float32)
        check(q, s, w, f"field bound {sign:+.0f}")


def test_workspace_reuse_across_shapes():
    """One workspace serves back-to-back calls of different K, N and M; each call's
    result is independent of what the previous call left in it."""
    shapes = [(1, 11008, 4096), (3, 4096, 1024), (1, 4096, 4096), (2, 192, 2048), (16, 4096, 4096)]
    ws = workspace(16, 11008, 4096, 0x5A)
    for i, (M, K, N) in enumerate(shapes):
        need = bw.bw_bitlinear_sparse_a8_gather_workspace_bytes(M, K, N)
        assert 0 < need <= ws.numel()
        q, s = half_sparse_codes(50 + i, M, K)
        w = synth.weight_tensor(synth.SEED_BASE + 50 + i, N, K)
        check(q, s, w, f"reuse {i}", ws=ws[:need])


def test_long_k_and_repeat():
    """K twice the sparsifier's row limit (32768: 128 segments of 256 inputs at M = 2,
    N = 96) and a second call on the same buffers: the two results must be identical."""
    M, K, N = 2, 32768, 96
    q, s = half_sparse_codes(61, M, K, keep=0.9)
    w = synth.weight_tensor(synth.SEED_BASE + 61, N, K)
    ws = workspace(M, K, N, 0x33)
    y1 = check(q, s, w, "long K", ws=ws)
    y2 = check(q, s, w, "long K repeat", ws=ws)
    assert torch.equal(y1, y2)
