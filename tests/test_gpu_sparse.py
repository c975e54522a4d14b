"""GPU parity: ReLU^2 + top-k + INT8 front end (bw_quantize_sparse_a8) vs the oracle, bit-exact."""
import numpy as np
import pytest
import torch

import synth
import ternary_weight_bit_amd as bw
from oracle import sparse8
from tests.gpu_helpers import assert_same, bf16_dev, f32_dev, host

pytestmark = pytest.mark.gpu


def run(g_dev, u_dev, k, M, K):
    mask = torch.empty((M, K // 32), dtype=torch.int32, device="cuda:0")
    codes, scales = bw.bw_quantize_sparse_a8(g_dev, u_dev, k, mask_dbg=mask)
    return host(codes), host(scales), host(mask).view(np.uint32)


def check(g_dev, u_dev, g32, u32, k, label):
    M, K = g32.shape
    c, s, m = run(g_dev, u_dev, k, M, K)
    _, keep, q, rs = sparse8.sparse_a8(g32, u32, k)
    assert_same(m, sparse8.mask_words(keep), f"{label} mask")
    assert_same(c, q, f"{label} codes")
    assert_same(s.view(np.uint32), rs.view(np.uint32), f"{label} scales")
    assert np.all(np.unpackbits(m.view(np.uint8), axis=1).sum(axis=1) == k)


@pytest.mark.parametrize("M,K", [(64, 11008), (7, 64), (33, 4096), (5, 16384), (3, 320), (4, 8192), (3, 6144)])
def test_relu2_gate_bf16(M, K):
    g, u = synth.gate_up(seed=M * 31 + K, M=M, K=K)
    check(bf16_dev(g), bf16_dev(u), g.f32, u.f32, K // 2, f"relu2 {M}x{K}")


@pytest.mark.parametrize("M,K", [(64, 4096), (9, 192)])
def test_out_proj_student_t(M, K):
    x = synth.heavy_tailed(seed=M + K, M=M, K=K)
    check(bf16_dev(x), None, x.f32, None, K // 2, f"out_proj {M}x{K}")


@pytest.mark.parametrize("k", [1, 2, 63, 64, 65, 2047, 4095, 4096])
@pytest.mark.parametrize("M", [6, 260])
def test_k_keep_range(k, M):
    K = 4096
    x = synth.heavy_tailed(seed=k, M=M, K=K)
    check(bf16_dev(x), None, x.f32, None, k, f"k={k}")


def tile_rows(a, reps):
    return None if a is None else np.ascontiguousarray(np.tile(a, (reps, 1)))


@pytest.mark.parametrize("reps", [1, 22])
def test_fp32_inputs_and_ties(reps):
    """reps = 22 gives 264 rows: rows of at most 4096 entries then go to the
    one-wave-per-row kernel (256 rows or fewer take a workgroup per row), so both
    selection kernels see every case."""
    M, K = 12, 1024
    rs = np.random.default_rng(3)
    g = rs.integers(-3, 4, size=(M, K)).astype(np.float32)  # heavy exact ties in |h|
    u = rs.integers(-2, 3, size=(M, K)).astype(np.float32)
    g[0] = 0.0  # all-zero row
    g[1] = 1.0
    u[1] = 1.0  # constant row: every key ties
    g[2] = -1.0  # ReLU kills the whole row
    g, u = tile_rows(g, reps), tile_rows(u, reps)
    for k in (1, K // 2, K - 1, K):
        check(f32_dev(g), f32_dev(u), g, u, k, f"ties k={k} reps={reps}")


@pytest.mark.parametrize("M,K", [(3, 16384), (2, 8256), (260, 12288)])
def test_long_rows_heavy_ties(M, K):
    """Integer-valued inputs: |h| takes a handful of values, so the chosen first-pass
    bin holds thousands of entries (more than the gathered list takes) and ties at tau
    straddle many 512-entry chunks held by different waves."""
    rs = np.random.default_rng(K + M)
    g = rs.integers(-3, 4, size=(M, K)).astype(np.float32)
    u = rs.integers(-2, 3, size=(M, K)).astype(np.float32)
    for k in (K // 2, K // 4 + 7, K - 64):
        check(f32_dev(g), f32_dev(u), g, u, k, f"long ties {M}x{K} k={k}")


@pytest.mark.parametrize("k", [255, 256, 257])
def test_nonzero_count_around_k(k):
    """Rows with exactly k-1, k and k+1 nonzero entries: the k-th largest magnitude is
    0 only when fewer than k entries are nonzero."""
    M, K = 6, 512
    rs = np.random.default_rng(k)
    x = np.zeros((M, K), np.float32)
    for m, nz in enumerate([255, 256, 257, 255, 256, 257]):
        idx = rs.choice(K, size=nz, replace=False)
        x[m, idx] = rs.standard_normal(nz).astype(np.float32)
    check(f32_dev(x), None, x, None, k, f"nnz around k={k}")
    x = tile_rows(x, 44)
    check(f32_dev(x), None, x, None, k, f"nnz around k={k}, 264 rows")


def plain_bf16_rows(K: int, M: int = 264) -> synth.Bf16:
    """bf16 rows without a gate, more than 256 of them (the one-wave-per-row kernel
    on 16-bit keys): integer values (a handful of magnitudes, so ties at tau straddle
    the 512-entry chunks), a zero row, a constant row, rows with K/2 - 1, K/2 and
    K/2 + 1 nonzero entries, rows of bf16 subnormals (every key in the first radix
    bin) mixed with zeros and with the largest finite magnitude, and Student-t rows."""
    rs = np.random.default_rng(K + 17)
    x = rs.integers(-3, 4, size=(M, K)).astype(np.float32)
    x[0] = 0.0
    x[1] = -2.0
    for r, nz in ((2, K // 2 - 1), (3, K // 2), (4, K // 2 + 1)):
        x[r] = 0.0
        x[r, rs.choice(K, size=nz, replace=False)] = rs.standard_normal(nz).astype(np.float32)
    sub = (rs.integers(0, 16, size=(2, K)).astype(np.uint32) << 16).view(np.float32)  # bf16 subnormals and zeros
    x[5:7] = sub * np.where(rs.random((2, K)) < 0.5, -1.0, 1.0).astype(np.float32)
    x[6, 7] = np.float32(3.3895314e38)  # largest finite bf16
    x[8:72] = rs.standard_t(3.0, size=(64, K)).astype(np.float32)
    return synth.to_bf16(x)


@pytest.mark.parametrize("K", [64, 576, 1024, 4032, 4096])
def test_plain_bf16_rows_ties_zeros_tail(K):
    """Every keep count class on the 16-bit-key kernel, with and without the keep mask
    (the mask-free call takes the tau = 0 shortcut); K < 4096 leaves lanes past K."""
    b = plain_bf16_rows(K)
    xd = bf16_dev(b)
    for k in sorted({1, 2, K // 2, K - 1, K}):
        check(xd, None, b.f32, None, k, f"plain bf16 K={K} k={k}")
        codes, scales = bw.bw_quantize_sparse_a8(xd, None, k)
        _, _, q, rsc = sparse8.sparse_a8(b.f32, None, k)
        assert_same(host(codes), q, f"plain bf16 K={K} k={k} codes (no mask)")
        assert_same(host(scales).view(np.uint32), rsc.view(np.uint32), f"plain bf16 K={K} k={k} scales (no mask)")


def test_full_down_proj_shape_sampled():
    """M=2048, K=11008 bf16 (the benchmark's launch), 64 sampled rows vs the oracle."""
    M, K = 2048, 11008
    g, u = synth.gate_up(M=M, K=K)
    c, s, m = run(bf16_dev(g), bf16_dev(u), K // 2, M, K)
    rows = np.sort(np.random.default_rng(8).choice(M, 64, replace=False))
    _, keep, q, rs = sparse8.sparse_a8(g.f32[rows], u.f32[rows], K // 2)
    assert_same(c[rows], q, "down codes")
    assert_same(s[rows].view(np.uint32), rs.view(np.uint32), "down scales")
    assert_same(m[rows], sparse8.mask_words(keep), "down mask")
    # property at every row: exactly K/2 survivors
    assert np.all(np.unpackbits(m.view(np.uint8), axis=1).sum(axis=1) == K // 2)


def test_determinism():
    g, u = synth.gate_up(seed=4, M=128, K=11008)
    gd, ud = bf16_dev(g), bf16_dev(u)
    a, sa = bw.bw_quantize_sparse_a8(gd, ud, 5504)
    b, sb = bw.bw_quantize_sparse_a8(gd, ud, 5504)
    torch.cuda.synchronize()
    assert torch.equal(a, b) and torch.equal(sa, sb)
