"""GPU parity: absmean ternary packer (bw_pack_ternary) vs the oracle, bit-exact bytes and beta."""
import numpy as np
import pytest
import torch

import synth
import ternary_weight_bit_amd as bw
from oracle import ternary
from tests.gpu_helpers import assert_same, bf16_dev, f32_dev, host

pytestmark = pytest.mark.gpu

ROLES = [(bw.BW_ROLE_A4, ternary.ROLE_A4, "A4"), (bw.BW_ROLE_A8, ternary.ROLE_A8, "A8"),
         (bw.BW_ROLE_A8_KMAJOR, ternary.ROLE_A8_KMAJOR, "A8K")]


def check(w_dev, w32, role_bw, role_or, label):
    N, K = w32.shape
    packed, beta = bw.bw_pack_ternary(w_dev, role_bw)
    t, b = ternary.quantize_weights(w32)
    ref = ternary.pack(t, role_or)
    gb = host(beta)
    assert_same(gb.view(np.uint32), np.full(N, b, np.float32).view(np.uint32), f"{label} beta")
    assert_same(host(packed), ref, f"{label} packed")


@pytest.mark.parametrize("rb,ro,name", ROLES)
def test_small_fp32(rb, ro, name):
    _, w = synth.small_bitlinear()
    check(f32_dev(w), w, rb, ro, f"256x256 {name}")


@pytest.mark.parametrize("rb,ro,name", ROLES)
@pytest.mark.parametrize("N,K", [(16, 64), (48, 320), (208, 1024)])
def test_ragged_bf16(rb, ro, name, N, K):
    w = synth.to_bf16(synth.normal(N * 7 + K, (N, K), 0.02))
    check(bf16_dev(w), w.f32, rb, ro, f"bf16 {N}x{K} {name}")


def test_full_7b_tensors():
    """One 4096x4096 (q) and one 11008x4096 (gate) tensor, fp32, every role."""
    for (N, K), seed in [((4096, 4096), 11), ((11008, 4096), 12)]:
        w = synth.weight_tensor(synth.SEED_BASE + seed, N, K)
        wd = f32_dev(w)
        for rb, ro, name in ROLES:
            check(wd, w, rb, ro, f"{N}x{K} {name}")
        del wd


def test_exact_sum_edge_cases():
    N, K = 16, 64
    cases = {
        "zero": np.zeros((N, K), np.float32),
        "one_big_many_tiny": np.where(np.arange(N * K).reshape(N, K) == 0, 1.0, 2.0**-30).astype(np.float32),
        "subnormals": np.full((N, K), 1e-41, np.float32) * np.where(np.arange(N * K).reshape(N, K) % 2, 1, -1),
        "wide_range": (synth.normal(5, (N, K)) * np.float32(10.0) ** synth.rng(6).integers(-30, 30, (N, K))).astype(np.float32),
        "halfway": np.tile(np.array([0.4, -0.2, 0.1, -0.1], np.float32), (N, K // 4)),
        "huge": np.full((N, K), 3e37, np.float32),
    }
    for name, w in cases.items():
        for rb, ro, rname in ROLES:
            check(f32_dev(w), w, rb, ro, f"{name} {rname}")


def test_fused_concatenation():
    """Packing q, k, v separately into slices of one buffer equals concatenating oracle packs."""
    K = 256
    parts = [synth.weight_tensor(100 + i, 64, K) for i in range(3)]
    N = 192
    packed = torch.empty(N * K // 4, dtype=torch.uint8, device="cuda:0")
    beta = torch.empty(N, dtype=torch.float32, device="cuda:0")
    ws = torch.empty(bw.bw_pack_ternary_workspace_bytes(64, K), dtype=torch.uint8, device="cuda:0")
    for i, w in enumerate(parts):
        bw.bw_pack_ternary(f32_dev(w), bw.BW_ROLE_A4, packed[i * 64 * K // 4 : (i + 1) * 64 * K // 4],
                           beta[i * 64 : (i + 1) * 64], ws)
    ref_p, ref_b = [], []
    for w in parts:
        t, b = ternary.quantize_weights(w)
        ref_p.append(ternary.pack(t, ternary.ROLE_A4))
        ref_b.append(np.full(64, b, np.float32))
    assert_same(host(packed), np.concatenate(ref_p), "fused packed")
    assert_same(host(beta).view(np.uint32), np.concatenate(ref_b).view(np.uint32), "fused beta")
