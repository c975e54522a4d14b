"""C-ABI boundary tests that need no GPU: the library loads, exports what
include/bw.h declares, and rejects bad arguments on the host before any launch."""
import ctypes
import os
import re

import pytest

import ternary_weight_bit_amd as bw

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "bw.h")

lib = bw._lib
A = 0x10000  # aligned fake device address: validation fails before it could be touched
MIS = 0x10004  # 4-byte aligned only


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(bw_[a-z0-9_]+)\s*\(", src)))


def test_exports_every_declared_symbol():
    names = declared_functions()
    assert len(names) == 24, names
    for n in names:
        assert hasattr(lib, n), n


def test_versions():
    assert bw.bw_abi_version() == 2
    assert bw.bw_pack_layout_version() == 2
    assert bw.bw_ternary_packed_bytes(4096, 4096) == 4096 * 4096 // 4
    assert bw.bw_ternary_packed_bytes(0, 64) == 0
    assert bw.bw_pack_ternary_workspace_bytes(16, 64) >= 4096 + 4


def q(x, dt, M, K, fmt, c, s):
    return lib.bw_quantize(x, dt, M, K, fmt, c, s, None)


def test_quantize_validation():
    assert q(A, 1, 4, 100, 0, A, A) == 2  # K % 64
    assert q(A, 1, 4, 0, 0, A, A) == 2
    assert q(A, 1, 4, 262144, 0, A, A) == 2  # K too large
    assert q(A, 1, -1, 64, 0, A, A) == 2
    assert q(A, 7, 4, 64, 0, A, A) == 4  # dtype
    assert q(A, 1, 4, 64, 9, A, A) == 4  # fmt
    assert q(None, 1, 4, 64, 0, A, A) == 1
    assert q(A, 1, 4, 64, 0, None, A) == 1
    assert q(MIS, 1, 4, 64, 0, A, A) == 3
    assert "16-byte" in bw.bw_last_error()
    assert q(None, 1, 0, 64, 0, None, None) == 0  # empty call
    assert bw.bw_last_error() == ""


def test_bitlinear_validation():
    f = lib.bw_bitlinear_a4
    assert f(A, A, 8, 4096, 0, A, A, 100, A, None, None) == 2  # N % 16
    assert f(A, A, 8, 4000, 0, A, A, 128, A, None, None) == 2  # K % 64
    assert f(A, A, 8, 4096, 3, A, A, 128, A, None, None) == 4
    assert f(A, A, 8, 4096, 0, None, A, 128, A, None, None) == 1
    assert f(A, A, 8, 4096, 0, A, A, 128, MIS, None, None) == 3
    assert f(A, A, 8, 4096, 0, A, A, 128, A, MIS, None) == 3  # acc_dbg alignment
    assert f(None, None, 0, 4096, 0, None, None, 128, None, None, None) == 0
    g = lib.bw_bitlinear_sparse_a8
    assert g(A, A, 8, 11008, A, A, 4095, A, None, None) == 2
    assert g(A, None, 8, 11008, A, A, 4096, A, None, None) == 1


def test_grouped_validation():
    P, I64 = ctypes.c_void_p, ctypes.c_int64
    w = (P * 2)(A, A)
    b = (P * 2)(A, A)
    y = (P * 2)(A, A)
    n_ok = (I64 * 2)(128, 4096)
    n_bad = (I64 * 2)(128, 100)
    f = lib.bw_bitlinear_a4_grouped
    assert f(A, A, 64, 4096, 0, 0, w, b, n_ok, y, None, None) == 5  # n_groups
    assert f(A, A, 64, 4096, 0, 5, w, b, n_ok, y, None, None) == 5
    assert f(A, A, 64, 4096, 0, 2, w, b, n_bad, y, None, None) == 2  # second product's N % 16
    assert f(A, A, 64, 4096, 3, 2, w, b, n_ok, y, None, None) == 4  # fmt
    assert f(A, A, 64, 4096, 0, 2, None, b, n_ok, y, None, None) == 1  # host array
    y_mis = (P * 2)(A, MIS)
    assert f(A, A, 64, 4096, 0, 2, w, b, n_ok, y_mis, None, None) == 3
    assert f(None, None, 0, 4096, 0, 2, w, b, n_ok, y, None, None) == 0  # no tokens
    g = lib.bw_bitlinear_sparse_a8_grouped
    assert g(A, A, 64, 11008, 0, w, b, n_ok, y, None, None) == 5
    assert g(A, A, 64, 11008, 2, w, b, n_bad, y, None, None) == 2
    assert g(A, None, 64, 11008, 2, w, b, n_ok, y, None, None) == 1


def test_e2m3_validation():
    """BW_ACT_INT4_E2M3 codes are read by the LDS GEMM only: shapes beyond its
    32-bit offsets are refused before anything is launched."""
    f = lib.bw_bitlinear_a4
    assert f(A, A, 1 << 20, 4096, 2, A, A, 128, A, None, None) == 7  # 3 GB of codes
    assert f(A, A, 64, 4096, 2, A, A, 100, A, None, None) == 2       # N % 16 still checked first
    g = lib.bw_quantize_bitlinear_a4
    assert g(A, 1, 1 << 20, 4096, 2, A, A, 128, A, A, A, None, None) == 7
    P, I64 = ctypes.c_void_p, ctypes.c_int64
    w = (P * 2)(A, A)
    n = (I64 * 2)(128, 4096)
    assert lib.bw_bitlinear_a4_grouped(A, A, 1 << 20, 4096, 2, 2, w, w, n, w, None, None) == 7


def test_gather_validation():
    ws = bw.bw_bitlinear_sparse_a8_gather_workspace_bytes(1, 11008, 4096)
    assert ws >= 4 * 4096 and ws % 256 == 0
    assert bw.bw_bitlinear_sparse_a8_gather_workspace_bytes(0, 11008, 4096) == 0
    assert bw.bw_bitlinear_sparse_a8_gather_workspace_bytes(17, 11008, 4096) == 0
    assert bw.bw_bitlinear_sparse_a8_gather_workspace_bytes(1, 100, 4096) == 0
    g = lib.bw_bitlinear_sparse_a8_gather
    assert g(A, A, 1, 11008, A, A, 4095, A, None, A, ws, None) == 2  # N % 16
    assert g(A, A, 1, 11000, A, A, 4096, A, None, A, ws, None) == 2  # K % 64
    assert g(A, A, 17, 4096, A, A, 4096, A, None, A, 1 << 40, None) == 2  # M
    assert g(A, A, 1, 131072, A, A, 1 << 17, A, None, A, 1 << 40, None) == 2  # weights above 2^31 bytes
    assert g(A, A, 1, 11008, A, A, 4096, A, None, None, ws, None) == 1  # workspace
    assert g(A, A, 1, 11008, A, A, 4096, A, None, MIS, ws, None) == 3
    assert g(A, A, 1, 11008, A, A, 4096, A, None, A, ws - 1, None) == 5
    assert "workspace" in bw.bw_last_error()
    assert g(None, None, 0, 11008, None, None, 4096, None, None, None, 0, None) == 0


def test_sparse_validation():
    f = lib.bw_quantize_sparse_a8
    assert f(A, A, 1, 8, 11008, 0, A, A, None, None) == 5  # k_keep
    assert f(A, A, 1, 8, 11008, 11009, A, A, None, None) == 5
    assert f(A, A, 1, 8, 32768, 100, A, A, None, None) == 2  # K above the row-resident limit
    assert f(A, MIS, 1, 8, 11008, 5504, A, A, None, None) == 3
    assert f(None, None, 1, 8, 11008, 5504, A, A, None, None) == 1
    assert f(A, None, 2, 8, 11008, 5504, A, A, None, None) == 4


def test_pack_validation():
    f = lib.bw_pack_ternary
    assert f(A, 0, 100, 64, 0, A, A, A, 4096, None) == 2
    assert f(A, 0, 16, 64, 5, A, A, A, 4096, None) == 4
    assert f(A, 0, 16, 64, 0, A, A, A, 16, None) == 5  # workspace too small
    assert f(A, 0, 16, 64, 0, A, A, None, 4096, None) == 1
    assert f(A, 0, 16, 64, 0, A, MIS, A, 4096, None) == 3


def test_kv_validation():
    f = lib.bw_kv_pack3
    assert f(A, 1, 8, 16, 4, 100, A, 2, A, A, A, A, None) == 2  # head_dim
    assert f(A, 1, 8, 16, 4, 128, A, 2, A, A, None, None, None) == 1  # side slab missing
    assert f(A, 1, 0, 16, 4, 128, None, 0, None, None, None, None, None) == 0  # empty
    g = lib.bw_kv_unpack3
    assert g(A, A, A, A, A, 8, 16, 4, 128, 2, 5, A, None) == 4
    assert g(A, A, A, A, A, 8, 16, 0, 128, 2, 1, A, None) == 2  # H = 0


def test_attn_validation():
    f = lib.bw_attn_decode_kv3
    ws = bw.bw_attn_decode_kv3_workspace_bytes(8, 4096, 32, 128)
    assert ws >= 8 * 32 * 128 * 4 and bw.bw_attn_decode_kv3_workspace_bytes(8, 4096, 32, 96) == 0

    def args(B, S, H, D, n=0, q=A, k4=None, out=A, w=A, wb=ws):
        return (q, A, A, k4, k4, A, A, k4, k4, A, n, B, S, H, D, out, w, wb, None)

    assert f(*args(8, 4096, 32, 96)) == 2  # head_dim
    assert f(*args(8, 0, 32, 128)) == 2  # S
    assert f(*args(8, 4096, 2048, 128)) == 2  # H above the LDS limit
    assert f(*args(8, 4096, 32, 128, n=3)) == 1  # side slabs missing
    assert f(*args(8, 4096, 32, 128, q=None)) == 1
    assert f(*args(8, 4096, 32, 128, w=None)) == 1
    assert f(*args(8, 4096, 32, 128, out=MIS)) == 3
    assert f(*args(8, 4096, 32, 128, wb=ws - 1)) == 5
    assert f(*args(0, 4096, 32, 128, q=None, out=None, w=None)) == 0  # empty batch


def test_block_validation():
    ws = bw.bw_block_decode_workspace_bytes(8, 4096, 32, 128, 11008)
    assert ws > 0 and bw.bw_block_decode_workspace_bytes(17, 4096, 32, 128, 11008) == 0
    f = lib.bw_block_decode

    def args(B=8, H=32, D=128, F=11008, S_cap=4096, pos=100, x=A, w=A, nsp=0, k4=None):
        return (x, A, B, H, D, F) + (A,) * 8 + (A, A, k4, k4, A, A, k4, k4) + (A, nsp, S_cap, pos, w, ws, None)

    assert f(*args(B=17)) == 2
    assert f(*args(D=96)) == 2
    assert f(*args(F=11000)) == 2
    assert f(*args(pos=4096)) == 5
    assert f(*args(x=None)) == 1
    assert f(*args(nsp=3)) == 1  # side slabs missing
    assert f(*args(w=MIS)) == 3


def _block_regions_except_attention(B, H, D, F):
    """Bytes of the decoder layer's workspace regions other than the attention's,
    each rounded up to 256 (codes, scales, q/k/v, attention output, INT8 codes,
    scales, x1, gate/up, INT8 codes, scales)."""
    r = lambda n: (n + 255) // 256 * 256
    hd = H * D
    return (r(B * hd // 2) + r(4 * B) + r(4 * B * 3 * hd) + r(4 * B * hd) + r(B * hd) + r(4 * B) + r(4 * B * hd)
            + r(8 * B * F) + r(B * F) + r(4 * B))


@pytest.mark.parametrize("H,D,S_cap", [(32, 128, 2048), (32, 128, 4096), (8, 64, 1500), (2, 128, 700)])
def test_block_workspace_covers_attention_at_every_position(H, D, S_cap):
    """For every batch size the layer takes and every attended length S <= S_cap, the
    attention launch's workspace fits inside the attention region of the layer's
    workspace (a launch at pos = S - 1 writes that many bytes)."""
    F = 256
    for B in range(1, 17):
        total = bw.bw_block_decode_workspace_bytes(B, S_cap, H, D, F)
        assert total > 0
        region = total - _block_regions_except_attention(B, H, D, F)
        worst = max(bw.bw_attn_decode_kv3_workspace_bytes(B, S, H, D) for S in range(1, S_cap + 1))
        assert 0 < worst <= region, (B, worst, region)


def test_block_noalloc_validation():
    """The allocation-free layer states its static workspace size and rejects, on the
    host, a shape whose workspace would not fit (32 MB of attention partials for 16
    sequences of 128 heads over 4096 positions) before it touches the device."""
    assert bw.bw_block_decode_noalloc_max_bytes() == 16 << 20
    f = lib.bw_block_decode_noalloc
    B, H, D, F, S_cap = 16, 128, 128, 16384, 4096
    assert bw.bw_block_decode_workspace_bytes(B, S_cap, H, D, F) > 16 << 20
    args = lambda B, pos: [A, A, B, H, D, F] + [A] * 16 + [A, 1, S_cap, pos, None]
    assert f(*args(B, 100)) == 7
    assert "static scratch" in bw.bw_last_error()
    assert f(*args(B, S_cap)) == 5  # pos out of range
    assert f(*args(17, 100)) == 2
    a = args(B, 100)
    a[0] = None
    assert f(*a) == 1
