"""Python binding of libbw, the gfx950 BitNet a4.8 BitLinear library.

The functions carry the names of the C entry points declared in
include/bw.h and only marshal arguments: they check tensor dtype, shape,
device and contiguity, allocate missing outputs with torch, and pass raw
device pointers plus torch's current HIP stream to the library.  Every step
of the computation runs in the library's HIP kernels; there is no fallback.
"""
from __future__ import annotations

import ctypes
import os

import torch

__all__ = [
    "BW_OK", "BW_F32", "BW_BF16", "BW_ACT_INT4", "BW_ACT_FP4_E2M1", "BW_ACT_INT4_E2M3", "BW_ROLE_A4", "BW_ROLE_A8",
    "BW_ROLE_A8_KMAJOR", "bw_bitlinear_sparse_a8_gather_workspace_bytes", "bw_bitlinear_sparse_a8_gather",
    "BwError", "lib_path", "bw_abi_version", "bw_pack_layout_version", "bw_last_error",
    "bw_ternary_packed_bytes", "bw_pack_ternary_workspace_bytes", "bw_pack_ternary", "bw_quantize",
    "bw_bitlinear_a4", "code_bytes", "bw_quantize_bitlinear_a4", "bw_quantize_sparse_a8", "bw_bitlinear_sparse_a8", "bw_kv_pack3", "bw_kv_unpack3",
    "bw_attn_decode_kv3_workspace_bytes", "bw_attn_decode_kv3", "bw_block_decode_workspace_bytes",
    "bw_block_decode", "bw_block_decode_noalloc_max_bytes", "bw_block_decode_noalloc", "bw_stream_read",
]

BW_OK = 0
STATUS_NAMES = {
    0: "BW_OK", 1: "BW_ERR_NULL", 2: "BW_ERR_SHAPE", 3: "BW_ERR_ALIGN", 4: "BW_ERR_DTYPE",
    5: "BW_ERR_ARG", 6: "BW_ERR_HIP", 7: "BW_ERR_UNSUPPORTED",
}
BW_F32, BW_BF16 = 0, 1
BW_ACT_INT4, BW_ACT_FP4_E2M1, BW_ACT_INT4_E2M3 = 0, 1, 2
BW_ROLE_A4, BW_ROLE_A8, BW_ROLE_A8_KMAJOR = 0, 1, 2

lib_path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libbw.so")


class BwError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {msg}")
        self.status = status


def _load() -> ctypes.CDLL:
    if not os.path.exists(lib_path):
        raise ImportError(
            f"{lib_path} is not built; run `python ternary_weight_bit_amd/_build.py` (hipcc, gfx950)"
        )
    lib = ctypes.CDLL(lib_path)
    P, I64, SZ, I = ctypes.c_void_p, ctypes.c_int64, ctypes.c_size_t, ctypes.c_int
    sig = {
        "bw_abi_version": ([], I),
        "bw_pack_layout_version": ([], I),
        "bw_last_error": ([], ctypes.c_char_p),
        "bw_ternary_packed_bytes": ([I64, I64], SZ),
        "bw_pack_ternary_workspace_bytes": ([I64, I64], SZ),
        "bw_pack_ternary": ([P, I, I64, I64, I, P, P, P, SZ, P], I),
        "bw_quantize": ([P, I, I64, I64, I, P, P, P], I),
        "bw_bitlinear_a4": ([P, P, I64, I64, I, P, P, I64, P, P, P], I),
        "bw_bitlinear_a4_grouped": ([P, P, I64, I64, I, I, P, P, P, P, P, P], I),
        "bw_quantize_bitlinear_a4": ([P, I, I64, I64, I, P, P, I64, P, P, P, P, P], I),
        "bw_quantize_sparse_a8": ([P, P, I, I64, I64, I64, P, P, P, P], I),
        "bw_bitlinear_sparse_a8": ([P, P, I64, I64, P, P, I64, P, P, P], I),
        "bw_bitlinear_sparse_a8_grouped": ([P, P, I64, I64, I, P, P, P, P, P, P], I),
        "bw_bitlinear_sparse_a8_gather_workspace_bytes": ([I64, I64, I64], SZ),
        "bw_bitlinear_sparse_a8_gather": ([P, P, I64, I64, P, P, I64, P, P, P, SZ, P], I),
        "bw_kv_pack3": ([P, I, I64, I64, I64, I64, P, I64, P, P, P, P, P], I),
        "bw_kv_unpack3": ([P, P, P, P, P, I64, I64, I64, I64, I64, I, P, P], I),
        "bw_attn_decode_kv3_workspace_bytes": ([I64, I64, I64, I64], SZ),
        "bw_attn_decode_kv3": ([P, P, P, P, P, P, P, P, P, P, I64, I64, I64, I64, I64, P, P, SZ, P], I),
        "bw_block_decode_workspace_bytes": ([I64, I64, I64, I64, I64], SZ),
        "bw_block_decode": ([P, P, I64, I64, I64, I64] + [P] * 8 + [P] * 8 + [P, I64, I64, I64, P, SZ, P], I),
        "bw_stream_read": ([P, I64, P, P], I),
        "bw_block_decode_noalloc_max_bytes": ([], SZ),
        "bw_block_decode_noalloc": ([P, P, I64, I64, I64, I64] + [P] * 8 + [P] * 8 + [P, I64, I64, I64, P], I),
    }
    for name, (argt, rest) in sig.items():
        fn = getattr(lib, name)
        fn.argtypes = argt
        fn.restype = rest
    return lib


_lib = _load()


def _check(status: int) -> None:
    if status != BW_OK:
        raise BwError(status, _lib.bw_last_error().decode())


def _dev(t: torch.Tensor, name: str, dtypes=None, shape=None) -> int:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtypes is not None and t.dtype not in dtypes:
        raise TypeError(f"{name} has dtype {t.dtype}, expected one of {dtypes}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    return t.data_ptr()


def _opt(t, name, dtypes=None, shape=None) -> int | None:
    return None if t is None else _dev(t, name, dtypes, shape)


def _stream(t: torch.Tensor) -> int:
    return torch.cuda.current_stream(t.device).cuda_stream


def _fdtype(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return BW_F32
    if t.dtype == torch.bfloat16:
        return BW_BF16
    raise TypeError(f"unsupported dtype {t.dtype}; expected float32 or bfloat16")


_FLOATS = (torch.float32, torch.bfloat16)


def bw_abi_version() -> int:
    return _lib.bw_abi_version()


def bw_pack_layout_version() -> int:
    return _lib.bw_pack_layout_version()


def bw_last_error() -> str:
    return _lib.bw_last_error().decode()


def bw_ternary_packed_bytes(N: int, K: int) -> int:
    return _lib.bw_ternary_packed_bytes(N, K)


def bw_pack_ternary_workspace_bytes(N: int, K: int) -> int:
    return _lib.bw_pack_ternary_workspace_bytes(N, K)


def bw_pack_ternary(W: torch.Tensor, role: int, w_packed=None, beta=None, workspace=None):
    """Absmean-ternarize W [N][K] and pack it; returns (w_packed uint8 [N*K/4], beta fp32 [N])."""
    N, K = W.shape
    dev = W.device
    if w_packed is None:
        w_packed = torch.empty(bw_ternary_packed_bytes(N, K), dtype=torch.uint8, device=dev)
    if beta is None:
        beta = torch.empty(N, dtype=torch.float32, device=dev)
    if workspace is None:
        workspace = torch.empty(bw_pack_ternary_workspace_bytes(N, K), dtype=torch.uint8, device=dev)
    _check(_lib.bw_pack_ternary(
        _dev(W, "W", _FLOATS), _fdtype(W), N, K, role,
        _dev(w_packed, "w_packed", (torch.uint8,), (N * K // 4,)),
        _dev(beta, "beta", (torch.float32,), (N,)),
        _dev(workspace, "workspace", (torch.uint8,)), workspace.numel(), _stream(W)))
    return w_packed, beta


def code_bytes(K: int, fmt: int) -> int:
    """Bytes of one token's 4-bit codes: K/2 (nibbles), 3K/4 (BW_ACT_INT4_E2M3 fields)."""
    return K // 4 * 3 if fmt == BW_ACT_INT4_E2M3 else K // 2


def _k_of_codes(row_bytes: int, fmt: int) -> int:
    return row_bytes // 3 * 4 if fmt == BW_ACT_INT4_E2M3 else 2 * row_bytes


def _acc_dtype(fmt: int):
    return (torch.float32,) if fmt == BW_ACT_FP4_E2M1 else (torch.int32,)


def bw_quantize(x: torch.Tensor, fmt: int, codes=None, scales=None):
    """Per-token 4-bit quantizer; returns (codes uint8 [M][code_bytes(K, fmt)], scales fp32 [M])."""
    M, K = x.shape
    cb = code_bytes(K, fmt)
    if codes is None:
        codes = torch.empty((M, cb), dtype=torch.uint8, device=x.device)
    if scales is None:
        scales = torch.empty(M, dtype=torch.float32, device=x.device)
    _check(_lib.bw_quantize(
        _dev(x, "x", _FLOATS), _fdtype(x), M, K, fmt,
        _dev(codes, "codes", (torch.uint8,), (M, cb)),
        _dev(scales, "scales", (torch.float32,), (M,)), _stream(x)))
    return codes, scales


def bw_bitlinear_a4(codes: torch.Tensor, x_scales: torch.Tensor, fmt: int, w_packed: torch.Tensor,
                    beta: torch.Tensor, y=None, acc_dbg=None):
    """y [M][N] fp32 = ternary(W) applied to 4-bit activations (codes from bw_quantize)."""
    M, Kh = codes.shape
    K = _k_of_codes(Kh, fmt)
    N = beta.shape[0]
    if y is None:
        y = torch.empty((M, N), dtype=torch.float32, device=codes.device)
    acc_dt = _acc_dtype(fmt)
    _check(_lib.bw_bitlinear_a4(
        _dev(codes, "codes", (torch.uint8,)), _dev(x_scales, "x_scales", (torch.float32,), (M,)), M, K, fmt,
        _dev(w_packed, "w_packed", (torch.uint8,), (N * K // 4,)),
        _dev(beta, "beta", (torch.float32,), (N,)), N,
        _dev(y, "y", (torch.float32,), (M, N)),
        _opt(acc_dbg, "acc_dbg", acc_dt, (M, N)), _stream(codes)))
    return y


def _grouped_args(weights, M, K, ys, accs, acc_dt):
    """Host arrays (ctypes) of the grouped calls: device pointers and sizes per product."""
    n = len(weights)
    if not 1 <= n <= 4:
        raise ValueError("1 to 4 products per grouped call")
    Ns = [beta.shape[0] for _, beta in weights]
    if ys is None:
        ys = [None] * n
    ys = [torch.empty((M, N), dtype=torch.float32, device=weights[0][1].device) if yv is None else yv
          for yv, N in zip(ys, Ns)]
    P = ctypes.c_void_p
    w_arr = (P * n)(*[_dev(w, "w_packed", (torch.uint8,), (N * K // 4,)) for (w, _), N in zip(weights, Ns)])
    b_arr = (P * n)(*[_dev(b, "beta", (torch.float32,), (N,)) for (_, b), N in zip(weights, Ns)])
    n_arr = (ctypes.c_int64 * n)(*Ns)
    y_arr = (P * n)(*[_dev(yv, "y", (torch.float32,), (M, N)) for yv, N in zip(ys, Ns)])
    a_arr = None
    if accs is not None:
        a_arr = (P * n)(*[_opt(a, "acc_dbg", acc_dt, (M, N)) for a, N in zip(accs, Ns)])
    return n, w_arr, b_arr, n_arr, y_arr, a_arr, ys


def bw_bitlinear_a4_grouped(codes: torch.Tensor, x_scales: torch.Tensor, fmt: int, weights, ys=None, accs=None):
    """bw_bitlinear_a4 for each (w_packed, beta) of `weights` over the same codes, in one launch
    at prefill sizes; returns the list of y [M][N_g]."""
    M, Kh = codes.shape
    K = _k_of_codes(Kh, fmt)
    acc_dt = _acc_dtype(fmt)
    n, w_arr, b_arr, n_arr, y_arr, a_arr, ys = _grouped_args(weights, M, K, ys, accs, acc_dt)
    _check(_lib.bw_bitlinear_a4_grouped(
        _dev(codes, "codes", (torch.uint8,)), _dev(x_scales, "x_scales", (torch.float32,), (M,)), M, K, fmt, n,
        w_arr, b_arr, n_arr, y_arr, a_arr, _stream(codes)))
    return ys


def bw_quantize_bitlinear_a4(x: torch.Tensor, fmt: int, w_packed: torch.Tensor, beta: torch.Tensor, y=None,
                             codes=None, scales=None, acc_dbg=None):
    """bw_quantize followed by bw_bitlinear_a4 in one call (one launch for M <= 2);
    returns (y fp32 [M][N], codes uint8 [M][code_bytes(K, fmt)], scales fp32 [M])."""
    M, K = x.shape
    N = beta.shape[0]
    dev = x.device
    cb = code_bytes(K, fmt)
    if y is None:
        y = torch.empty((M, N), dtype=torch.float32, device=dev)
    if codes is None:
        codes = torch.empty((M, cb), dtype=torch.uint8, device=dev)
    if scales is None:
        scales = torch.empty(M, dtype=torch.float32, device=dev)
    acc_dt = _acc_dtype(fmt)
    _check(_lib.bw_quantize_bitlinear_a4(
        _dev(x, "x", _FLOATS), _fdtype(x), M, K, fmt,
        _dev(w_packed, "w_packed", (torch.uint8,), (N * K // 4,)), _dev(beta, "beta", (torch.float32,), (N,)), N,
        _dev(codes, "codes", (torch.uint8,), (M, cb)), _dev(scales, "scales", (torch.float32,), (M,)),
        _dev(y, "y", (torch.float32,), (M, N)), _opt(acc_dbg, "acc_dbg", acc_dt, (M, N)), _stream(x)))
    return y, codes, scales


def bw_quantize_sparse_a8(gate_or_x: torch.Tensor, up=None, k_keep=None, codes=None, scales=None,
                          mask_dbg=None):
    """ReLU^2 gate (when up is given) + per-token top-k + INT8; returns (codes int8 [M][K], scales fp32 [M])."""
    M, K = gate_or_x.shape
    if k_keep is None:
        k_keep = K // 2
    if up is not None and (up.dtype != gate_or_x.dtype or up.shape != gate_or_x.shape):
        raise ValueError("up must match gate in dtype and shape")
    if codes is None:
        codes = torch.empty((M, K), dtype=torch.int8, device=gate_or_x.device)
    if scales is None:
        scales = torch.empty(M, dtype=torch.float32, device=gate_or_x.device)
    _check(_lib.bw_quantize_sparse_a8(
        _dev(gate_or_x, "gate_or_x", _FLOATS), _opt(up, "up", _FLOATS), _fdtype(gate_or_x), M, K, k_keep,
        _dev(codes, "codes", (torch.int8,), (M, K)), _dev(scales, "scales", (torch.float32,), (M,)),
        _opt(mask_dbg, "mask_dbg", (torch.int32, torch.uint32), (M, K // 32)), _stream(gate_or_x)))
    return codes, scales


def bw_bitlinear_sparse_a8(codes: torch.Tensor, x_scales: torch.Tensor, w_packed: torch.Tensor,
                           beta: torch.Tensor, y=None, acc_dbg=None):
    """y [M][N] fp32 = ternary(W) applied to INT8 codes (from bw_quantize_sparse_a8)."""
    M, K = codes.shape
    N = beta.shape[0]
    if y is None:
        y = torch.empty((M, N), dtype=torch.float32, device=codes.device)
    _check(_lib.bw_bitlinear_sparse_a8(
        _dev(codes, "codes", (torch.int8,)), _dev(x_scales, "x_scales", (torch.float32,), (M,)), M, K,
        _dev(w_packed, "w_packed", (torch.uint8,), (N * K // 4,)),
        _dev(beta, "beta", (torch.float32,), (N,)), N,
        _dev(y, "y", (torch.float32,), (M, N)), _opt(acc_dbg, "acc_dbg", (torch.int32,), (M, N)),
        _stream(codes)))
    return y


def bw_bitlinear_sparse_a8_grouped(codes: torch.Tensor, x_scales: torch.Tensor, weights, ys=None, accs=None):
    """bw_bitlinear_sparse_a8 for each (w_packed, beta) of `weights` over the same INT8 codes,
    in one launch at prefill sizes; returns the list of y [M][N_g]."""
    M, K = codes.shape
    n, w_arr, b_arr, n_arr, y_arr, a_arr, ys = _grouped_args(weights, M, K, ys, accs, (torch.int32,))
    _check(_lib.bw_bitlinear_sparse_a8_grouped(
        _dev(codes, "codes", (torch.int8,)), _dev(x_scales, "x_scales", (torch.float32,), (M,)), M, K, n,
        w_arr, b_arr, n_arr, y_arr, a_arr, _stream(codes)))
    return ys


def bw_bitlinear_sparse_a8_gather_workspace_bytes(M: int, K: int, N: int) -> int:
    return _lib.bw_bitlinear_sparse_a8_gather_workspace_bytes(M, K, N)


def bw_bitlinear_sparse_a8_gather(codes: torch.Tensor, x_scales: torch.Tensor, w_kmajor: torch.Tensor,
                                  beta: torch.Tensor, workspace: torch.Tensor, y=None, acc_dbg=None):
    """y [M][N] fp32 from INT8 codes and K-major ternary weights, reading only the rows of
    nonzero codes.  workspace: uint8, >= bw_bitlinear_sparse_a8_gather_workspace_bytes(M, K, N)."""
    M, K = codes.shape
    N = beta.shape[0]
    if y is None:
        y = torch.empty((M, N), dtype=torch.float32, device=codes.device)
    _check(_lib.bw_bitlinear_sparse_a8_gather(
        _dev(codes, "codes", (torch.int8,)), _dev(x_scales, "x_scales", (torch.float32,), (M,)), M, K,
        _dev(w_kmajor, "w_kmajor", (torch.uint8,), (N * K // 4,)),
        _dev(beta, "beta", (torch.float32,), (N,)), N,
        _dev(y, "y", (torch.float32,), (M, N)), _opt(acc_dbg, "acc_dbg", (torch.int32,), (M, N)),
        _dev(workspace, "workspace", (torch.uint8,)), workspace.numel(), _stream(codes)))
    return y


def bw_kv_pack3(kv: torch.Tensor, slot_of: torch.Tensor, n_special: int, p3=None, s3=None, p4=None, s4=None):
    """3-bit KV pack; returns (p3 uint8 [B][S][H][3D/8], s3 fp32 [B][S][H], p4 uint8 [n][H][D/2], s4 fp32 [n][H])."""
    B, S, H, D = kv.shape
    dev = kv.device
    if p3 is None:
        p3 = torch.empty((B, S, H, 3 * D // 8), dtype=torch.uint8, device=dev)
    if s3 is None:
        s3 = torch.empty((B, S, H), dtype=torch.float32, device=dev)
    if p4 is None:
        p4 = torch.zeros((max(n_special, 1), H, D // 2), dtype=torch.uint8, device=dev)
    if s4 is None:
        s4 = torch.zeros((max(n_special, 1), H), dtype=torch.float32, device=dev)
    _check(_lib.bw_kv_pack3(
        _dev(kv, "kv", _FLOATS), _fdtype(kv), B, S, H, D,
        _dev(slot_of, "slot_of", (torch.int32,), (B, S)), n_special,
        _dev(p3, "p3", (torch.uint8,), (B, S, H, 3 * D // 8)), _dev(s3, "s3", (torch.float32,), (B, S, H)),
        _dev(p4, "p4", (torch.uint8,)), _dev(s4, "s4", (torch.float32,)), _stream(kv)))
    return p3, s3, p4, s4


def bw_kv_unpack3(p3: torch.Tensor, s3: torch.Tensor, p4: torch.Tensor, s4: torch.Tensor,
                  slot_of: torch.Tensor, n_special: int, out_dtype=torch.float32, out=None):
    """Dequantize the 3-bit KV cache; returns out [B][S][H][D] (fp32 or bf16)."""
    B, S, H, pd = p3.shape
    D = pd * 8 // 3
    if out is None:
        out = torch.empty((B, S, H, D), dtype=out_dtype, device=p3.device)
    _check(_lib.bw_kv_unpack3(
        _dev(p3, "p3", (torch.uint8,)), _dev(s3, "s3", (torch.float32,), (B, S, H)),
        _dev(p4, "p4", (torch.uint8,)), _dev(s4, "s4", (torch.float32,)),
        _dev(slot_of, "slot_of", (torch.int32,), (B, S)), B, S, H, D, n_special, _fdtype(out),
        _dev(out, "out", _FLOATS, (B, S, H, D)), _stream(p3)))
    return out


def bw_attn_decode_kv3_workspace_bytes(B: int, S: int, H: int, D: int) -> int:
    return _lib.bw_attn_decode_kv3_workspace_bytes(B, S, H, D)


def bw_attn_decode_kv3(q: torch.Tensor, k_pack, v_pack, slot_of: torch.Tensor, n_special: int, out=None,
                       workspace=None):
    """Single-token attention over the 3-bit KV cache.  q fp32 [B][H][D]; k_pack / v_pack =
    (p3, s3, p4, s4) as returned by bw_kv_pack3 with this slot_of; returns out fp32 [B][H][D]."""
    B, H, D = q.shape
    kp3, ks3, kp4, ks4 = k_pack
    vp3, vs3, vp4, vs4 = v_pack
    S = kp3.shape[1]
    if out is None:
        out = torch.empty((B, H, D), dtype=torch.float32, device=q.device)
    if workspace is None:
        workspace = torch.empty(max(bw_attn_decode_kv3_workspace_bytes(B, S, H, D), 16), dtype=torch.uint8,
                                device=q.device)
    shp3, shs = (B, S, H, 3 * D // 8), (B, S, H)
    shp4, shs4 = (n_special, H, D // 2), (n_special, H)
    _check(_lib.bw_attn_decode_kv3(
        _dev(q, "q", (torch.float32,)),
        _dev(kp3, "k_p3", (torch.uint8,), shp3), _dev(ks3, "k_s3", (torch.float32,), shs),
        _opt(kp4, "k_p4", (torch.uint8,), shp4), _opt(ks4, "k_s4", (torch.float32,), shs4),
        _dev(vp3, "v_p3", (torch.uint8,), shp3), _dev(vs3, "v_s3", (torch.float32,), shs),
        _opt(vp4, "v_p4", (torch.uint8,), shp4), _opt(vs4, "v_s4", (torch.float32,), shs4),
        _dev(slot_of, "slot_of", (torch.int32,), (B, S)), n_special, B, S, H, D,
        _dev(out, "out", (torch.float32,), (B, H, D)),
        _dev(workspace, "workspace", (torch.uint8,)), workspace.numel(), _stream(q)))
    return out


def bw_block_decode_workspace_bytes(B: int, S_cap: int, H: int, D: int, F: int) -> int:
    return _lib.bw_block_decode_workspace_bytes(B, S_cap, H, D, F)


def _block_args(x, weights, k_pack, v_pack, slot_of, n_special, pos, H, x_out):
    B, HD = x.shape
    D = HD // H
    w_qkv, b_qkv, w_o, b_o, w_gu, b_gu, w_down, b_down = weights
    F = b_gu.shape[0] // 2
    S_cap = k_pack[0].shape[1]
    u8, f32 = (torch.uint8,), (torch.float32,)
    shp3, shs = (B, S_cap, H, 3 * D // 8), (B, S_cap, H)
    shp4, shs4 = (n_special, H, D // 2), (n_special, H)
    cache = []
    for name, (p3, s3, p4, s4) in (("k", k_pack), ("v", v_pack)):
        cache += [_dev(p3, name + "_p3", u8, shp3), _dev(s3, name + "_s3", f32, shs),
                  _opt(p4, name + "_p4", u8, shp4), _opt(s4, name + "_s4", f32, shs4)]
    return [
        _dev(x, "x", f32, (B, HD)), _dev(x_out, "x_out", f32, (B, HD)), B, H, D, F,
        _dev(w_qkv, "w_qkv", u8, (3 * HD * HD // 4,)), _dev(b_qkv, "b_qkv", f32, (3 * HD,)),
        _dev(w_o, "w_o", u8, (HD * HD // 4,)), _dev(b_o, "b_o", f32, (HD,)),
        _dev(w_gu, "w_gate_up", u8, (2 * F * HD // 4,)), _dev(b_gu, "b_gate_up", f32, (2 * F,)),
        _dev(w_down, "w_down", u8, (HD * F // 4,)), _dev(b_down, "b_down", f32, (HD,)),
        *cache, _dev(slot_of, "slot_of", (torch.int32,), (B, S_cap)), n_special, S_cap, pos]


def bw_block_decode(x: torch.Tensor, weights, k_pack, v_pack, slot_of: torch.Tensor, n_special: int, pos: int,
                    H: int, x_out=None, workspace=None):
    """One decoder layer for one new token per sequence.  x fp32 [B][H*D]; weights =
    (w_qkv, b_qkv, w_o, b_o, w_gate_up, b_gate_up, w_down, b_down) from bw_pack_ternary;
    k_pack / v_pack = (p3, s3, p4, s4) cache slabs [B][S_cap]...; returns x_out fp32 [B][H*D]."""
    B, HD = x.shape
    F = weights[5].shape[0] // 2
    S_cap = k_pack[0].shape[1]
    if x_out is None:
        x_out = torch.empty_like(x)
    if workspace is None:
        workspace = torch.empty(max(bw_block_decode_workspace_bytes(B, S_cap, H, HD // H, F), 16),
                                dtype=torch.uint8, device=x.device)
    args = _block_args(x, weights, k_pack, v_pack, slot_of, n_special, pos, H, x_out)
    _check(_lib.bw_block_decode(*args, _dev(workspace, "workspace", (torch.uint8,)), workspace.numel(), _stream(x)))
    return x_out


def bw_stream_read(src: torch.Tensor, sink=None):
    """Measurement aid: read src's bytes once in the decode GEMV's access pattern; returns
    sink uint32 [4 * ceil(bytes / 16384)], the XOR of each 4 KB quarter's 32-bit words."""
    nbytes = src.numel() * src.element_size()
    if sink is None:
        sink = torch.empty(4 * ((nbytes + 16383) // 16384), dtype=torch.int32, device=src.device)
    elif sink.numel() < 4 * ((nbytes + 16383) // 16384):
        raise ValueError("sink needs 4 * ceil(bytes / 16384) words")
    _check(_lib.bw_stream_read(_dev(src, "src"), nbytes, _dev(sink, "sink", (torch.int32, torch.uint32)),
                               _stream(src)))
    return sink


def bw_block_decode_noalloc_max_bytes() -> int:
    return _lib.bw_block_decode_noalloc_max_bytes()


def bw_block_decode_noalloc(x: torch.Tensor, weights, k_pack, v_pack, slot_of: torch.Tensor, n_special: int,
                            pos: int, H: int, x_out: torch.Tensor):
    """bw_block_decode with the library's static per-GPU workspace: allocates nothing
    (x_out, like every other buffer, is the caller's)."""
    args = _block_args(x, weights, k_pack, v_pack, slot_of, n_special, pos, H, x_out)
    _check(_lib.bw_block_decode_noalloc(*args, _stream(x)))
    return x_out
