"""One BitNet a4.8 decoder layer for one new token per sequence (oracle; test
infrastructure).

BitNet a4.8 abstract: 4-bit activations for the inputs of the attention and
feed-forward layers, sparsified then 8-bit intermediate states, 3-bit KV cache;
toshoseti review, «Метод»: INT4 for the q/k/v and gate/up inputs, top-k at 50 %
for the out projection input, ReLU^2 gate for the down projection;
«Эксперименты»: bos/eos tokens stay at 4 bits in the KV cache.  The pages give
no layer formula.  Reading: the plainest composition of those pieces, with no
normalization and no rotary embedding (neither is described), every
intermediate handed on in fp32 as a BitLinear call produces it:

    y_qkv = BitLinearA4(x)                  (fp32: fl(fl(acc * s) * beta))
    the new k, v (columns HD..2HD, 2HD..3HD) are packed at position pos
    a     = attention(q = y_qkv[:, :HD], positions 0..pos)   (fp64, then fp32)
    x1    = x + BitLinearA8(top-k HD/2 INT8 of a)            (fp32 add)
    g, u  = BitLinearA4(x1) with W_gate, W_up
    x_out = x1 + BitLinearA8(top-k F/2 INT8 of relu(g)^2 * u)
"""
from __future__ import annotations

import numpy as np

from . import act4, attn3, bitlinear, kv3, sparse8


def fp32_handoff(acc: np.ndarray, s_x: np.ndarray, beta: np.ndarray) -> np.ndarray:
    """y = fl(fl(acc * s_x[m]) * beta[n]) in fp32: the value a BitLinear call hands on
    (acc is an exact integer below 2^24, so its fp32 conversion is exact)."""
    a = np.asarray(acc).astype(np.float32)
    s = np.asarray(s_x, dtype=np.float32)[:, None]
    b = np.asarray(beta, dtype=np.float32)[None, :]
    return ((a * s).astype(np.float32) * b).astype(np.float32)


def append_kv(pack, new: np.ndarray, slot_of: np.ndarray, n_special: int, pos: int):
    """Copy of the cache slabs with the vectors new [B][H][D] packed at position pos."""
    p3, s3, p4, s4 = (a.copy() for a in pack)
    q3, sc3, q4, sc4 = kv3.kv_pack3(new[:, None], slot_of[:, pos : pos + 1], n_special)
    p3[:, pos] = q3[:, 0]
    s3[:, pos] = sc3[:, 0]
    for b in range(new.shape[0]):
        sl = int(slot_of[b, pos])
        if 0 <= sl < n_special:
            p4[sl] = q4[sl]
            s4[sl] = sc4[sl]
    return p3, s3, p4, s4


def decode_block(x, t_qkv, b_qkv, t_o, b_o, t_gu, b_gu, t_down, b_down, k_pack, v_pack, slot_of,
                 n_special: int, pos: int, H: int):
    """x fp32 [B][HD]; t_* ternary int8 [N][K] with per-row beta b_* (fp32); k_pack / v_pack
    as kv3.kv_pack3 returns them for [B][S_cap][H][D].  Returns (x_out fp32 [B][HD],
    k_pack, v_pack after the append, dict of intermediates)."""
    x = np.asarray(x, dtype=np.float32)
    B, HD = x.shape
    D = HD // H
    F = t_gu.shape[0] // 2
    q4, s = act4.quantize_int4(x)
    y_qkv = fp32_handoff(bitlinear.contract(q4, t_qkv), s, b_qkv)
    kp = append_kv(k_pack, y_qkv[:, HD : 2 * HD].reshape(B, H, D), slot_of, n_special, pos)
    vp = append_kv(v_pack, y_qkv[:, 2 * HD :].reshape(B, H, D), slot_of, n_special, pos)
    upto = lambda p: (p[0][:, : pos + 1], p[1][:, : pos + 1], p[2], p[3])
    att, _ = attn3.decode_attention(y_qkv[:, :HD].reshape(B, H, D), upto(kp), upto(vp),
                                    slot_of[:, : pos + 1], D)
    a32 = att.reshape(B, HD).astype(np.float32)
    _, keep_o, q8, s8 = sparse8.sparse_a8(a32, None, HD // 2)
    y_o = fp32_handoff(bitlinear.contract(q8, t_o), s8, b_o)
    x1 = (x + y_o).astype(np.float32)
    q4b, sb = act4.quantize_int4(x1)
    g = fp32_handoff(bitlinear.contract(q4b, t_gu[:F]), sb, b_gu[:F])
    u = fp32_handoff(bitlinear.contract(q4b, t_gu[F:]), sb, b_gu[F:])
    h_d, keep_d, q8d, s8d = sparse8.sparse_a8(g, u, F // 2)
    y_d = fp32_handoff(bitlinear.contract(q8d, t_down), s8d, b_down)
    x_out = (x1 + y_d).astype(np.float32)
    return x_out, kp, vp, dict(y_qkv=y_qkv, att=a32, keep_o=keep_o, q8=q8, s8=s8, y_o=y_o, x1=x1, g=g, u=u,
                               h_d=h_d, keep_d=keep_d, q8d=q8d, s8d=s8d, y_d=y_d)
