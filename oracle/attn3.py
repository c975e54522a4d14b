"""Single-token attention over the 3-bit KV cache (oracle; test infrastructure).

BitNet a4.8 abstract: the model supports a 3-bit KV cache; 9pt.com article,
methodology: the 3-bit key-value cache is part of what makes inference more
memory-efficient and faster.  The pages give no attention formula, so the
reading is the plainest one: standard scaled dot-product attention of one new
query per (batch, head) over all S cached positions,

    z_s = (q . k_s) / sqrt(D),   p = softmax(z),   out = sum_s p_s v_s,

where k_s and v_s are the codec's dequantized vectors (kv3.kv_unpack3: fl(code
* scale) in fp32, and the 4-bit side-slab codes at special positions).
Everything after dequantization is evaluated in fp64.
"""
from __future__ import annotations

import numpy as np

from . import kv3


def decode_attention(q, k_pack, v_pack, slot_of, D: int, n_special: int | None = None):
    """q float32 [B][H][D]; k_pack / v_pack = (p3, s3, p4, s4) as written by kv3.kv_pack3;
    slot_of int32 [B][S]; n_special as for kv3.kv_unpack3.  Returns (out float64
    [B][H][D], p float64 [B][H][S])."""
    Kd = kv3.kv_unpack3(*k_pack, slot_of, D, n_special).astype(np.float64)  # [B][S][H][D]
    Vd = kv3.kv_unpack3(*v_pack, slot_of, D, n_special).astype(np.float64)
    qd = np.asarray(q, dtype=np.float64)
    z = np.einsum("bhd,bshd->bhs", qd, Kd) / np.sqrt(D)
    z = z - z.max(axis=-1, keepdims=True)
    e = np.exp(z)
    p = e / e.sum(axis=-1, keepdims=True)
    out = np.einsum("bhs,bshd->bhd", p, Vd)
    return out, p
