#!/usr/bin/env python3
"""Benchmark of the BitNet a4.8 hybrid-quantized BitLinear hot path on one MI355X.

One step is one pass of every hot-path kernel over synthetic 7B-shape inputs
that are resident in HBM before timing starts:

  prefill, M=2048 tokens, K=4096:    INT4 quantizer -> W1.58A4 GEMMs (N=11008, N=4096)
                                     FP4 quantizer  -> W1.58.FP4 GEMMs (N=11008, N=4096)
  sparse path, M=2048:               ReLU^2.up + top-k 50% + INT8 (K=11008) -> W1.58A8 down_proj (N=4096)
                                     top-k 50% + INT8 of a Student-t(3) input (K=4096) -> W1.58A8 out_proj
  decode, M = 1, 2, 4, 8 tokens:     INT4 quantizer -> W1.58A4 GEMV over 32 layers of fused q/k/v
                                     (N=12288) and gate/up (N=22016) weights (1.12 GB, > 4x the
                                     256 MB Infinity Cache, so weights stream from HBM); the same as
                                     one call (bw_quantize_bitlinear_a4: one launch for M <= 2);
                                     a bare read of the same weight bytes in the GEMV's launch shape
                                     (the read ceiling); one layer's q/k/v + gate/up projections on
                                     a4.8's 4-bit path against b1.58's INT8 path
  decode down_proj / out_proj, M = 1: W1.58A8 GEMV on the tiled weights vs the gather product on
                                     K-major weights (reads only the rows of nonzero codes),
                                     32 layers each
  KV cache, one layer (8x4096x32x128): 3-bit pack of K and V, unpack of both to bf16,
                                     single-token attention over the packed K and V (one
                                     launch after a cache eviction, and over 32 layers' caches)
  decoder layer, one new token for each of 8 sequences over that cache: the whole
                                     chain (bw_block_decode) over 32 layers of weights
  weights:                           absmean ternary pack of one 4096x4096 fp32 tensor

Each decode row's 32-64 launches are recorded once into a HIP graph; the other
rows are single launches.  A step runs the rows in order, each bracketed by HIP
events on the stream it runs on.  The host enqueues far faster than the GPU
drains, so an event pair measures GPU time only.
Warm-up runs the W requested steps and then keeps running untimed steps until
--settle-seconds of wall time have passed (default 1 s): the GPU raises its
clock only after tens of milliseconds of sustained load (a W1.58A4 GEMM at
N=11008 runs ~115 us in the first milliseconds and ~81 us at the sustained
clock), and the timed steps are meant to see the sustained operating point.
The printed line's `value` is the W1.58A4 prefill throughput: int ops of the
two products over the time of the INT4 quantizer followed by both products,
which share its codes and run as one grouped launch (row a0, one event pair
around the two launches); `value_from_separate_rows` divides the same ops by
the sum of the individually bracketed rows a1 + a4 (one launch per product,
each also paying its own launch latency and its own tail).
`b158_baseline` runs the same two projections on BitNet b1.58's activation
path (INT8 absmax of every entry, no top-k, W1.58A8 products grouped the same
way; row b0) and gives the ratio of the two.  `decode_gbs` is the decode GEMV rate in algorithmic
bytes (`decode_quant_gemv_gbs` with the quantizer in the same call);
`decode_read_ceiling` sets each GEMV beside the bare read of its weight bytes;
`decode_b158` compares the decode projections on the two activation paths;
`gather_decode_m1` sets the single-token gather product beside the tiled
GEMV; `roofline` covers the N=11008 prefill GEMM.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

HBM_PEAK_GBS = 8000.0
INT8_PEAK_TOPS = 5000.0  # dense int8 MFMA, MI355X
FP4_PEAK_TOPS = 10100.0  # dense fp4/fp6 MFMA, MI355X (the e2m3 x e2m1 products run at this rate)

M_PREFILL, HIDDEN, FFN = 2048, 4096, 11008

# HBM traffic of the dominant kernel (W1.58A4 GEMM on e2m3 fields, M=2048 K=4096 N=11008) from two
# rocprofv3 counter passes (FETCH_SIZE x 1.9998 + WRITE_SIZE x 1.0000, scales from a plain
# 256 MiB copy in the same runs; summary in profiles/gemm_int4_e2m3_m2048_k4096_n11008_hbm_bytes.md).
# It is reported only while the kernel sources still hash to the digest they were taken at.
GEMM_TRAFFIC = {
    "bytes": 227_119_986,
    "sources": ("gemm_lds.hip", "bw_widen.h", "bw_device.h"),
    "sha256": "6e5afd6b06fd9f492e21d8c66438bf1f47f939c5d79e4c5646fbd5bc11506de9",
}


def gemm_traffic_bytes():
    """The recorded counter traffic, or None once the GEMM sources have changed."""
    import hashlib

    csrc = os.path.join(os.path.dirname(os.path.abspath(__file__)), "ternary_weight_bit_amd", "csrc")
    h = hashlib.sha256()
    for f in GEMM_TRAFFIC["sources"]:
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(fh.read())
    return GEMM_TRAFFIC["bytes"] if h.hexdigest() == GEMM_TRAFFIC["sha256"] else None
DECODE_MS = (1, 2, 4, 8)
LAYERS = 32
KV_SHAPE = (8, 4096, 32, 128)


def parse():
    p = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=3)
    p.add_argument("--settle-seconds", type=float, default=1.0,
                   help="after the warm-up steps, keep running untimed steps until this much wall time has "
                        "passed since warm-up began (the GPU clock rises under sustained load)")
    p.add_argument("--no-cpu-baseline", action="store_true", help="skip the oracle timing leg")
    p.add_argument("--cpu-seconds", type=float, default=12.0, help="target CPU time of the oracle leg")
    p.add_argument("--rows", action="store_true", help="also print a per-row table to stderr")
    p.add_argument("--only", default="", help="comma-separated row-name prefixes: run just those rows "
                   "(for profiler passes; `value` is null unless the prefill rows are among them)")
    p.add_argument("--no-vendor-gemm", action="store_true",
                   help="skip timing the vendor library's int8/fp8 GEMMs on the prefill shapes")
    p.add_argument("--copy-calibration", action="store_true",
                   help="add a row that copies 256 MiB device-to-device (a plain copy kernel of known size, "
                        "to scale HBM byte counters)")
    return p.parse_args()


class Bench:
    """Holds device inputs/outputs and the launch list of one step."""

    def __init__(self, only=(), copy_calibration=False):
        import torch

        import synth
        import ternary_weight_bit_amd as bw

        self.torch, self.bw = torch, bw
        dev = "cuda:0"
        t = torch

        def bf16(b):
            return t.from_numpy(np.ascontiguousarray(b.bits).view(np.int16)).to(dev).view(t.bfloat16)

        def f32(a):
            return t.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(dev)

        S = synth.SEED_BASE
        # ---------------- prefill
        self.x_pre = bf16(synth.prefill_activations(S + 2, M_PREFILL, HIDDEN))
        self.w_up = f32(synth.weight_tensor(S + 12, FFN, HIDDEN))
        self.wp_11008, self.b_11008 = bw.bw_pack_ternary(self.w_up, bw.BW_ROLE_A4)
        self.wp8_11008, self.b8_11008 = bw.bw_pack_ternary(self.w_up, bw.BW_ROLE_A8)  # b1.58 baseline
        w_q = f32(synth.weight_tensor(S + 11, HIDDEN, HIDDEN))
        self.w_q = w_q
        self.wp_4096, self.b_4096 = bw.bw_pack_ternary(w_q, bw.BW_ROLE_A4)
        self.wp8_4096, self.b8_4096 = bw.bw_pack_ternary(w_q, bw.BW_ROLE_A8)
        del self.w_up
        self.c4 = t.empty((M_PREFILL, HIDDEN // 2), dtype=t.uint8, device=dev)
        self.s4 = t.empty(M_PREFILL, dtype=t.float32, device=dev)
        self.c6 = t.empty((M_PREFILL, HIDDEN // 4 * 3), dtype=t.uint8, device=dev)  # INT4 values as e2m3 fields
        self.s6 = t.empty(M_PREFILL, dtype=t.float32, device=dev)
        self.cf = t.empty_like(self.c4)
        self.sf = t.empty_like(self.s4)
        self.y_11008 = t.empty((M_PREFILL, FFN), dtype=t.float32, device=dev)
        self.y_4096 = t.empty((M_PREFILL, HIDDEN), dtype=t.float32, device=dev)
        # cache eviction between rows: a read of 384 MB (more than the 256 MB Infinity Cache)
        # through the library's streaming read; reading leaves the cache lines clean, so the
        # next timed kernel does not pay for writing back the evicting bytes, as it would
        # after a write fill
        self.evict = t.empty(384 * 1024 * 1024 // 4, dtype=t.float32, device=dev)
        self.evict_sink = t.empty(4 * ((384 * 1024 * 1024 + 16383) // 16384), dtype=t.int32, device=dev)
        self.c8_pre = t.empty((M_PREFILL, HIDDEN), dtype=t.int8, device=dev)
        self.s8_pre = t.empty(M_PREFILL, dtype=t.float32, device=dev)
        # ---------------- sparse path
        g, u = synth.gate_up(S + 3, M_PREFILL, FFN)
        self.gate, self.up = bf16(g), bf16(u)
        del g, u
        self.w_down = f32(synth.weight_tensor(S + 14, HIDDEN, FFN))
        self.wp_down, self.b_down = bw.bw_pack_ternary(self.w_down, bw.BW_ROLE_A8)
        wk_down, _ = bw.bw_pack_ternary(self.w_down, bw.BW_ROLE_A8_KMAJOR)  # single-token gather layout
        del self.w_down
        self.x_out = bf16(synth.heavy_tailed(S + 13, M_PREFILL, HIDDEN))
        self.wp_o, self.b_o = bw.bw_pack_ternary(w_q, bw.BW_ROLE_A8)
        wk_o, _ = bw.bw_pack_ternary(w_q, bw.BW_ROLE_A8_KMAJOR)
        self.c8_down = t.empty((M_PREFILL, FFN), dtype=t.int8, device=dev)
        self.s8_down = t.empty(M_PREFILL, dtype=t.float32, device=dev)
        self.c8_out = t.empty((M_PREFILL, HIDDEN), dtype=t.int8, device=dev)
        self.s8_out = t.empty(M_PREFILL, dtype=t.float32, device=dev)
        self.y_down = t.empty((M_PREFILL, HIDDEN), dtype=t.float32, device=dev)
        self.y_o = t.empty((M_PREFILL, HIDDEN), dtype=t.float32, device=dev)
        # ---------------- decode: 32 layers of fused qkv + gate/up weights
        self.n_qkv = sum(synth.QKV_PARTS)
        self.n_gu = sum(synth.GATE_UP_PARTS)
        qkv_p = t.empty(self.n_qkv * HIDDEN // 4, dtype=t.uint8, device=dev)
        qkv_b = t.empty(self.n_qkv, dtype=t.float32, device=dev)
        gu_p = t.empty(self.n_gu * HIDDEN // 4, dtype=t.uint8, device=dev)
        gu_b = t.empty(self.n_gu, dtype=t.float32, device=dev)
        for parts, seed, P, B in ((synth.QKV_PARTS, S + 21, qkv_p, qkv_b), (synth.GATE_UP_PARTS, S + 22, gu_p, gu_b)):
            off = 0
            for w in synth.fused_weights(seed, parts, HIDDEN):
                n = w.shape[0]
                bw.bw_pack_ternary(f32(w), bw.BW_ROLE_A4, P[off * HIDDEN // 4 : (off + n) * HIDDEN // 4], B[off : off + n])
                off += n
        # distinct addresses per layer (copies of one layer's packed bytes)
        self.layers = [(qkv_p.clone(), qkv_b.clone(), gu_p.clone(), gu_b.clone()) for _ in range(LAYERS)]
        del qkv_p, gu_p
        # the same projections packed for 8-bit codes (BitNet b1.58's decode path)
        qkv_p8 = t.empty(self.n_qkv * HIDDEN // 4, dtype=t.uint8, device=dev)
        gu_p8 = t.empty(self.n_gu * HIDDEN // 4, dtype=t.uint8, device=dev)
        for parts, seed, P, B in ((synth.QKV_PARTS, S + 21, qkv_p8, qkv_b), (synth.GATE_UP_PARTS, S + 22, gu_p8, gu_b)):
            off = 0
            for w in synth.fused_weights(seed, parts, HIDDEN):
                n = w.shape[0]
                bw.bw_pack_ternary(f32(w), bw.BW_ROLE_A8, P[off * HIDDEN // 4 : (off + n) * HIDDEN // 4], B[off : off + n])
                off += n
        self.layers8 = [(qkv_p8.clone(), gu_p8.clone()) for _ in range(LAYERS)]
        del qkv_p8, gu_p8
        self.sink = t.empty(4 * ((self.n_gu * HIDDEN // 4 + 16383) // 16384), dtype=t.int32, device=dev)
        self.dec = {}
        for M in DECODE_MS:
            xa = bf16(synth.decode_activations(S + 1 + M, M, HIDDEN))
            xf = bf16(synth.decode_activations(S + 101 + M, M, HIDDEN))
            self.dec[M] = dict(
                xa=xa, xf=xf,
                ca=t.empty((M, HIDDEN // 2), dtype=t.uint8, device=dev), sa=t.empty(M, dtype=t.float32, device=dev),
                cf=t.empty((M, HIDDEN // 2), dtype=t.uint8, device=dev), sf=t.empty(M, dtype=t.float32, device=dev),
                ya=t.empty((M, self.n_qkv), dtype=t.float32, device=dev),
                yf=t.empty((M, self.n_gu), dtype=t.float32, device=dev),
                c8a=t.empty((M, HIDDEN), dtype=t.int8, device=dev), s8a=t.empty(M, dtype=t.float32, device=dev),
                c8f=t.empty((M, HIDDEN), dtype=t.int8, device=dev), s8f=t.empty(M, dtype=t.float32, device=dev),
                # the same INT4 values as e2m3 fields, quantized once here (rows a5e)
                c6a=t.empty((M, HIDDEN * 3 // 4), dtype=t.uint8, device=dev), s6a=t.empty(M, dtype=t.float32, device=dev),
                c6f=t.empty((M, HIDDEN * 3 // 4), dtype=t.uint8, device=dev), s6f=t.empty(M, dtype=t.float32, device=dev),
            )
            d = self.dec[M]
            bw.bw_quantize(xa, bw.BW_ACT_INT4_E2M3, d["c6a"], d["s6a"])
            bw.bw_quantize(xf, bw.BW_ACT_INT4_E2M3, d["c6f"], d["s6f"])
        # ---------------- decode down_proj / out_proj, one token: sparsified INT8 codes
        # and 32 layers of weights in both the tiled and the K-major layout
        gd, ud = synth.gate_up(S + 31, 1, FFN)
        x1 = bf16(synth.heavy_tailed(S + 32, 1, HIDDEN))
        self.one = {}
        for name, K1, N1, tiled, kmaj, beta in (("down", FFN, HIDDEN, self.wp_down, wk_down, self.b_down),
                                                ("outproj", HIDDEN, HIDDEN, self.wp_o, wk_o, self.b_o)):
            c = t.empty((1, K1), dtype=t.int8, device=dev)
            sc = t.empty(1, dtype=t.float32, device=dev)
            if name == "down":
                bw.bw_quantize_sparse_a8(bf16(gd), bf16(ud), K1 // 2, c, sc)
            else:
                bw.bw_quantize_sparse_a8(x1, None, K1 // 2, c, sc)
            self.one[name] = dict(
                K=K1, N=N1, codes=c, scales=sc, beta=beta, nnz=int((c != 0).sum().item()),
                layers=[(tiled.clone(), kmaj.clone()) for _ in range(LAYERS)],
                ws=t.empty(bw.bw_bitlinear_sparse_a8_gather_workspace_bytes(1, K1, N1), dtype=t.uint8, device=dev),
                yt=t.empty((1, N1), dtype=t.float32, device=dev), yg=t.empty((1, N1), dtype=t.float32, device=dev))
        del gd, ud, wk_down, wk_o
        # ---------------- KV cache, one layer
        B_, S_, H_, D_ = KV_SHAPE
        self.kv = [bf16(synth.kv_tensor(S + 5 + i, *KV_SHAPE)) for i in range(2)]
        slot_of, self.n_special = synth.kv_special_slots(S + 5, B_, S_)
        self.slot_of = t.from_numpy(slot_of).to(dev)
        self.kvp = []
        for _ in range(2):
            self.kvp.append((
                t.empty((B_, S_, H_, 3 * D_ // 8), dtype=t.uint8, device=dev),
                t.empty((B_, S_, H_), dtype=t.float32, device=dev),
                t.zeros((self.n_special, H_, D_ // 2), dtype=t.uint8, device=dev),
                t.zeros((self.n_special, H_), dtype=t.float32, device=dev),
            ))
        self.kv_out = [t.empty(KV_SHAPE, dtype=t.bfloat16, device=dev) for _ in range(2)]
        # single-token attention over that layer's packed K (kvp[0]) and V (kvp[1])
        self.q_att = f32(synth.normal(S + 6, (B_, H_, D_)))
        self.att_out = t.empty((B_, H_, D_), dtype=t.float32, device=dev)
        self.att_ws = t.empty(bw.bw_attn_decode_kv3_workspace_bytes(B_, S_, H_, D_), dtype=t.uint8, device=dev)
        # ---------------- one decoder layer per new token (8 sequences, 4096 cached positions):
        # 32 layers of weights (copies of one layer's packed bytes) and of the KV cache
        HD = H_ * D_

        def pack_parts(shapes, role, seed0):
            N = sum(n for n, _ in shapes)
            K = shapes[0][1]
            wp = t.empty(N * K // 4, dtype=t.uint8, device=dev)
            bp = t.empty(N, dtype=t.float32, device=dev)
            off = 0
            for i, (n, k) in enumerate(shapes):
                bw.bw_pack_ternary(f32(synth.weight_tensor(seed0 + i, n, k)), role,
                                   wp[off * K // 4 : (off + n) * K // 4], bp[off : off + n])
                off += n
            return wp, bp

        lw = (*pack_parts([(HD, HD)] * 3, bw.BW_ROLE_A4, S + 40), *pack_parts([(HD, HD)], bw.BW_ROLE_A8, S + 43),
              *pack_parts([(FFN, HD)] * 2, bw.BW_ROLE_A4, S + 44), *pack_parts([(HD, FFN)], bw.BW_ROLE_A8, S + 46))
        self.blk_pos = S_ - 1
        self.blk_x = f32(synth.normal(S + 47, (B_, HD)))
        self.blk_out = t.empty((B_, HD), dtype=t.float32, device=dev)
        self.blk_ws = t.empty(bw.bw_block_decode_workspace_bytes(B_, S_, H_, D_, FFN), dtype=t.uint8, device=dev)
        # the layers' caches start as copies of this layer's packed K and V (real codes of
        # the synthetic K/V, not uninitialized slabs)
        for i in range(2):
            bw.bw_kv_pack3(self.kv[i], self.slot_of, self.n_special, *self.kvp[i])
        t.cuda.synchronize()
        self.blk_layers = [(tuple(w.clone() for w in lw), tuple(a.clone() for a in self.kvp[0]),
                            tuple(a.clone() for a in self.kvp[1])) for _ in range(LAYERS)]
        self.blk_weight_bytes = sum(w.numel() * w.element_size() for w in lw)
        del lw
        # ---------------- weight packing (offline row): one 4096x4096 fp32 tensor
        self.pk = t.empty(HIDDEN * HIDDEN // 4, dtype=t.uint8, device=dev)
        self.pk_b = t.empty(HIDDEN, dtype=t.float32, device=dev)
        self.pk_ws = t.empty(bw.bw_pack_ternary_workspace_bytes(HIDDEN, HIDDEN), dtype=t.uint8, device=dev)
        torch.cuda.synchronize()
        self.launches = self._launch_list()
        if only:
            self.launches = [r for r in self.launches if r[1] is None or any(r[0].startswith(o) for o in only)]
        if copy_calibration:
            n = 256 << 20
            src = t.empty(n, dtype=t.uint8, device=dev).fill_(1)
            dst = t.empty_like(src)
            self.launches.append(("z_copy_256MiB", "GB/s", 2.0 * n, [lambda: dst.copy_(src)]))

    # ------------------------------------------------------------------ launches
    def _launch_list(self):
        """Rows of the step: (name, unit, algorithmic amount per launch, [launch fns])."""
        bw = self.bw
        R = []

        def gemm_ops(M, N, K):
            return 2.0 * M * N * K

        def gemv_bytes(M, N, K):
            return N * K / 4 + 4 * N + M * K / 2 + 4 * M + 4 * M * N

        M, K = M_PREFILL, HIDDEN

        def prefill_int4():
            bw.bw_quantize(self.x_pre, bw.BW_ACT_INT4_E2M3, self.c6, self.s6)
            bw.bw_bitlinear_a4_grouped(self.c6, self.s6, bw.BW_ACT_INT4_E2M3,
                                       [(self.wp_11008, self.b_11008), (self.wp_4096, self.b_4096)],
                                       ys=[self.y_11008, self.y_4096])

        def prefill_int4_nibbles():
            bw.bw_quantize(self.x_pre, bw.BW_ACT_INT4, self.c4, self.s4)
            bw.bw_bitlinear_a4_grouped(self.c4, self.s4, bw.BW_ACT_INT4,
                                       [(self.wp_11008, self.b_11008), (self.wp_4096, self.b_4096)],
                                       ys=[self.y_11008, self.y_4096])

        # the W1.58A4 prefill hot path as one stream sequence (one event pair around
        # the INT4 quantizer and the two products, which share its codes and run as
        # one grouped launch): the basis of `value`.  The INT4 values are stored as
        # e2m3 fields and multiplied on the fp6 x fp4 matrix instruction (the same
        # accumulators and y as the nibble path, bit for bit).
        R.append(("a0_prefill_int4_sequence", "TOPS", gemm_ops(M, FFN, K) + gemm_ops(M, HIDDEN, K), [prefill_int4]))
        # untimed: read more than the 256 MB Infinity Cache, so the rows below see the
        # prefill weights cold again, as a0 did
        R.append(("_evict_cache", None, 0, [self.evict_cache]))
        # the same sequence with INT4 nibble codes on the int8 matrix instruction
        R.append(("a0n_prefill_int4_nibbles_sequence", "TOPS", gemm_ops(M, FFN, K) + gemm_ops(M, HIDDEN, K),
                  [prefill_int4_nibbles]))
        R.append(("_evict_cache_0", None, 0, [self.evict_cache]))

        def prefill_fp4():
            bw.bw_quantize(self.x_pre, bw.BW_ACT_FP4_E2M1, self.cf, self.sf)
            bw.bw_bitlinear_a4_grouped(self.cf, self.sf, bw.BW_ACT_FP4_E2M1,
                                       [(self.wp_11008, self.b_11008), (self.wp_4096, self.b_4096)],
                                       ys=[self.y_11008, self.y_4096])

        # the pages' FP4 alternative to INT4: e2m1 activation codes (per-token scale)
        # and the two products on the fp4 x fp4 matrix instruction, same sequence
        R.append(("a0f_prefill_fp4_sequence", "TOPS", gemm_ops(M, FFN, K) + gemm_ops(M, HIDDEN, K), [prefill_fp4]))
        R.append(("_evict_cache_1", None, 0, [self.evict_cache]))

        def prefill_b158():
            bw.bw_quantize_sparse_a8(self.x_pre, None, K, self.c8_pre, self.s8_pre)
            bw.bw_bitlinear_sparse_a8_grouped(self.c8_pre, self.s8_pre,
                                              [(self.wp8_11008, self.b8_11008), (self.wp8_4096, self.b8_4096)],
                                              ys=[self.y_11008, self.y_4096])

        # the same two projections on BitNet b1.58's activation path (INT8 absmax of
        # every entry, no top-k, W1.58A8 products, grouped the same way): the
        # baseline the pages compare against
        R.append(("b0_prefill_b158_int8_sequence", "TOPS", gemm_ops(M, FFN, K) + gemm_ops(M, HIDDEN, K), [prefill_b158]))
        R.append(("_evict_cache_2", None, 0, [self.evict_cache]))
        R.append(("a1e_quantize_int4_e2m3", "GB/s", M * K * 2 + M * K * 3 / 4 + 4 * M,
                  [lambda: bw.bw_quantize(self.x_pre, bw.BW_ACT_INT4_E2M3, self.c6, self.s6)]))
        R.append(("a4e_gemm_int4_e2m3_n11008", "TOPS", gemm_ops(M, FFN, K),
                  [lambda: bw.bw_bitlinear_a4(self.c6, self.s6, bw.BW_ACT_INT4_E2M3, self.wp_11008, self.b_11008,
                                              self.y_11008)]))
        R.append(("a4e_gemm_int4_e2m3_n4096", "TOPS", gemm_ops(M, HIDDEN, K),
                  [lambda: bw.bw_bitlinear_a4(self.c6, self.s6, bw.BW_ACT_INT4_E2M3, self.wp_4096, self.b_4096,
                                              self.y_4096)]))
        R.append(("a1_quantize_int4", "GB/s", M * K * 2 + M * K / 2 + 4 * M,
                  [lambda: bw.bw_quantize(self.x_pre, bw.BW_ACT_INT4, self.c4, self.s4)]))
        R.append(("a4_gemm_int4_n11008", "TOPS", gemm_ops(M, FFN, K),
                  [lambda: bw.bw_bitlinear_a4(self.c4, self.s4, bw.BW_ACT_INT4, self.wp_11008, self.b_11008, self.y_11008)]))
        R.append(("a4_gemm_int4_n4096", "TOPS", gemm_ops(M, HIDDEN, K),
                  [lambda: bw.bw_bitlinear_a4(self.c4, self.s4, bw.BW_ACT_INT4, self.wp_4096, self.b_4096, self.y_4096)]))
        R.append(("a2_quantize_fp4", "GB/s", M * K * 2 + M * K / 2 + 4 * M,
                  [lambda: bw.bw_quantize(self.x_pre, bw.BW_ACT_FP4_E2M1, self.cf, self.sf)]))
        R.append(("a6_gemm_fp4_n11008", "TOPS", gemm_ops(M, FFN, K),
                  [lambda: bw.bw_bitlinear_a4(self.cf, self.sf, bw.BW_ACT_FP4_E2M1, self.wp_11008, self.b_11008, self.y_11008)]))
        R.append(("a6_gemm_fp4_n4096", "TOPS", gemm_ops(M, HIDDEN, K),
                  [lambda: bw.bw_bitlinear_a4(self.cf, self.sf, bw.BW_ACT_FP4_E2M1, self.wp_4096, self.b_4096, self.y_4096)]))
        R.append(("a7_relu2_topk_int8_k11008", "GB/s", 2 * M * FFN * 2 + M * FFN + 4 * M,
                  [lambda: bw.bw_quantize_sparse_a8(self.gate, self.up, FFN // 2, self.c8_down, self.s8_down)]))
        R.append(("a9_gemm_a8_down", "TOPS", gemm_ops(M, HIDDEN, FFN),
                  [lambda: bw.bw_bitlinear_sparse_a8(self.c8_down, self.s8_down, self.wp_down, self.b_down, self.y_down)]))
        R.append(("a8_topk_int8_k4096", "GB/s", M * K * 2 + M * K + 4 * M,
                  [lambda: bw.bw_quantize_sparse_a8(self.x_out, None, HIDDEN // 2, self.c8_out, self.s8_out)]))
        R.append(("a9_gemm_a8_outproj", "TOPS", gemm_ops(M, HIDDEN, HIDDEN),
                  [lambda: bw.bw_bitlinear_sparse_a8(self.c8_out, self.s8_out, self.wp_o, self.b_o, self.y_o)]))

        def quant_gemv_bytes(M, N, K):  # bf16 x in, codes + scales + y out, weights + beta
            return N * K / 4 + 4 * N + 2 * M * K + M * K / 2 + 4 * M + 4 * M * N

        def gemv8_bytes(M, N, K):
            return N * K / 4 + 4 * N + M * K + 4 * M + 4 * M * N

        for Md in DECODE_MS:
            d = self.dec[Md]
            R.append((f"a1_quantize_int4_decode_m{Md}", "GB/s", Md * K * 2 + Md * K / 2 + 4 * Md,
                      [lambda d=d: bw.bw_quantize(d["xa"], bw.BW_ACT_INT4, d["ca"], d["sa"]),
                       lambda d=d: bw.bw_quantize(d["xf"], bw.BW_ACT_INT4, d["cf"], d["sf"])] * LAYERS))
            R.append((f"a5_gemv_qkv_m{Md}", "GB/s", gemv_bytes(Md, self.n_qkv, K),
                      [lambda d=d, qp=qp, qb=qb: bw.bw_bitlinear_a4(d["ca"], d["sa"], bw.BW_ACT_INT4, qp, qb, d["ya"])
                       for qp, qb, _, _ in self.layers]))
            R.append((f"a5_gemv_gateup_m{Md}", "GB/s", gemv_bytes(Md, self.n_gu, K),
                      [lambda d=d, gp=gp, gb=gb: bw.bw_bitlinear_a4(d["cf"], d["sf"], bw.BW_ACT_INT4, gp, gb, d["yf"])
                       for _, _, gp, gb in self.layers]))
            if Md in (1, 8):
                # the same products over the INT4 values stored as e2m3 fields (fp6 x fp4 GEMV)
                def gemv6_bytes(M, N, K):
                    return N * K / 4 + 4 * N + M * K * 3 / 4 + 4 * M + 4 * M * N

                R.append((f"a5e_gemv_qkv_e2m3_m{Md}", "GB/s", gemv6_bytes(Md, self.n_qkv, K),
                          [lambda d=d, qp=qp, qb=qb: bw.bw_bitlinear_a4(d["c6a"], d["s6a"], bw.BW_ACT_INT4_E2M3, qp,
                                                                        qb, d["ya"])
                           for qp, qb, _, _ in self.layers]))
                R.append((f"a5e_gemv_gateup_e2m3_m{Md}", "GB/s", gemv6_bytes(Md, self.n_gu, K),
                          [lambda d=d, gp=gp, gb=gb: bw.bw_bitlinear_a4(d["c6f"], d["s6f"], bw.BW_ACT_INT4_E2M3, gp,
                                                                        gb, d["yf"])
                           for _, _, gp, gb in self.layers]))
            if Md == DECODE_MS[0]:
                # read ceilings: the same 32 layers' weight bytes read once in the GEMV's access
                # pattern, right behind GEMV rows (same cache state: no dirty output lines of the
                # prefill rows left to write back)
                R.append(("c0_read_qkv_weights", "GB/s", self.n_qkv * K / 4,
                          [lambda qp=qp: bw.bw_stream_read(qp, self.sink) for qp, _, _, _ in self.layers]))
                R.append(("c0_read_gateup_weights", "GB/s", self.n_gu * K / 4,
                          [lambda gp=gp: bw.bw_stream_read(gp, self.sink) for _, _, gp, _ in self.layers]))
            # the 4-bit quantizer and the GEMV as one call (one launch for M <= 2)
            R.append((f"a5q_quant_gemv_qkv_m{Md}", "GB/s", quant_gemv_bytes(Md, self.n_qkv, K),
                      [lambda d=d, qp=qp, qb=qb: bw.bw_quantize_bitlinear_a4(d["xa"], bw.BW_ACT_INT4, qp, qb, d["ya"],
                                                                             d["ca"], d["sa"])
                       for qp, qb, _, _ in self.layers]))
            R.append((f"a5q_quant_gemv_gateup_m{Md}", "GB/s", quant_gemv_bytes(Md, self.n_gu, K),
                      [lambda d=d, gp=gp, gb=gb: bw.bw_quantize_bitlinear_a4(d["xf"], bw.BW_ACT_INT4, gp, gb, d["yf"],
                                                                             d["cf"], d["sf"])
                       for _, _, gp, gb in self.layers]))
            # decode projections of one layer on each activation path, 32 layers: a4.8 (4-bit
            # codes for the q/k/v and gate/up inputs) against b1.58 (INT8 absmax of every entry,
            # W1.58A8 GEMV), the comparison the pages' speed claim makes
            # (each entry is one layer: the row's average is a per-layer time)
            def a48_layer(d=d, qp=None, qb=None, gp=None, gb=None):
                bw.bw_quantize_bitlinear_a4(d["xa"], bw.BW_ACT_INT4, qp, qb, d["ya"], d["ca"], d["sa"])
                bw.bw_quantize_bitlinear_a4(d["xf"], bw.BW_ACT_INT4, gp, gb, d["yf"], d["cf"], d["sf"])

            def b158_layer(d=d, qp8=None, qb=None, gp8=None, gb=None):
                bw.bw_quantize_sparse_a8(d["xa"], None, K, d["c8a"], d["s8a"])
                bw.bw_bitlinear_sparse_a8(d["c8a"], d["s8a"], qp8, qb, d["ya"])
                bw.bw_quantize_sparse_a8(d["xf"], None, K, d["c8f"], d["s8f"])
                bw.bw_bitlinear_sparse_a8(d["c8f"], d["s8f"], gp8, gb, d["yf"])

            R.append((f"d0_decode_a48_m{Md}", "GB/s",
                      quant_gemv_bytes(Md, self.n_qkv, K) + quant_gemv_bytes(Md, self.n_gu, K),
                      [lambda qp=qp, qb=qb, gp=gp, gb=gb, f=a48_layer: f(qp=qp, qb=qb, gp=gp, gb=gb)
                       for qp, qb, gp, gb in self.layers]))
            R.append((f"d1_decode_b158_m{Md}", "GB/s",
                      2 * (Md * K * 2 + Md * K + 4 * Md) + gemv8_bytes(Md, self.n_qkv, K)
                      + gemv8_bytes(Md, self.n_gu, K),
                      [lambda qp8=qp8, qb=qb, gp8=gp8, gb=gb, f=b158_layer: f(qp8=qp8, qb=qb, gp8=gp8, gb=gb)
                       for (qp8, gp8), (_, qb, _, gb) in zip(self.layers8, self.layers)]))
        for name, o in self.one.items():
            K1, N1 = o["K"], o["N"]
            # tiled W1.58A8 GEMV: every weight byte; gather: only the rows of nonzero codes.
            # Each row starts behind an untimed cache fill: the gather's rows of all 32 layers
            # (~108 MB for down_proj) would otherwise stay in the 256 MB Infinity Cache.
            R.append((f"_evict_cache_{name}_t", None, 0, [self.evict_cache]))
            R.append((f"a9_gemv_a8_{name}_m1", "GB/s", N1 * K1 / 4 + 4 * N1 + K1 + 4 + 4 * N1,
                      [lambda o=o, wt=wt: bw.bw_bitlinear_sparse_a8(o["codes"], o["scales"], wt, o["beta"], o["yt"])
                       for wt, _ in o["layers"]]))
            R.append((f"_evict_cache_{name}_g", None, 0, [self.evict_cache]))
            R.append((f"k10_gather_a8_{name}_m1", "GB/s", o["nnz"] * N1 / 4 + 4 * N1 + K1 + 4 + 4 * N1,
                      [lambda o=o, wk=wk: bw.bw_bitlinear_sparse_a8_gather(o["codes"], o["scales"], wk, o["beta"],
                                                                           o["ws"], o["yg"])
                       for _, wk in o["layers"]]))
        B_, S_, H_, D_ = KV_SHAPE
        nvec = B_ * S_ * H_
        pack_bytes = nvec * D_ * 2 + nvec * (3 * D_ // 8) + 4 * nvec + 4 * B_ * S_ + self.n_special * H_ * (D_ // 2 + 4)
        R.append(("a10_kv_pack3", "GB/s", pack_bytes,
                  [lambda i=i: bw.bw_kv_pack3(self.kv[i], self.slot_of, self.n_special, *self.kvp[i]) for i in range(2)]))
        R.append(("a10_kv_unpack3", "GB/s", pack_bytes,
                  [lambda i=i: bw.bw_kv_unpack3(*self.kvp[i], self.slot_of, self.n_special,
                                                out_dtype=self.torch.bfloat16, out=self.kv_out[i]) for i in range(2)]))
        # single-token attention over the packed cache: algorithmic bytes are the 3-bit
        # planes and scales of K and V, slot ids, both side slabs, q and out
        att_bytes = (2 * nvec * (3 * D_ // 8 + 4) + 4 * B_ * S_ + 2 * self.n_special * H_ * (D_ // 2 + 4)
                     + 2 * 4 * B_ * H_ * D_)
        R.append(("_evict_cache_attn", None, 0, [self.evict_cache]))
        R.append(("k11_attn_decode_kv3", "GB/s", att_bytes,
                  [lambda: bw.bw_attn_decode_kv3(self.q_att, self.kvp[0], self.kvp[1], self.slot_of, self.n_special,
                                                 self.att_out)]))
        # the same attention over each of the 32 layers' caches in turn (each read cold, as a
        # decode step reads them), averaged per layer
        R.append(("_evict_cache_attn_l", None, 0, [self.evict_cache]))
        R.append(("k11l_attn_decode_kv3_layers", "GB/s", att_bytes,
                  [lambda kc=kc, vc=vc: bw.bw_attn_decode_kv3(self.q_att, kc, vc, self.slot_of, self.n_special,
                                                              self.att_out, workspace=self.att_ws)
                   for _, kc, vc in self.blk_layers]))
        # one decoder layer per new token: algorithmic bytes = the layer's packed weights and
        # beta + the attended cache (as the attention row) + small activations
        blk_bytes = self.blk_weight_bytes + att_bytes
        R.append(("_evict_cache_blk", None, 0, [self.evict_cache]))
        R.append(("k12_block_decode_b8", "GB/s", blk_bytes,
                  [lambda lw=lw, kc=kc, vc=vc: bw.bw_block_decode(self.blk_x, lw, kc, vc, self.slot_of, self.n_special,
                                                                  self.blk_pos, H_, x_out=self.blk_out,
                                                                  workspace=self.blk_ws)
                   for lw, kc, vc in self.blk_layers]))
        R.append(("a3_pack_ternary_4096x4096", "GB/s", HIDDEN * HIDDEN * 4 + HIDDEN * HIDDEN / 4 + 4 * HIDDEN,
                  [lambda: bw.bw_pack_ternary(self.w_q, bw.BW_ROLE_A4, self.pk, self.pk_b, self.pk_ws)]))
        return R

    def evict_cache(self):
        self.bw.bw_stream_read(self.evict, self.evict_sink)

    def capture(self):
        """Record each multi-launch row (the decode loops) once into a HIP graph (no
        allocation, no memset inside), so a replay costs the host one call for the
        row; single-launch rows are launched directly."""
        torch = self.torch
        self.graphs = []
        for name, _, _, fns in self.launches:
            if len(fns) == 1:
                self.graphs.append(fns[0])
                continue
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=torch.cuda.current_stream()):
                for fn in fns:
                    fn()
            self.graphs.append(g.replay)

    def step_eager(self):
        for _, _, _, fns in self.launches:
            for fn in fns:
                fn()

    def step(self, ev=None):
        stream = self.torch.cuda.current_stream()
        for i, run in enumerate(self.graphs):
            if ev is not None:
                ev[2 * i].record(stream)
            run()
            if ev is not None:
                ev[2 * i + 1].record(stream)


def vendor_gemm_reference(reps: int = 20):
    """The vendor library's dense GEMMs on the prefill shapes, for context: int8 x int8 -> int32
    (torch._int_mm) and fp8 e4m3 (torch._scaled_mm), both with plain 8-bit operands (no 4-bit or
    2-bit unpacking).  Not part of `value`."""
    import torch

    dev = "cuda:0"
    out = {}
    for N in (FFN, HIDDEN):
        a = torch.randint(-7, 8, (M_PREFILL, HIDDEN), dtype=torch.int8, device=dev)
        b = torch.randint(-1, 2, (N, HIDDEN), dtype=torch.int8, device=dev).t()
        one = torch.ones((), device=dev)
        cases = {"int8_int_mm": lambda: torch._int_mm(a, b)}
        try:
            a8, b8 = a.to(torch.float8_e4m3fn), b.to(torch.float8_e4m3fn)
            cases["fp8_scaled_mm"] = lambda: torch._scaled_mm(a8, b8, one, one, out_dtype=torch.bfloat16)
        except Exception:  # pragma: no cover - dtype missing in this build
            pass
        for name, fn in cases.items():
            try:
                for _ in range(3):
                    fn()
                torch.cuda.synchronize()
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record()
                for _ in range(reps):
                    fn()
                e1.record()
                torch.cuda.synchronize()
                us = e0.elapsed_time(e1) * 1e3 / reps
                out[f"{name}_m{M_PREFILL}_k{HIDDEN}_n{N}"] = {
                    "avg_us": round(us, 2), "TOPS": round(2.0 * M_PREFILL * N * HIDDEN / us / 1e6, 1)}
            except Exception as e:  # pragma: no cover - library call unavailable
                out[f"{name}_m{M_PREFILL}_k{HIDDEN}_n{N}"] = {"error": str(e)[:120]}
    return out


def _cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:  # pragma: no cover
        pass
    return "unknown"


def cpu_baseline(target_s: float):
    """The oracle, as it stands, on a bounded sample of the W1.58A4 prefill work:
    INT4 quantizer + exact contraction + epilogue for a sample of token rows
    against the N=11008 and N=4096 weights (already ternarized, as on the GPU side),
    once with every host thread the BLAS library uses and once on one thread."""
    import synth
    from oracle import act4, bitlinear, ternary

    try:
        from threadpoolctl import threadpool_info, threadpool_limits
    except Exception:  # pragma: no cover
        threadpool_info = threadpool_limits = None
    S = synth.SEED_BASE
    x = synth.prefill_activations(S + 2, M_PREFILL, HIDDEN).f32
    weights = []
    for seed, n in ((S + 12, FFN), (S + 11, HIDDEN)):
        t, b = ternary.quantize_weights(synth.weight_tensor(seed, n, HIDDEN))
        weights.append((t, np.full(n, b, np.float32)))

    def run(rows):
        t0 = time.perf_counter()
        for tq, beta in weights:
            bitlinear.bitlinear_a4_int4(x[:rows], tq, beta)
        return time.perf_counter() - t0

    def leg(budget_s):
        rows = 32
        dt = run(rows)
        while dt < budget_s / 4 and rows < M_PREFILL:
            rows = min(M_PREFILL, rows * 4)
            dt = run(rows)
        # the whole workload finishes well under the budget: repeat it to about budget_s
        reps = max(1, min(64, int(budget_s / max(dt, 1e-3))))
        if reps > 1:
            dt = sum(run(rows) for _ in range(reps))
        ops = 2.0 * rows * HIDDEN * (FFN + HIDDEN) * reps
        return ops / dt / 1e12, rows, reps, dt

    threads = max([d.get("num_threads", 1) for d in threadpool_info()] + [1]) if threadpool_info else os.cpu_count()
    v_all, rows, reps, dt = leg(target_s)
    single = None
    if threadpool_limits is not None:
        with threadpool_limits(limits=1):
            v1, rows1, reps1, dt1 = leg(target_s / 3)
        single = {"value": v1, "unit": "TOPS", "cores": 1,
                  "sample": f"{rows1} of 2048 token rows, {reps1} passes; {dt1:.1f} s"}
    return {
        "value": v_all,
        "unit": "TOPS",
        "cores": int(threads),
        "kind": "oracle",
        "sample": f"W1.58A4 prefill (INT4 quantize + exact contraction + epilogue) on {rows} of 2048 token rows, "
                  f"K=4096, N=11008 and N=4096, {reps} passes; {dt:.1f} s",
        "single_thread": single,
        "cpu_model": _cpu_model(),
        "logical_cpus": os.cpu_count(),
    }


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the hot path is data-parallel and would shard by tokens or output channels)", file=sys.stderr)
        return 2
    import torch

    torch.cuda.set_device(0)
    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        t0 = time.perf_counter()
        b = Bench(only=tuple(o for o in args.only.split(",") if o), copy_calibration=args.copy_calibration)
        print(f"bench: inputs resident ({time.perf_counter() - t0:.1f} s)", file=sys.stderr, flush=True)
        n_rows = len(b.launches)
        b.step_eager()  # eager pass before capture
        torch.cuda.synchronize()
        b.capture()
        print("bench: row graphs captured", file=sys.stderr, flush=True)
        w0 = time.perf_counter()
        n_warm = 0
        while n_warm < args.warmup or time.perf_counter() - w0 < args.settle_seconds:
            b.step()
            n_warm += 1
            if n_warm % 16 == 0:
                torch.cuda.synchronize()  # keep the host within a few steps of the GPU
        torch.cuda.synchronize()
        print(f"bench: {n_warm} untimed warm-up steps ({time.perf_counter() - w0:.2f} s)", file=sys.stderr, flush=True)
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(2 * n_rows)] for _ in range(args.steps)]
        t_start = torch.cuda.Event(enable_timing=True)
        t_end = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        # one untimed step in flight ahead of the timed region, so the GPU is busy
        # (and the host ahead of it) from the first timed event on
        b.step()
        wall0 = time.perf_counter()
        t_start.record(stream)
        for s_ in range(args.steps):
            b.step(evs[s_])
        t_end.record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - wall0
    ms_total = t_start.elapsed_time(t_end)
    ms_per_step = ms_total / args.steps

    # per-row statistics: average launch duration = row time / launches in the row
    table = {}
    for i, (name, unit, amount, fns) in enumerate(b.launches):
        if unit is None:  # untimed helper row
            continue
        row_ms = [evs[s_][2 * i].elapsed_time(evs[s_][2 * i + 1]) for s_ in range(args.steps)]
        avg_ms = float(np.mean(row_ms)) / len(fns)
        rate = amount / (avg_ms * 1e-3) / (1e9 if unit == "GB/s" else 1e12)
        peak = HBM_PEAK_GBS if unit == "GB/s" else (
            FP4_PEAK_TOPS if ("fp4" in name or "e2m3" in name or name.startswith(("a0_", "a0f_"))) else INT8_PEAK_TOPS)
        table[name] = {"avg_us": round(avg_ms * 1e3, 3), "launches_per_step": len(fns), "rate": round(rate, 2),
                       "unit": unit, "frac_of_peak": round(rate / peak, 4), "amount_per_launch": amount,
                       # spread over the timed steps (per launch), to show steps that ran slow
                       "min_us": round(min(row_ms) * 1e3 / len(fns), 3),
                       "max_us": round(max(row_ms) * 1e3 / len(fns), 3)}

    def row_ms(names):
        return sum(table[n]["avg_us"] * table[n]["launches_per_step"] for n in names) / 1e3

    prefill_ops = 2.0 * M_PREFILL * HIDDEN * (FFN + HIDDEN)
    prefill_rows = ("a1e_quantize_int4_e2m3", "a4e_gemm_int4_e2m3_n11008", "a4e_gemm_int4_e2m3_n4096")
    value = value_rows = None
    if "a0_prefill_int4_sequence" in table:
        value = round(prefill_ops / (row_ms(("a0_prefill_int4_sequence",)) * 1e-3) / 1e12, 2)
    if all(n in table for n in prefill_rows):
        value_rows = round(prefill_ops / (row_ms(prefill_rows) * 1e-3) / 1e12, 2)
    nibbles = None
    if "a0n_prefill_int4_nibbles_sequence" in table:
        nibbles = round(prefill_ops / (row_ms(("a0n_prefill_int4_nibbles_sequence",)) * 1e-3) / 1e12, 2)
    fp4seq = None
    if "a0f_prefill_fp4_sequence" in table:
        fp4seq = round(prefill_ops / (row_ms(("a0f_prefill_fp4_sequence",)) * 1e-3) / 1e12, 2)
    b158 = None
    if "b0_prefill_b158_int8_sequence" in table:
        b158 = round(prefill_ops / (row_ms(("b0_prefill_b158_int8_sequence",)) * 1e-3) / 1e12, 2)
    gemv = [n for n in table if n.startswith("a5_gemv")]
    decode_gbs = None
    if gemv:
        dec_bytes = sum(table[n]["amount_per_launch"] * table[n]["launches_per_step"] for n in gemv)
        decode_gbs = dec_bytes / (row_ms(gemv) * 1e-3) / 1e9
    decode_q = None
    gemvq = [n for n in table if n.startswith("a5q_quant_gemv")]
    if gemvq:
        dq_bytes = sum(table[n]["amount_per_launch"] * table[n]["launches_per_step"] for n in gemvq)
        decode_q = round(dq_bytes / (row_ms(gemvq) * 1e-3) / 1e9, 1)
    # the GEMV against a bare read of the same weight bytes in the same launch shape
    read_ceiling = {}
    for proj in ("qkv", "gateup"):
        rn = f"c0_read_{proj}_weights"
        if rn not in table:
            continue
        e = {"read_us": table[rn]["avg_us"], "read_gbs": table[rn]["rate"],
             "read_frac_hbm": table[rn]["frac_of_peak"]}
        for Md in DECODE_MS:
            for kind, gn in (("gemv", f"a5_gemv_{proj}_m{Md}"), ("quant_gemv", f"a5q_quant_gemv_{proj}_m{Md}")):
                if gn in table:
                    e[f"{kind}_m{Md}_us"] = table[gn]["avg_us"]
                    e[f"{kind}_m{Md}_read_over_time"] = round(table[rn]["avg_us"] / table[gn]["avg_us"], 3)
        read_ceiling[proj] = e
    decode_b158 = {}
    for Md in DECODE_MS:
        a, b_ = f"d0_decode_a48_m{Md}", f"d1_decode_b158_m{Md}"
        if a in table and b_ in table:
            decode_b158[f"m{Md}"] = {"a48_us_per_layer": table[a]["avg_us"], "b158_us_per_layer": table[b_]["avg_us"],
                                     "a48_over_b158_speed": round(table[b_]["avg_us"] / table[a]["avg_us"], 3)}
    block = None
    if "k12_block_decode_b8" in table:
        block = {"us_per_layer": table["k12_block_decode_b8"]["avg_us"],
                 "basis": "one decoder layer for one new token of each of 8 sequences with 4096 cached positions "
                          "(INT4 q/k/v, 3-bit KV append and attention, top-k INT8 out_proj, INT4 gate/up, "
                          "ReLU^2 top-k INT8 down_proj, residuals), averaged over 32 layers of weights and caches"}
    attn = None
    if "k11_attn_decode_kv3" in table and "k11l_attn_decode_kv3_layers" in table:
        attn = {"single_launch_after_eviction_us": table["k11_attn_decode_kv3"]["avg_us"],
                "per_layer_us": table["k11l_attn_decode_kv3_layers"]["avg_us"],
                "basis": "one new query per (batch, head) over 8 x 4096 cached positions, 32 heads of 128: one "
                         "launch right after a 384 MB cache eviction (row k11), and the average over 32 layers' "
                         "caches launched in turn, each read cold from HBM (row k11l)"}
    gather = {}
    for name, o in b.one.items():
        rt, rg = f"a9_gemv_a8_{name}_m1", f"k10_gather_a8_{name}_m1"
        if rt in table and rg in table:
            gather[name] = {
                "K": o["K"], "N": o["N"], "nonzero_codes": o["nnz"],
                "weight_bytes_read_frac": round(o["nnz"] / o["K"], 4),
                "tiled_us": table[rt]["avg_us"], "gather_us": table[rg]["avg_us"],
                "tiled_over_gather_time": round(table[rt]["avg_us"] / table[rg]["avg_us"], 3)}
    roof = None
    if "a4e_gemm_int4_e2m3_n11008" in table:
        dom = table["a4e_gemm_int4_e2m3_n11008"]
        roof = {
            "bound": "mfma", "kernel": "k_gemm_lds256<E2M3> (W1.58A4 GEMM, INT4 values as e2m3 fields, "
                                       "M=2048 K=4096 N=11008)",
            "achieved": dom["rate"], "peak": FP4_PEAK_TOPS, "unit": "TFLOP/s",
            "frac": round(dom["rate"] / FP4_PEAK_TOPS, 4), "traffic": gemm_traffic_bytes(),
            "note": "ops (2*M*N*K per launch) on the fp6 x fp4 MFMA (dense peak 10.1 POPS) / average launch "
                    "duration from HIP events; traffic = HBM bytes per launch from rocprofv3 FETCH_SIZE/WRITE_SIZE "
                    "(copy-calibrated)",
        }
        if "a4_gemm_int4_n11008" in table:
            nb = table["a4_gemm_int4_n11008"]
            roof["int4_nibble_path"] = {
                "kernel": "k_gemm_lds256<INT4> (same product, INT4 nibbles widened to int8)", "avg_us": nb["avg_us"],
                "achieved": nb["rate"], "peak": INT8_PEAK_TOPS, "frac": nb["frac_of_peak"]}
    out = {
        "metric": "BitLinear W1.58A4 prefill TOPS + decode GEMV HBM GB/s at 7B shapes, 1 GPU",
        "value": value,
        "unit": "TOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "warmup_steps_run": n_warm,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int4 (as e2m3 fp6 fields) x ternary (as e2m1) -> exact fp32 sums (prefill); e2m1 fp4, int8 on "
                 "the other rows",
        "data": "synthetic (seeded N(0,1)/Student-t activations, N(0,0.02) weights; 7B Llama-like shapes)",
        "config": {"workload": "a4.8 BitLinear hot path at 7B shapes: prefill M=2048 K=4096 N=11008/4096 "
                               "(INT4+FP4), sparse A8 down/out_proj M=2048, decode GEMV M=1,2,4,8 over 32 layers "
                               "of qkv (N=12288) + gate/up (N=22016), KV 3-bit pack/unpack 8x4096x32x128, "
                               "ternary pack 4096x4096; also the M=1 gather GEMV (down/out_proj), attention over "
                               "the 3-bit cache 8x4096x32x128 and one decoder layer for 8 sequences x 4096 cached "
                               "positions", "global_batch": M_PREFILL, "seq_len": KV_SHAPE[1],
                   "parallelism": "none (1 GPU)"},
        "value_basis": "2*2048*4096*(11008+4096) ops / time of the INT4 quantizer (values stored as e2m3 fields) "
                       "+ the W1.58A4 products N=11008 and N=4096 over its codes (one grouped launch on the fp6 x "
                       "fp4 MFMA; accumulators and y equal to the INT4 nibble path bit for bit), back to back as "
                       "one stream sequence (row a0)",
        "value_from_separate_rows": value_rows,
        "int4_nibble_sequence": None if nibbles is None else {
            "value": nibbles, "unit": "TOPS",
            "basis": "the same sequence with INT4 nibble codes widened to int8 for the int8 MFMA (row a0n)"},
        "fp4_sequence": None if fp4seq is None else {
            "value": fp4seq, "unit": "TOPS", "frac_of_fp4_peak": round(fp4seq / FP4_PEAK_TOPS, 4),
            "basis": "the same two products with FP4 e2m1 activation codes (the pages' alternative to INT4, "
                     "per-token scale): e2m1 quantizer + both W1.58 x FP4 products in one grouped launch on the "
                     "fp4 x fp4 MFMA, back to back (row a0f); a variant beside value, not its basis"},
        "b158_baseline": None if b158 is None else {
            "value": b158, "unit": "TOPS",
            "basis": "same ops / time of INT8 absmax (all entries, no top-k) + the two W1.58A8 products over its "
                     "codes (one grouped launch), back to back (row b0)",
            "a48_over_b158": None if value is None else round(value / b158, 3)},
        "gather_decode_m1": gather or None,
        "attn_decode_kv3": attn,
        "block_decode": block,
        "decode_gbs": None if decode_gbs is None else round(decode_gbs, 1),
        "decode_frac_hbm": None if decode_gbs is None else round(decode_gbs / HBM_PEAK_GBS, 4),
        "decode_quant_gemv_gbs": decode_q,
        "decode_read_ceiling": read_ceiling or None,
        "decode_b158": None if not decode_b158 else {
            "basis": "one layer's q/k/v and gate/up projections for M tokens, 32 layers: a4.8 = 4-bit quantizer + "
                     "W1.58A4 GEMV (bw_quantize_bitlinear_a4, one launch for M <= 2) per projection; b1.58 = INT8 "
                     "absmax of every entry + W1.58A8 GEMV per projection; speed ratio = b1.58 time / a4.8 time",
            **decode_b158},
        "roofline": roof,
        "rows": table,
        "wall_s_timed": round(wall, 3),
    }
    print(f"bench: timed {args.steps} steps, {ms_per_step:.3f} ms/step", file=sys.stderr, flush=True)
    if not args.no_vendor_gemm and not args.only:
        out["vendor_gemm_reference"] = vendor_gemm_reference()
    if not args.no_cpu_baseline and not args.only:
        out["cpu_baseline"] = cpu_baseline(args.cpu_seconds)
    if args.rows:
        for n, r in table.items():
            print(f"{n:34s} {r['avg_us']:10.2f} us x{r['launches_per_step']:4d}  {r['rate']:9.1f} {r['unit']:5s} "
                  f"{100 * r['frac_of_peak']:6.1f}%  [{r['min_us']:.2f} .. {r['max_us']:.2f} us]", file=sys.stderr)
    print(json.dumps(out))
    return 0


if __name__ == "__main__":
    sys.exit(main())
