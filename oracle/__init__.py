"""CPU oracle for the BitNet a4.8 hybrid-quantized BitLinear path.

TEST INFRASTRUCTURE.  This package is a plain, slow, obviously-correct numpy
statement of what the path computes.  Only the test suite, the smoke check and
the benchmark's CPU-baseline leg may import it; the product path (the HIP
library and its Python binding) never does, and shares no code with it.

Sources.  The method is described on these pages (cited by title and section;
the pages print no formula, table or worked example):

* "BitNet a4.8: 4-bit Activations for 1-bit LLMs", abstract (arXiv 2411.04965v1,
  reproduced on the shd-paper.top and groovesquid.com summary pages) -- 4-bit
  activations for the inputs of attention and FFN, sparsified intermediate
  states followed by 8-bit quantization, INT4/FP4 kernels, 3-bit KV cache.
* shd-paper.top summary of the same paper, sections 方法详解 (技术框架 / 关键设计)
  -- the same split of layers, stated as a pipeline.
* toshoseti Telegram review of BitNet a4.8, paragraph «Метод» -- which layers get
  4-bit activations (q/k/v/gate/up), top-k sparsification at 50 % for the out
  projection input, ReLU^2 in place of swish in the FFN gate, FP4 as an
  alternative to INT4; paragraph «Эксперименты» -- 3-bit KV cache with the
  bos/eos tokens kept at 4 bits; and its opening lines -- BitNet b1.58 has
  ternary weights and absmax INT8 activations.
* 9pt.com article on BitNet a4.8 (methodology paragraph) -- sparsity drops
  low-magnitude activation entries.

Where the pages are silent the oracle takes one explicit reading; every
reading is listed, with its reason, in the design notes at the repository root.
The arithmetic conventions are:

* every quantizer decision is taken in IEEE fp32, one correctly-rounded
  operation at a time (numpy float32 ops; no fused multiply-add), with
  round-half-to-even (``np.rint``);
* contractions are exact integer sums (int64 here);
* dequantized outputs are computed in fp64 and compared with a relative
  tolerance.

Modules: ``act4`` (INT4 / FP4 activation quantizers), ``ternary`` (absmean
ternary weights and their 2-bit packing), ``bitlinear`` (the contractions and
the dequant epilogue), ``sparse8`` (ReLU^2 gate, top-k, INT8), ``kv3`` (3-bit
KV cache codec).  Each function is pinned by the ``-m "not gpu"`` tests to
hand-derived examples, closed forms, invariants or brute force.
"""
from . import act4, bitlinear, kv3, sparse8, ternary  # noqa: F401

__all__ = ["act4", "bitlinear", "kv3", "sparse8", "ternary"]
