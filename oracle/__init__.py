"""CPU oracle for packed, variable-length, interval-masked attention (forward and
gradients).

TEST INFRASTRUCTURE ONLY.  Only tests/, __graft_entry__.smoke() and the
cpu_baseline leg of bench.py may import this package.  It shares no code
with the HIP path (packed_varlen_masked_amd) and never imports it.

Every floating-point step is NumPy float64; integer steps use int64.
Each function cites the passage of the pages it follows:
  [FM]  PaddleNLP FlashMask article (m.nxbn.cn/news/70198)
  [VP]  Varlen-Packing technical document (www.gsyq.cn/news/432802)
  [US]  Unsloth packing blog (unsloth.ai, "3x faster training + packing"): packing,
        the fused QK RoPE

Pinning status (what fixes each function other than itself) is listed in
the docstring of each function; every function here is pinned.
"""
from .flashmask import (  # noqa: F401
    FULL, PARTIAL, UNMASKED,
    fill_vectors, element_mask, attention, attention_rows, attention_bwd,
    attention_bwd_rows, extrema,
    classify, class_counts, worklist, unmasked_pairs, effective_flops,
    fa_varlen_grid_blocks, rope,
    philox4x32_10, dropout_threshold, dropout_keep, attention_dropout, attention_bwd_dropout,
)
