"""CPU oracle for the fused exact-attention forward pass.

TEST INFRASTRUCTURE ONLY.  Nothing in the library's product path imports,
calls or links anything in this package: only the tests, the smoke check
and the CPU-baseline leg of the benchmark use it.  It shares no code with
the HIP kernels (no kernels, headers, helpers, tables or constant
generators); the only module both sides use is ``workloads`` (seeded input
draws, which hold none of the method's arithmetic).

Contents
--------
``attention``       plain fp64 softmax attention, the definition the tiled
                    online-softmax method reaches exactly (up to rounding).
``online_softmax``  the tile-by-tile online softmax with conditional
                    rescaling, in fp64, following the algorithm's steps;
                    used to pin that conditional rescaling is exact and to
                    count how many rescales a threshold skips.
``exp2_poly``       the Cody-Waite range-reduced degree-3 polynomial exp2
                    and its relative-minimax (Remez) coefficient fit.
``attention_backward``  the plain fp64 gradient of softmax attention (dQ, dK,
                    dV and the row term D) by the chain rule.
``block_sparse``    plain fp64 attention restricted by a 128 x 128 block mask.
``fp8``             the OCP E4M3 decode and attention of dequantised FP8 inputs.

Sources (web pages about FlashAttention-4):
  [ainexis]  ainexis.cn deep dive on Tri Dao's FlashAttention-4
             algorithm/kernel co-design
  [wittx]    wittx news "FlashAttention-4" (2026-03-11)
  [newton]   newton.com.tw wiki "FlashAttention-4"
  [jsqmd]    jsqmd.com news "GPU 算力翻倍，AI 反而变慢了？FlashAttention-4 给出了惊人的答案"

Parity status: every function here is pinned by ``tests/test_oracle.py``,
``tests/test_oracle_backward.py``, ``tests/test_oracle_block_sparse.py``, ``tests/test_oracle_fp8.py`` and
``tests/test_exp2_poly.py`` against closed forms, invariants, an
mpmath brute force and the pages' stated constants; none is
"parity unpinned".
"""
from .attention import attention, attention_f64, attention_probs_f64, bf16_bits_to_f64
from .online_softmax import online_softmax_attention_f64
from .attention_backward import attention_backward, attention_backward_f64
from .block_sparse import block_sparse_attention, block_sparse_attention_f64
from .fp8 import attention_fp8, e4m3_to_f64
from .exp2_poly import (exp2_poly_f64, exp2_poly_f32, remez_exp2_relative,
                        poly_relative_error)

__all__ = [
    "attention", "attention_f64", "attention_probs_f64", "bf16_bits_to_f64",
    "online_softmax_attention_f64", "attention_backward", "attention_backward_f64",
    "block_sparse_attention", "block_sparse_attention_f64",
    "exp2_poly_f64", "exp2_poly_f32", "remez_exp2_relative", "poly_relative_error",
    "attention_fp8", "e4m3_to_f64",
]
