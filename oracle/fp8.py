"""Attention on FP8 (e4m3) inputs, in fp64: the definition the FP8 kernel reaches.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Source of the variant: the pages name FP8 as the low-precision arithmetic the
Hopper generation adopted ([ainexis], background section, third stage) and as
a precision future versions will support ([wittx], closing section "FA4越快，
Mamba们越尴尬").  They give no formulas for it, so the plain reading is taken:
the inputs are stored as 8-bit floats with one positive fp32 dequantisation
factor per tensor, and the operation is ordinary softmax attention of the
dequantised values,

    q = q_descale * fp8(Q8),  k = k_descale * fp8(K8),  v = v_descale * fp8(V8)
    O, LSE = attention(q, k, v)            (``attention.attention_f64``)

The 8-bit format is the OCP "E4M3" encoding: bit 7 sign, bits 6..3 a biased
exponent (bias 7), bits 2..0 the mantissa.  Exponent field 0 holds the
subnormals m/8 * 2^-6; every other exponent field e holds (1 + m/8) * 2^(e-7);
S.1111.111 is NaN and there are no infinities, so the largest finite value is
1.75 * 2^8 = 448.  ``e4m3_to_f64`` writes that definition out bit by bit.

Every e4m3 value is exact in fp64, so the dequantised inputs are exact and the
rest is the pinned fp64 attention oracle.  How the GPU kernel rounds P for its
second product is not part of the definition; the tests bound that rounding's
effect separately.
"""
from __future__ import annotations

import numpy as np

from .attention import attention_f64

__all__ = ["e4m3_to_f64", "attention_fp8"]


def e4m3_to_f64(codes: np.ndarray) -> np.ndarray:
    """Decode OCP E4M3 bit patterns (uint8) to float64 (exact; NaN for S.1111.111)."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where((c >> 7) & 1, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    sub = m / 8.0 * 2.0 ** -6
    norm = (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - 7.0)
    mag = np.where(e == 0, sub, norm)
    mag = np.where((e == 0xF) & ((c & 0x7) == 0x7), np.nan, mag)
    return sign * mag


def attention_fp8(q8, k8, v8, cu_seqlens, causal: bool, scale: float,
                  q_descale: float = 1.0, k_descale: float = 1.0, v_descale: float = 1.0,
                  rows=None, heads=None, block: int = 1024):
    """Exact attention of the dequantised e4m3 inputs.

    q8, k8: uint8 [T, H, d_qk]; v8: uint8 [T, H, d_v]; descales are the fp32
    factors the stored values are multiplied by.  Returns (O [R, nH, d_v],
    LSE [nH, R]) in float64, with the row and head selection of
    ``attention_f64``.
    """
    # attention_f64 widens every operand with one function; hand it views
    # that decode and scale each slice it takes.
    class _Scaled:
        def __init__(self, arr, f):
            self.arr, self.f = arr, float(f)
            self.shape = arr.shape

        def __getitem__(self, idx):
            return e4m3_to_f64(self.arr[idx]) * self.f

    return attention_f64(_Scaled(np.asarray(q8), q_descale), _Scaled(np.asarray(k8), k_descale),
                         _Scaled(np.asarray(v8), v_descale), cu_seqlens, causal, scale,
                         rows=rows, block=block, heads=heads)
