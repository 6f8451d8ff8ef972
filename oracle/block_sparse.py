"""Plain fp64 block-sparse attention: attention restricted by a block mask.

TEST INFRASTRUCTURE ONLY (see the package docstring).

What is computed
----------------
The pages report FlexAttention and block-sparse attention variants built
on the FlashAttention-4 kernels ([wittx], section on writing GPU kernels in
Python; [newton], development history: a FlexAttention backend).  Block
sparsity is the form of mask modification a tiled kernel can exploit: a
boolean mask over (query block, key block) pairs of BLOCK x BLOCK tokens
says which score blocks exist at all.  The definition
is ordinary softmax attention over a reduced key set per query:

    A(i) = { j : mask[b, h, i // BLOCK, j // BLOCK] != 0 }  (and j <= i if causal)
    O_i  = sum_{j in A(i)} softmax_j(scale q_i.k_j) v_j,  LSE_i = ln sum_{j in A(i)} exp(scale q_i.k_j)

A query whose A(i) is empty gets O_i = 0 and LSE_i = -inf (the limit of an
empty sum; no key contributes).  Positions i, j are within their sequence.
BLOCK is 128.
"""
from __future__ import annotations

import numpy as np

from .attention import bf16_bits_to_f64

__all__ = ["BLOCK", "block_sparse_attention_f64", "block_sparse_attention", "n_blocks"]

BLOCK = 128


def n_blocks(n: int) -> int:
    return (int(n) + BLOCK - 1) // BLOCK


def block_sparse_attention_f64(q, k, v, cu_seqlens, causal: bool, scale: float, mask, widen=None, heads=None):
    """Exact block-sparse attention.

    q, k: [T, H, d_qk]; v: [T, H, d_v]; cu_seqlens [B+1]; mask: [B, H, nb, nb]
    (any integer/bool dtype, nonzero = keep), nb = ceil(N / 128) with N >= every
    sequence length.  Returns (O [T, nH, d_v], LSE [nH, T]) in float64.
    """
    cvt = widen if widen is not None else (lambda a: np.asarray(a, dtype=np.float64))
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    mask = np.asarray(mask)
    T, H, d_qk = q.shape
    d_v = v.shape[2]
    head_list = list(range(H)) if heads is None else [int(x) for x in heads]
    O = np.zeros((T, len(head_list), d_v))
    LSE = np.full((len(head_list), T), -np.inf)
    for b in range(len(cu) - 1):
        s, e = int(cu[b]), int(cu[b + 1])
        L = e - s
        if L == 0:
            continue
        blk = np.arange(L) // BLOCK
        for hi, h in enumerate(head_list):
            vis = mask[b, h][np.ix_(blk, blk)] != 0                  # [L, L] query x key
            if causal:
                vis &= np.arange(L)[None, :] <= np.arange(L)[:, None]
            S = scale * (cvt(q[s:e, h, :]) @ cvt(k[s:e, h, :]).T)
            S[~vis] = -np.inf
            rows = vis.any(axis=1)
            m = np.where(rows, S.max(axis=1), 0.0)
            P = np.exp(S - m[:, None])                             # exp(-inf) = 0 for hidden keys
            l = P.sum(axis=1)
            out = np.zeros((L, d_v))
            out[rows] = (P[rows] @ cvt(v[s:e, h, :])) / l[rows, None]
            O[s:e, hi, :] = out
            LSE[hi, s:e] = np.where(rows, m + np.log(np.where(rows, l, 1.0)), -np.inf)
    return O, LSE


def block_sparse_attention(q_bits, k_bits, v_bits, cu_seqlens, causal: bool, scale: float, mask, heads=None):
    """Block-sparse attention on bf16 bit-pattern inputs (uint16 arrays, ``workloads`` layout)."""
    return block_sparse_attention_f64(q_bits, k_bits, v_bits, cu_seqlens, causal, scale, mask,
                                      widen=bf16_bits_to_f64, heads=heads)
