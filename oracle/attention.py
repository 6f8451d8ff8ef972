"""Plain fp64 softmax attention: the definition the tiled method reaches.

TEST INFRASTRUCTURE ONLY (see the package docstring).

What is computed
----------------
For every sequence b (tokens cu[b] .. cu[b+1]-1, length L), every head h and
every query row i of that sequence:

    s_ij   = scale * sum_c q_ic k_jc          for keys j in A(i)
    A(i)   = {0..L-1}                          non-causal
           = {0..i}                            causal (square: L_q = L_k)
    m_i    = max_j s_ij
    l_i    = sum_j exp(s_ij - m_i)
    O_i    = sum_j exp(s_ij - m_i) v_j / l_i
    LSE_i  = m_i + ln l_i                      (natural log of the scaled logits)

This is exact softmax attention with an N x N score matrix -- the standard
formulation whose score matrix the FlashAttention line avoids writing to HBM
([ainexis], background section on the memory wall; [jsqmd] sections one and
two).  The tiled online-softmax computation with a running max and running
sum ([ainexis], "horizontal extension", concept two) is an exact
reorganisation of it, and conditional rescaling keeps it exact because the
final normalisation divides out whichever (possibly stale) max was used
([wittx], section on skipping 90% of rescales).  So the oracle is the plain
definition, not a tile emulation.

Precision: bf16 inputs widen to fp64 exactly; each bf16 x bf16 product is
exact in fp64; the sums are fp64 (matrix products through BLAS).  Outputs
stay fp64 -- no bf16 rounding of O.

Rows are processed per (sequence, head) in blocks of at most ``block``
queries; a causal block only multiplies against keys up to its last row.
Each row still sees its full key set A(i): this is blocking of the matrix
product, not online softmax.
"""
from __future__ import annotations

import numpy as np

__all__ = ["bf16_bits_to_f64", "attention", "attention_f64", "attention_probs_f64"]


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns (uint16) to float64; exact."""
    b = np.asarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def _rows_by_sequence(cu: np.ndarray, rows):
    """Split a sorted set of global token indices by sequence."""
    B = len(cu) - 1
    if rows is None:
        return [np.arange(cu[b], cu[b + 1], dtype=np.int64) for b in range(B)]
    rows = np.asarray(rows, dtype=np.int64)
    if rows.size and (np.any(np.diff(rows) <= 0) or rows[0] < 0 or rows[-1] >= cu[-1]):
        raise ValueError("rows must be strictly increasing token indices in [0, T)")
    out = []
    for b in range(B):
        lo, hi = np.searchsorted(rows, [cu[b], cu[b + 1]])
        out.append(rows[lo:hi])
    return out


def attention_f64(q, k, v, cu_seqlens, causal: bool, scale: float, rows=None,
                  block: int = 1024, widen=None, heads=None):
    """Exact attention on float inputs.

    q, k: [T, H, d_qk]; v: [T, H, d_v] (any float dtype, or bf16 bit patterns
    when ``widen`` converts them); cu_seqlens: [B+1] token offsets.
    rows: optional strictly increasing global token indices; only those query
    rows are computed (keys still span each row's whole sequence).
    heads: optional list of head indices to compute (default: all heads).

    Returns (O [R, nH, d_v] float64, LSE [nH, R] float64), R = len(rows) or T,
    nH = len(heads) or H, heads in the order given.
    """
    cvt = widen if widen is not None else (lambda a: np.asarray(a, dtype=np.float64))
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    T, H, d_qk = q.shape
    d_v = v.shape[2]
    head_list = list(range(H)) if heads is None else [int(x) for x in heads]
    per_seq = _rows_by_sequence(cu, rows)
    R = sum(len(r) for r in per_seq)
    O = np.empty((R, len(head_list), d_v), dtype=np.float64)
    LSE = np.empty((len(head_list), R), dtype=np.float64)
    r0 = 0
    for b, qrows in enumerate(per_seq):
        s, e = int(cu[b]), int(cu[b + 1])
        n = len(qrows)
        if n == 0:
            continue
        local = qrows - s                      # query positions within the sequence
        for hi, h in enumerate(head_list):
            kb = cvt(k[s:e, h, :])             # [L, d_qk]
            vb = cvt(v[s:e, h, :])             # [L, d_v]
            for c0 in range(0, n, block):
                c1 = min(n, c0 + block)
                pos = local[c0:c1]
                qb = cvt(q[qrows[c0:c1], h, :])            # [n_blk, d_qk]
                kmax = int(pos.max()) + 1 if causal else (e - s)
                S = scale * (qb @ kb[:kmax].T)             # [n_blk, kmax]
                if causal:
                    S[np.arange(kmax)[None, :] > pos[:, None]] = -np.inf
                m = S.max(axis=1)
                P = np.exp(S - m[:, None])
                l = P.sum(axis=1)
                O[r0 + c0:r0 + c1, hi, :] = (P @ vb[:kmax]) / l[:, None]
                LSE[hi, r0 + c0:r0 + c1] = m + np.log(l)
        r0 += n
    return O, LSE


def attention(q_bits, k_bits, v_bits, cu_seqlens, causal: bool, scale: float, rows=None,
              block: int = 1024, heads=None):
    """Exact attention on bf16 bit-pattern inputs (uint16 arrays, ``workloads`` layout)."""
    return attention_f64(q_bits, k_bits, v_bits, cu_seqlens, causal, scale, rows=rows,
                         block=block, widen=bf16_bits_to_f64, heads=heads)


def attention_probs_f64(q, k, causal: bool, scale: float):
    """Softmax probabilities P for one sequence and one head (small inputs).

    q: [L, d], k: [L, d] float arrays.  Returns P [L, L] (masked entries 0).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    L = q.shape[0]
    S = scale * (q @ k.T)
    if causal:
        S[np.arange(L)[None, :] > np.arange(L)[:, None]] = -np.inf
    m = S.max(axis=1)
    P = np.exp(S - m[:, None])
    return P / P.sum(axis=1)[:, None]
