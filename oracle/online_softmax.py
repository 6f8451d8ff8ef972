"""Tile-by-tile online softmax with conditional rescaling, in fp64.

TEST INFRASTRUCTURE ONLY (see the package docstring).

This follows the steps of the method rather than the plain definition, so
that two things can be pinned on the CPU:

* conditional rescaling is exact: whatever threshold is used, the result
  equals plain softmax attention (``attention.attention_f64``) up to fp64
  rounding, because the final division by l removes the stale max;
* how many rescales a threshold skips on a given input, which the GPU's
  optional statistics counters are compared against.

Steps, per query row, over key tiles of ``tile`` keys in order
([ainexis] "horizontal extension", concept two: keep a running max and a
running sum and correct the earlier accumulation when a new block raises the
max; [wittx] section on skipping 90% of rescales: only rescale when the new
block's row max exceeds the old one by more than a threshold, the threshold
8.0 standing for a factor of 256, i.e. it is measured in log2 units; the
final normalisation then fixes the result exactly):

    x      = c * s_ij over the tile's visible keys, c = scale * log2(e)
    m_t    = max x over the tile
    if the row has no max yet, or m_t - m > tau:      (rescale taken)
        alpha = 2^(m - m_t); O <- alpha O; l <- alpha l; m <- m_t
    P      = 2^(x - m)        (at most 2^tau when the max is stale)
    l     += sum P;  O += P v
    end:   O / l,  LSE = (m + log2 l) * ln 2

``tau < 0`` selects the unconditional rule: m <- max(m, m_t) and the
rescale is applied on every tile.
"""
from __future__ import annotations

import math

import numpy as np

__all__ = ["online_softmax_attention_f64"]

LOG2E = 1.0 / math.log(2.0)


def online_softmax_attention_f64(q, k, v, cu_seqlens, causal: bool, scale: float,
                                 tau: float = 8.0, tile: int = 64):
    """Online-softmax attention over float inputs [T, H, d] (fp64 arithmetic).

    Returns (O [T, H, d_v], LSE [H, T], stats) where stats counts
    ``considered`` (row-tile pairs after a row's first visible tile) and
    ``taken`` (those pairs whose rescale was applied).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    T, H, _ = q.shape
    d_v = v.shape[2]
    c = scale * LOG2E
    O_out = np.zeros((T, H, d_v))
    LSE = np.zeros((H, T))
    considered = 0
    taken = 0
    for b in range(len(cu) - 1):
        s0, e0 = int(cu[b]), int(cu[b + 1])
        L = e0 - s0
        if L == 0:
            continue
        pos = np.arange(L)
        for h in range(H):
            qb, kb, vb = q[s0:e0, h], k[s0:e0, h], v[s0:e0, h]
            m = np.full(L, -np.inf)
            l = np.zeros(L)
            acc = np.zeros((L, d_v))
            for k0 in range(0, L, tile):
                k1 = min(L, k0 + tile)
                x = c * (qb @ kb[k0:k1].T)                       # [L, n_t]
                if causal:
                    x[np.arange(k0, k1)[None, :] > pos[:, None]] = -np.inf
                visible = np.isfinite(x).any(axis=1)
                m_t = x.max(axis=1)
                fresh = ~np.isfinite(m)
                if tau < 0:
                    m_new = np.where(visible, np.maximum(m, m_t), m)
                    do = visible
                else:
                    do = visible & (fresh | (m_t - m > tau))
                    m_new = np.where(do, m_t, m)
                considered += int(np.count_nonzero(visible & ~fresh))
                taken += int(np.count_nonzero(do & ~fresh))
                alpha = np.where(do & ~fresh, np.exp2(np.where(do & ~fresh, m - m_new, 0.0)), 1.0)
                alpha = np.where(fresh & do, 0.0, alpha)
                acc *= alpha[:, None]
                l *= alpha
                m = m_new
                P = np.where(visible[:, None], np.exp2(x - np.where(np.isfinite(m), m, 0.0)[:, None]), 0.0)
                l += P.sum(axis=1)
                acc += P @ vb[k0:k1]
            O_out[s0:e0, h] = acc / l[:, None]
            LSE[h, s0:e0] = (m + np.log2(l)) / LOG2E
    return O_out, LSE, {"considered": considered, "taken": taken}
