"""Plain fp64 gradient of softmax attention: what the backward pass computes.

TEST INFRASTRUCTURE ONLY (see the package docstring).

What is computed
----------------
The pages describe a backward pass for the attention of ``attention.py``
([wittx], section on backward-pass optimisation; [newton], core-technology
section): it produces the gradients of the loss with respect to Q, K and V
from the output gradient dO, and its dQ is a reduction over the key/value
sequence dimension.  The pages give no formulas; the gradient itself has a
plain definition -- the derivative of

    O_i = sum_{j in A(i)} P_ij v_j,   P_ij = exp(s_ij) / sum_{j' in A(i)} exp(s_ij'),
    s_ij = scale * q_i . k_j

-- and this module writes it out by the chain rule, per (sequence, head):

    dV_j  = sum_i P_ij dO_i                        (dV = P^T dO)
    dP_ij = dO_i . v_j                             (dP = dO V^T)
    D_i   = sum_j P_ij dP_ij  = dO_i . O_i         (softmax Jacobian row term)
    dS_ij = P_ij (dP_ij - D_i)                     (d loss / d s_ij)
    dQ_i  = scale * sum_j dS_ij k_j                (dQ = scale dS K)
    dK_j  = scale * sum_i dS_ij q_i                (dK = scale dS^T Q)

with masked pairs (j not in A(i)) contributing nothing.  D is returned too:
the GPU path computes it from the forward's output as dO_i . O_i.

Precision: bf16 inputs widen to fp64 exactly; products through BLAS in
fp64; outputs stay fp64.
"""
from __future__ import annotations

import numpy as np

from .attention import bf16_bits_to_f64

__all__ = ["attention_backward_f64", "attention_backward"]


def attention_backward_f64(q, k, v, do, cu_seqlens, causal: bool, scale: float, widen=None, heads=None):
    """Gradients of exact attention.

    q, k: [T, H, d_qk]; v, do: [T, H, d_v]; cu_seqlens: [B+1] token offsets.
    heads: optional list of head indices (default all), in the order given.

    Returns (dQ [T, nH, d_qk], dK [T, nH, d_qk], dV [T, nH, d_v], D [nH, T]),
    all float64.
    """
    cvt = widen if widen is not None else (lambda a: np.asarray(a, dtype=np.float64))
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    T, H, d_qk = q.shape
    d_v = v.shape[2]
    head_list = list(range(H)) if heads is None else [int(x) for x in heads]
    nH = len(head_list)
    dQ = np.zeros((T, nH, d_qk))
    dK = np.zeros((T, nH, d_qk))
    dV = np.zeros((T, nH, d_v))
    D = np.zeros((nH, T))
    for b in range(len(cu) - 1):
        s, e = int(cu[b]), int(cu[b + 1])
        L = e - s
        if L == 0:
            continue
        for hi, h in enumerate(head_list):
            qb, kb = cvt(q[s:e, h, :]), cvt(k[s:e, h, :])
            vb, dob = cvt(v[s:e, h, :]), cvt(do[s:e, h, :])
            S = scale * (qb @ kb.T)
            if causal:
                S[np.arange(L)[None, :] > np.arange(L)[:, None]] = -np.inf
            P = np.exp(S - S.max(axis=1)[:, None])
            P /= P.sum(axis=1)[:, None]
            dP = dob @ vb.T
            Di = (P * dP).sum(axis=1)
            dS = P * (dP - Di[:, None])
            dQ[s:e, hi, :] = scale * (dS @ kb)
            dK[s:e, hi, :] = scale * (dS.T @ qb)
            dV[s:e, hi, :] = P.T @ dob
            D[hi, s:e] = Di
    return dQ, dK, dV, D


def attention_backward(q_bits, k_bits, v_bits, do_bits, cu_seqlens, causal: bool, scale: float, heads=None):
    """Gradients on bf16 bit-pattern inputs (uint16 arrays, ``workloads`` layout)."""
    return attention_backward_f64(q_bits, k_bits, v_bits, do_bits, cu_seqlens, causal, scale,
                                  widen=bf16_bits_to_f64, heads=heads)
