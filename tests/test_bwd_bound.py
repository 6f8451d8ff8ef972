"""CPU checks of the backward parity bound (``_bwd_bound.grad_bounds``).

The GPU tests accept a gradient element only within a bound derived from the
kernels' arithmetic.  Here the derivation itself is tested: an emulation of
the kernels' rounding steps in numpy (fp32 products and sums, bf16 rounding
of the forward output, of P and of dS, fp32 exp2) must land inside the bound
on every element, and each plausible mistake in the gradient (a dropped row
term D, a flipped sign, a missing scale, Q and K swapped in dK, P used for
its transpose) must land outside it somewhere.  The emulation is test
scaffolding for the bound, not a second oracle: the reference values are the
fp64 oracle's.
"""
import numpy as np
import pytest

import oracle
import workloads
from _bwd_bound import check_within, grad_bounds

LOG2E = 1.4426950408889634


def bf16_round(x):
    return workloads.bf16_bits_to_f32(workloads.f32_to_bf16_bits(np.asarray(x, dtype=np.float32)))


def emulate(inp, dout, causal, scale, plant=None):
    """fp32 / bf16 emulation of the backward kernels' steps, per (sequence, head)."""
    q, k, v = (workloads.bf16_bits_to_f32(inp[n]) for n in ("q", "k", "v"))
    dO = workloads.bf16_bits_to_f32(dout)
    O_ref, L_ref = oracle.attention(inp["q"], inp["k"], inp["v"], inp["cu_seqlens"], causal, scale)
    o = bf16_round(O_ref)                          # the forward's bf16 output
    lse = L_ref.astype(np.float32)                 # the forward's fp32 LSE
    dq, dk, dv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    cu = inp["cu_seqlens"]
    c = np.float32(scale * LOG2E)
    for b in range(len(cu) - 1):
        s, e = int(cu[b]), int(cu[b + 1])
        n = e - s
        for h in range(q.shape[1]):
            Q, K, V, G = q[s:e, h], k[s:e, h], v[s:e, h], dO[s:e, h]
            S = (Q @ K.T).astype(np.float32)
            x = S * c - (lse[h, s:e] * np.float32(LOG2E))[:, None]
            if causal:
                x[np.triu_indices(n, 1)] = -np.inf
            P = np.exp2(x).astype(np.float32)
            Pb = bf16_round(P)
            D = (G * o[s:e, h]).sum(axis=1, dtype=np.float32)
            dP = (G @ V.T).astype(np.float32)
            Dm = np.zeros_like(D) if plant == "dropped D" else D
            sgn = np.float32(-1.0) if plant == "sign" else np.float32(1.0)
            dS_k = bf16_round(sgn * Pb * (dP - Dm[:, None]))
            dS_q = bf16_round(sgn * P * (dP - Dm[:, None]))
            sc = np.float32(1.0) if plant == "scale" else np.float32(scale)
            dq[s:e, h] = bf16_round(sc * (dS_q @ K))
            dk[s:e, h] = bf16_round(sc * (dS_k.T @ (K if plant == "Q for K in dK" else Q)))
            dv[s:e, h] = bf16_round((Pb if plant == "P for its transpose" else Pb.T) @ G)
    return o.astype(np.float64), lse.astype(np.float64), dq, dk, dv, O_ref, L_ref


CASES = [   # lengths, H, d_qk, d_v, causal, scale, input std
    ([1, 77, 300, 129], 2, 64, 64, True, 0.125, 1.0),
    ([200, 130], 2, 128, 128, False, -0.05, 1.0),
    ([150, 64], 2, 192, 128, True, 0.25, 2.0),
    ([200, 130], 2, 128, 128, True, 0.3, 3.0),      # logits of std ~30: P underflows fp32
]


@pytest.mark.parametrize("case", range(len(CASES)))
def test_bound_covers_emulated_rounding(case):
    lengths, H, d_qk, d_v, causal, scale, std = CASES[case]
    inp = workloads.make_custom_inputs(lengths, H, d_qk, d_v, seed=60 + case, std=std)
    dout = workloads.make_output_grad(inp, case)
    o, lse, dq, dk, dv, O_ref, L_ref = emulate(inp, dout, causal, scale)
    rq, rk, rv, _ = oracle.attention_backward(inp["q"], inp["k"], inp["v"], dout, inp["cu_seqlens"], causal, scale)
    bq, bk, bv = grad_bounds(inp["q"], inp["k"], inp["v"], dout, o, lse, O_ref, L_ref, rq, rk, rv,
                             inp["cu_seqlens"], causal, scale)
    for name, got, ref, bnd in (("dq", dq, rq, bq), ("dk", dk, rk, bk), ("dv", dv, rv, bv)):
        ratio, _ = check_within(name, got.astype(np.float64), ref, bnd)
        assert ratio > 1e-3          # the bound is not vacuous by orders of magnitude


@pytest.mark.parametrize("plant", ["dropped D", "sign", "scale", "Q for K in dK", "P for its transpose"])
def test_bound_catches_planted_mistakes(plant):
    lengths, H, d_qk, d_v, causal, scale = [64, 100], 2, 64, 64, True, 0.2
    inp = workloads.make_custom_inputs(lengths, H, d_qk, d_v, seed=70)
    dout = workloads.make_output_grad(inp, 1)
    o, lse, dq, dk, dv, O_ref, L_ref = emulate(inp, dout, causal, scale, plant=plant)
    rq, rk, rv, _ = oracle.attention_backward(inp["q"], inp["k"], inp["v"], dout, inp["cu_seqlens"], causal, scale)
    bq, bk, bv = grad_bounds(inp["q"], inp["k"], inp["v"], dout, o, lse, O_ref, L_ref, rq, rk, rv,
                             inp["cu_seqlens"], causal, scale)
    caught = False
    for name, got, ref, bnd in (("dq", dq, rq, bq), ("dk", dk, rk, bk), ("dv", dv, rv, bv)):
        try:
            check_within(name, got.astype(np.float64), ref, bnd)
        except AssertionError:
            caught = True
    assert caught, f"planted '{plant}' stayed inside the bound"
