"""Per-element error bound of the GPU backward pass (attn_bwd), derived from
its arithmetic, for the parity tests.

What the kernels compute, per (sequence, head), with u = 2^-8 (bf16 unit
roundoff, round to nearest even) and uf = 2^-24 (fp32):

  s_ij  = q_i . k_j                 fp32 sum of exact bf16 x bf16 products
  P~_ij = exp2(c s_ij - lse_i log2 e)   fp32, from the forward's fp32 lse;
          the dK/dV kernel rounds it to bf16 (dV's operand, and the factor of
          its dS), the dQ kernel keeps it in fp32
  D~_i  = dO_i . o_i                fp32, from the forward's bf16 output o
  dP~_ij = dO_i . v_j               fp32
  dS~_ij = bf16(P~_ij (dP~_ij - D~_i))
  dQ_i  = bf16(scale sum_j dS~_ij k_j),  dK_j = bf16(scale sum_i dS~_ij q_i),
  dV_j  = bf16(sum_i bf16(P~_ij) dO_i)   fp32 accumulation over n terms

Against the exact gradient (P, dP, D, dS from exact O and LSE; the oracle):

  P~ = P e^eps with |eps| <= eP_ij = |lse_i - LSE_i|
                                     + (d_qk + 2) uf |scale| sum_c |q_ic k_jc|
                                     + 2 uf |LSE_i| + 2^-21
        (the forward's lse error; the fp32 score sum and its fused scaling;
        the fp32 log2 conversion; v_exp_f32 within 2 ulp), so the relative
        error of P, after an optional bf16 rounding, is at most
        eP' = (1 + u) e^eP - 1;
  |D~ - D|   <= dD_i  = sum_c |dO_ic| |o_ic - O_ic| + (d_v + 2) uf sum_c |dO_ic o_ic|;
  |dP~ - dP| <= ddP_ij = (d_v + 2) uf sum_c |dO_ic v_jc|;
  |dS~ - dS| <= EdS = E1 + u (|dS| + E1),
        E1 = P [eP' |dP - D| + (1 + eP') (ddP + dD)] (1 + 2 uf) + 2 uf P |dP - D|;
  |dQ~ - dQ|_ic <= B + u (|dQ_ic| + B),
        B = |scale| (1 + uf) sum_j [EdS_ij + g_n (|dS_ij| + EdS_ij)] |k_jc|,
        g_n = (n + 2) uf for the n keys of the sequence (fp32 accumulation);
  dK likewise with q_i in place of k_j, summed over i;
  |dV~ - dV|_jc <= B' + u (|dV_jc| + B'),
        B' = sum_i P_ij [eP'_ij + g_n (1 + eP'_ij)] |dO_ic|.

Underflow: fp32 (and bf16, with the same exponent range) hold nothing below
2^-126 once denormals are flushed, which the hardware may do for exp2, the
conversions and the matrix operands; every P, dS and output element therefore
carries an absolute error of up to tiny = 2^-125 besides the relative ones
above (P~ within P eP' + tiny, dS~ within EdS + tiny (1 + |dP - D| + ddP + dD),
each output within its bound + tiny).  This matters only where the reference
itself is below about 1e-36, e.g. keys that no query weights above 2^-126.

The bound is first order in u with the second-order terms covered by the
(1 + ...) factors.  It is a worst case (every rounding error of a sum taken
with the same sign), so on random inputs the errors sit well below it, but it
holds element by element, small gradient entries included; a wrong mask,
scale, sign, transpose or dropped term breaks it by orders of magnitude.
"""
from __future__ import annotations

import numpy as np

U = 2.0 ** -8
UF = 2.0 ** -24
TINY = 2.0 ** -125          # flushed denormals: absolute error of one P, dS or output element


def bf16_f64(bits):
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def grad_bounds(q, k, v, dout, o_gpu, lse_gpu, O_ref, LSE_ref, dQ_ref, dK_ref, dV_ref, cu_seqlens, causal,
                scale, heads=None):
    """Element-wise bounds (bQ, bK, bV) on |GPU gradient - exact gradient].

    q, k, v, dout: bf16 bit patterns [T, H, d]; o_gpu: the forward output the
    backward was given, float64 [T, nH, d_v]; lse_gpu: float64 [nH, T];
    O_ref, LSE_ref: exact forward outputs [T, nH, d_v], [nH, T]; dQ_ref, dK_ref,
    dV_ref: exact gradients [T, nH, d]; heads: the nH head indices of the
    reference arrays (default all)."""
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    T, H, d_qk = q.shape
    d_v = v.shape[2]
    heads = list(range(H)) if heads is None else [int(h) for h in heads]
    bQ = np.zeros_like(dQ_ref)
    bK = np.zeros_like(dK_ref)
    bV = np.zeros_like(dV_ref)
    a = abs(scale)
    for b in range(len(cu) - 1):
        s, e = int(cu[b]), int(cu[b + 1])
        n = e - s
        if n == 0:
            continue
        gn = (n + 2) * UF
        for hi, h in enumerate(heads):
            Q, K, V, dO = (bf16_f64(x[s:e, h]) for x in (q, k, v, dout))
            o = o_gpu[s:e, hi]
            lse, LSE = lse_gpu[hi, s:e], LSE_ref[hi, s:e]
            D = np.einsum("ic,ic->i", dO, O_ref[s:e, hi])
            P = scale * (Q @ K.T) - LSE[:, None]
            if causal:
                P[np.triu_indices(n, 1)] = -np.inf
            np.exp(P, out=P)
            eP = np.abs(Q) @ np.abs(K).T
            eP *= (d_qk + 2) * UF * a
            eP += (np.abs(lse - LSE) + 2 * UF * np.abs(LSE) + 2.0 ** -21)[:, None]
            np.exp(eP, out=eP)
            eP *= 1.0 + U
            eP -= 1.0                                             # eP' (relative error of P~)
            dD = (np.abs(dO) * np.abs(o - O_ref[s:e, hi])).sum(axis=1) + (d_v + 2) * UF * np.abs(dO * o).sum(axis=1)
            dd = np.abs(dO) @ np.abs(V).T
            dd *= (d_v + 2) * UF
            dd += dD[:, None]                                    # |dP~ - dP| + |D~ - D|
            dPD = dO @ V.T
            dPD -= D[:, None]                                    # dP - D
            np.abs(dPD, out=dPD)                                 # |dP - D|
            dS_abs = P * dPD                                     # |dS|
            # underflow of P~ (times its factor) and of dS~ itself
            under = TINY * (1.0 + (dPD + dd) * (1.0 + eP))
            # E1 = P [eP' |dP - D| + (1 + eP')(ddP + dD)](1 + 2uf) + 2uf P |dP - D|
            E = eP * dS_abs
            dd *= P
            dd *= 1.0 + eP
            E += dd
            E *= 1.0 + 2 * UF
            E += 2 * UF * dS_abs
            E += U * (dS_abs + E)                                # EdS
            E += under
            W = E + gn * (dS_abs + E)
            BQ = a * (1 + UF) * (W @ np.abs(K))
            BK = a * (1 + UF) * (W.T @ np.abs(Q))
            del W, E, dd, dS_abs, dPD, under
            Wv = P * (eP + gn * (1.0 + eP)) + TINY
            BV = Wv.T @ np.abs(dO)
            del Wv, P, eP
            bQ[s:e, hi] = BQ + U * (np.abs(dQ_ref[s:e, hi]) + BQ) + TINY
            bK[s:e, hi] = BK + U * (np.abs(dK_ref[s:e, hi]) + BK) + TINY
            bV[s:e, hi] = BV + U * (np.abs(dV_ref[s:e, hi]) + BV) + TINY
    return bQ, bK, bV


def check_within(name, got, ref, bound, say=print):
    """Assert |got - ref| <= bound element by element (and finite); report the
    largest error-to-bound ratio and the relative RMS error."""
    assert np.isfinite(got).all(), f"{name}: non-finite gradient"
    err = np.abs(got - ref)
    ratio = float((err / np.maximum(bound, 1e-300)).max()) if err.size else 0.0
    nref = float(np.linalg.norm(ref))
    rel = float(np.linalg.norm(got - ref)) / max(nref, 1e-30)
    say(f"  {name}: max err/bound {ratio:.3f}  rel_rms {rel:.3e}  max_abs {float(err.max()) if err.size else 0.0:.3e}")
    bad = err > bound
    if bad.any():
        i = np.unravel_index(int(np.argmax(err - bound)), err.shape)
        raise AssertionError(f"{name}: {int(bad.sum())} elements outside the bound, e.g. at {i}: "
                             f"|err| {err[i]:.3e} > bound {bound[i]:.3e} (ref {ref[i]:.3e})")
    return ratio, rel
