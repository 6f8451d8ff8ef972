"""Software exp2: Cody-Waite range reduction plus a degree-3 polynomial.

TEST INFRASTRUCTURE ONLY (see the package docstring).

The method ([wittx] section on faking a hardware instruction in software;
[jsqmd] section four, item 1; [newton] core-technology section) computes
2^y without the transcendental unit:

    n = floor(y)                 integer part
    r = y - n                    fraction, in [0, 1)
    p = ((c3 r + c2) r + c1) r + c0    Horner's rule on FMA
    2^y = p * 2^n                n goes straight into the IEEE exponent

The pages say the fit is a cubic, that its fp32 relative error is far worse
than the hardware unit's yet well below bf16's own rounding error, and that
after rounding to bf16 it matches the hardware result on about 99% of
inputs; the coefficients themselves did not survive on the pages.  Reading
adopted: the relative-minimax cubic for 2^r on [0, 1] with c0 = 1 (so
integer y is exact), found here with the Remez exchange algorithm.

Functions
---------
remez_exp2_relative(degree, fix_c0)  minimax coefficients + error level
poly_relative_error(coeffs, r)       (p(r) - 2^r) / 2^r
exp2_poly_f64(y, coeffs)             the split in fp64
exp2_poly_f32(y, coeffs)             the split with each step rounded to fp32
                                     (FMA = one rounding of a*b + c)
"""
from __future__ import annotations

import numpy as np

__all__ = ["remez_exp2_relative", "poly_relative_error", "exp2_poly_f64", "exp2_poly_f32"]


def _horner(coeffs, r):
    """coeffs = (c0, c1, ..., cd); evaluates c0 + c1 r + ... + cd r^d by Horner's rule."""
    acc = np.full_like(np.asarray(r, dtype=np.float64), coeffs[-1])
    for c in coeffs[-2::-1]:
        acc = acc * r + c
    return acc


def poly_relative_error(coeffs, r):
    r = np.asarray(r, dtype=np.float64)
    return (_horner(coeffs, r) - np.exp2(r)) / np.exp2(r)


def _alternating_extrema(r, e):
    """Split the error curve into runs of constant sign; return argmax|e| of each run."""
    sgn = np.sign(e)
    # zeros join the following run
    for i in range(len(sgn) - 2, -1, -1):
        if sgn[i] == 0:
            sgn[i] = sgn[i + 1]
    cuts = np.flatnonzero(np.diff(sgn) != 0) + 1
    runs = np.split(np.arange(len(r)), cuts)
    return [run[np.argmax(np.abs(e[run]))] for run in runs if len(run)]


def remez_exp2_relative(degree: int = 3, fix_c0: bool = True, iters: int = 60,
                        grid: int = 200001):
    """Relative-minimax polynomial for 2^r on [0, 1] by the Remez exchange.

    Solves for coefficients and the level E such that the relative error
    takes the values +-E with alternating signs at the reference points,
    then moves the references to the extrema of the new error curve, until
    the level stops changing.  With ``fix_c0`` the constant term is 1 and
    the error vanishes at r = 0, so the references lie in (0, 1].

    Returns (coeffs (c0..c_degree), E = max |relative error| on the grid).
    """
    n_free = degree if fix_c0 else degree + 1
    n_ref = n_free + 1
    lo = 0.0
    k = np.arange(n_ref)
    refs = 0.5 - 0.5 * np.cos(np.pi * (k + (1 if fix_c0 else 0)) / (n_ref - (0 if fix_c0 else 1)))
    rg = np.linspace(lo, 1.0, grid)
    coeffs = None
    level = None
    for _ in range(iters):
        A = np.zeros((n_ref, n_ref))
        rhs = np.zeros(n_ref)
        for i, x in enumerate(refs):
            powers = [x ** j for j in range(1 if fix_c0 else 0, degree + 1)]
            A[i, :n_free] = powers
            A[i, n_free] = -((-1) ** i) * 2.0 ** x
            rhs[i] = 2.0 ** x - (1.0 if fix_c0 else 0.0)
        sol = np.linalg.solve(A, rhs)
        coeffs = ([1.0] if fix_c0 else []) + list(sol[:n_free])
        e = poly_relative_error(coeffs, rg)
        ext = _alternating_extrema(rg[1:] if fix_c0 else rg, e[1:] if fix_c0 else e)
        base = rg[1:] if fix_c0 else rg
        cand = base[ext]
        evals = np.abs(poly_relative_error(coeffs, cand))
        if len(cand) >= n_ref:
            # keep n_ref consecutive alternating extrema containing the largest one
            best = int(np.argmax(evals))
            start = min(max(0, best - n_ref + 1), len(cand) - n_ref)
            window = max(range(max(0, best - n_ref + 1), min(best, len(cand) - n_ref) + 1),
                         key=lambda s: evals[s:s + n_ref].min(), default=start)
            refs = cand[window:window + n_ref]
        new_level = float(np.max(np.abs(e)))
        if level is not None and abs(new_level - level) < 1e-15:
            level = new_level
            break
        level = new_level
    return tuple(float(c) for c in coeffs), level


def exp2_poly_f64(y, coeffs):
    """2^y by range reduction + polynomial, all in fp64.  y = -inf gives 0."""
    y = np.asarray(y, dtype=np.float64)
    out = np.zeros_like(y)
    fin = np.isfinite(y)
    n = np.floor(y[fin])
    r = y[fin] - n
    out[fin] = np.ldexp(_horner(coeffs, r), n.astype(np.int64))
    out[np.isposinf(y)] = np.inf
    return out


def _fma32(a, b, c):
    """round_fp32(a*b + c) for fp32 inputs: a*b is exact in fp64; one final fp32 rounding
    (the fp64 sum can round first in rare cases; immaterial at the tolerances used)."""
    return (a.astype(np.float64) * b.astype(np.float64) + c.astype(np.float64)).astype(np.float32)


def exp2_poly_f32(y, coeffs, clamp: float = -127.0):
    """The split with every step in fp32, as a GPU evaluates it.

    y is clamped below at ``clamp`` (so -inf maps to a value < 2^-126 instead
    of NaN), n = floor(y) and r = y - n are exact in fp32, the cubic runs as
    three fp32 FMAs with c0 as the last addend, and the result is p * 2^n
    (an exact scaling unless it underflows).
    """
    y = np.maximum(np.asarray(y, dtype=np.float32), np.float32(clamp))
    n = np.floor(y)
    r = (y - n).astype(np.float32)
    c = [np.float32(x) for x in coeffs]
    p = np.full_like(r, c[-1])
    for cj in c[-2::-1]:
        p = _fma32(p, r, np.full_like(r, cj))
    return np.ldexp(p.astype(np.float64), n.astype(np.int64)).astype(np.float32)
