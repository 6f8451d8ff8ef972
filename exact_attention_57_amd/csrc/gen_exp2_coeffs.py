"""Derive the cubic used by the kernels' software exp2 (build-support script).

The kernels compute 2^y = 2^n * p(r) with n = floor(y), r = y - n in [0, 1)
and p a cubic with p(0) = 1.  The coefficients minimise the maximum relative
error |p(r)/2^r - 1| over [0, 1].  This script finds them as a linear
program on a dense grid (variables c1, c2, c3, t; minimise t subject to
-t <= (1 + c1 r + c2 r^2 + c3 r^3 - 2^r) / 2^r <= t), then rounds them to
fp32 and prints them as hexadecimal float literals for attn_fwd_kernel.hip.

Run:  python exact_attention_57_amd/csrc/gen_exp2_coeffs.py
"""
import numpy as np
from scipy.optimize import linprog


def fit(grid: int = 20001):
    r = np.linspace(0.0, 1.0, grid)
    w = np.exp2(-r)                       # 1 / 2^r
    basis = np.stack([r * w, r * r * w, r ** 3 * w], axis=1)
    const = w - 1.0                       # (1 - 2^r) / 2^r
    ones = np.ones((grid, 1))
    # basis.c + const <= t   and   -(basis.c + const) <= t
    A = np.vstack([np.hstack([basis, -ones]), np.hstack([-basis, -ones])])
    b = np.concatenate([-const, const])
    res = linprog(c=[0, 0, 0, 1], A_ub=A, b_ub=b, bounds=[(None, None)] * 4, method="highs")
    assert res.success, res.message
    return res.x[:3], res.x[3]


if __name__ == "__main__":
    c, t = fit()
    c32 = np.asarray(c, dtype=np.float32)
    r = np.linspace(0, 1, 1_000_001)
    p = 1.0 + r * (c32[0] + r * (c32[1] + r * c32[2]))
    err = np.max(np.abs(p / np.exp2(r) - 1))
    print(f"// max relative error (fp64 eval of fp32 coefficients): {err:.4e}; LP level {t:.4e}")
    for i, v in enumerate(c32, start=1):
        print(f"constexpr float kExp2C{i} = {float(v).hex()}f;  // {float(v):.9g}")
