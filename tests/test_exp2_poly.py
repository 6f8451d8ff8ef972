"""Pins for the software exp2 model (CPU) and the kernel's exp2 (GPU).

CPU pins the oracle's Remez fit and range reduction against mathematics:
Chebyshev's alternation theorem (a minimax error equioscillates), exactness
at integers when c0 = 1, a least-squares fit never beating the minimax
level, and the pages' claim that after bf16 rounding the cubic matches the
exact exponential on about 99% of inputs.  The GPU test runs the kernel's
own exp2 routines through ``attn_debug_exp2`` and checks them against exact
2^y with the same bounds.
"""
import json
import os

import numpy as np
import pytest

from oracle import exp2_poly_f32, exp2_poly_f64, poly_relative_error, remez_exp2_relative

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "pages_constants.json")))


def round_bf16_f64(x):
    """Round positive fp64 values directly to bf16 precision (8 significant bits, RNE)."""
    x = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(x)                      # x = m 2^e, m in [0.5, 1)
    return np.ldexp(np.rint(m * 256.0), e - 8)


@pytest.fixture(scope="module")
def fit():
    return remez_exp2_relative(3, fix_c0=True)


def test_fit_equioscillates(fit):
    coeffs, E = fit
    assert coeffs[0] == 1.0
    r = np.linspace(0, 1, 400001)
    e = poly_relative_error(coeffs, r)
    assert abs(e[0]) < 1e-15                       # c0 = 1: exact at r = 0
    assert np.max(np.abs(e)) <= E * (1 + 1e-9)
    # Chebyshev alternation: at least degree + 1 = 4 extrema of size E with
    # alternating signs (the endpoint r = 0 is pinned to zero by c0 = 1)
    sgn = np.sign(e[1:])
    runs = np.split(np.abs(e[1:]), np.flatnonzero(np.diff(sgn) != 0) + 1)
    peaks = [run.max() for run in runs]
    assert len(peaks) >= 4
    assert min(peaks) >= E * (1 - 1e-3)
    assert 5e-5 < E < 1e-4


def test_free_c0_fit_is_better_and_alternates_more():
    coeffs, E = remez_exp2_relative(3, fix_c0=False)
    _, E1 = remez_exp2_relative(3, fix_c0=True)
    assert E < E1
    r = np.linspace(0, 1, 400001)
    e = poly_relative_error(coeffs, r)
    sgn = np.sign(e)
    runs = np.split(np.abs(e), np.flatnonzero(np.diff(sgn) != 0) + 1)
    assert len(runs) >= 5 and min(run.max() for run in runs) >= E * (1 - 1e-3)


def test_least_squares_never_beats_minimax(fit):
    _, E = fit
    r = np.cos(np.linspace(0, np.pi, 2001)) * 0.5 + 0.5
    # weighted LS for the relative error with c0 = 1: minimise sum ((p - 2^r)/2^r)^2
    A = np.stack([r, r ** 2, r ** 3], axis=1) / np.exp2(r)[:, None]
    b = (np.exp2(r) - 1.0) / np.exp2(r)
    c = np.linalg.lstsq(A, b, rcond=None)[0]
    e_ls = poly_relative_error([1.0, *c], np.linspace(0, 1, 200001))
    assert np.max(np.abs(e_ls)) >= E * (1 - 1e-9)


def test_split_exact_at_integers(fit):
    coeffs, _ = fit
    n = np.arange(-126, 9, dtype=np.float64)
    assert np.array_equal(exp2_poly_f64(n, coeffs), np.exp2(n))
    assert np.array_equal(exp2_poly_f32(n.astype(np.float32), coeffs), np.exp2(n).astype(np.float32))
    assert exp2_poly_f64(np.array([-np.inf]), coeffs)[0] == 0.0


def test_split_relative_error_bound(fit):
    coeffs, E = fit
    y = np.random.default_rng(0).uniform(-126, 8, 1_000_000)
    rel = np.abs(exp2_poly_f64(y, coeffs) / np.exp2(y) - 1)
    assert rel.max() <= E * (1 + 1e-9)
    y32 = y.astype(np.float32)
    rel32 = np.abs(exp2_poly_f32(y32, coeffs).astype(np.float64) / np.exp2(y32.astype(np.float64)) - 1)
    assert rel32.max() <= E + 4 * 2.0 ** -24


@pytest.mark.parametrize("lo,hi", [(-16.0, 0.0), (-126.0, 8.0)])
def test_bf16_agreement_matches_pages(fit, lo, hi):
    """After bf16 rounding the cubic agrees with the exact exponential on
    about 99% of inputs (golden: pages_constants.json, poly_bf16_agreement)."""
    coeffs, _ = fit
    y = np.random.default_rng(1).uniform(lo, hi, 2_000_000)
    a = round_bf16_f64(exp2_poly_f64(y, coeffs))
    b = round_bf16_f64(np.exp2(y))
    rate = float(np.mean(a == b))
    target = GOLDEN["poly_bf16_agreement"]["value"]
    assert abs(rate - target) <= 0.005, rate


def test_planted_horner_order_mistake_is_caught(fit):
    coeffs, E = fit
    wrong = tuple(reversed(coeffs))       # Horner with the coefficient order reversed
    y = np.linspace(-4, 4, 10001)
    rel = np.abs(exp2_poly_f64(y, wrong) / np.exp2(y) - 1)
    assert rel.max() > 100 * E


def test_pages_threshold_constant():
    g = GOLDEN["rescale_threshold_log2"]
    assert 2.0 ** g["value"] == g["factor"]
    lo, hi = GOLDEN["poly_emulated_fraction"]["lo"], GOLDEN["poly_emulated_fraction"]["hi"]
    # the kernel's emulated fractions 1/8 and 1/4 fall in the pages' range
    assert lo <= 1 / 8 <= hi and lo <= 1 / 4 <= hi


# ------------------------------------------------------------------ GPU: the kernels' exp2

@pytest.mark.gpu
def test_kernel_exp2_against_exact(fit):
    """attn_debug_exp2 runs the kernels' own exp2 routines on the GPU."""
    import torch
    import exact_attention_57_amd as ea
    coeffs, E = fit
    rng = np.random.default_rng(2)
    y = np.concatenate([rng.uniform(-16, 0, 1_000_000), rng.uniform(-126, 8, 1_000_000),
                        np.arange(-126, 9), [0.0, -0.0, 1e-7, -1e-7]]).astype(np.float32)
    x = torch.from_numpy(y).cuda()
    hw = ea.debug_exp2(x, False).cpu().numpy().astype(np.float64)
    sw = ea.debug_exp2(x, True).cpu().numpy().astype(np.float64)
    exact = np.exp2(y.astype(np.float64))
    rel_hw = np.abs(hw / exact - 1)
    rel_sw = np.abs(sw / exact - 1)
    print(f"hw max rel {rel_hw.max():.3e}; sw max rel {rel_sw.max():.3e} (fit level {E:.3e})")
    assert rel_hw.max() <= 2.0 ** -21
    assert rel_sw.max() <= E + 4 * 2.0 ** -24
    ints = np.arange(-126, 9).astype(np.float32)
    sel = np.isin(y, ints) & (np.abs(y) >= 1)
    assert np.array_equal(sw[sel], exact[sel])          # exact at integers (c0 = 1)
    # agreement with the oracle's independent fit run through the same fp32 steps
    ref = exp2_poly_f32(y, coeffs).astype(np.float64)
    assert np.max(np.abs(sw / ref - 1)) <= 1e-6
    # bf16 agreement with the exact exponential (pages: about 99%)
    lo = (y >= -16) & (y <= 0)
    rate = float(np.mean(round_bf16_f64(sw[lo]) == round_bf16_f64(exact[lo])))
    print(f"bf16 agreement of the kernel's cubic with exact exp2 on [-16, 0]: {rate:.4f}")
    assert rate >= 0.985
    # masked keys: exp2(-inf) is 0 on the hardware path and below 2^-126 on the software path
    z = torch.tensor([-np.inf], dtype=torch.float32, device="cuda")
    assert ea.debug_exp2(z, False).item() == 0.0
    assert 0.0 <= ea.debug_exp2(z, True).item() < 2.0 ** -126
