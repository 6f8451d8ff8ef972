"""Pins for the FP8 (e4m3) oracle (CPU only).

The decoder is checked against values the OCP E4M3 format fixes and against
torch's independent float8_e4m3fn implementation; the attention of
dequantised inputs against closed forms and the descale algebra.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import workloads

ALL = np.arange(256, dtype=np.uint8)


def test_decode_matches_torch_on_every_code():
    ours = oracle.e4m3_to_f64(ALL)
    ref = torch.from_numpy(ALL.copy()).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    fin = ~np.isnan(ref)
    assert np.array_equal(ours[fin], ref[fin])


def test_decode_format_values():
    d = oracle.e4m3_to_f64
    assert d([0x00])[0] == 0.0 and math.copysign(1.0, d([0x80])[0]) == -1.0
    assert d([0x38])[0] == 1.0                       # exponent field 7 = bias
    assert d([0x7E])[0] == 448.0                     # largest finite: 1.75 * 2^8
    assert d([0x01])[0] == 2.0 ** -9                 # smallest subnormal
    assert d([0x07])[0] == 7 / 8 * 2.0 ** -6         # largest subnormal
    assert d([0x08])[0] == 2.0 ** -6                 # smallest normal
    assert np.isnan(d([0x7F])[0]) and np.isnan(d([0xFF])[0])
    pos = d(ALL[:0x7F])
    assert np.all(np.diff(pos) > 0)                  # monotone, all distinct
    assert np.array_equal(d(ALL[0x80:0xFF]), -pos)   # sign symmetry


def test_wrong_exponent_bias_fails_the_pins():
    """A decoder with bias 8 (the other common FP8 variant) is caught."""
    c = ALL[:0x7F].astype(np.int64)
    e, m = (c >> 3) & 0xF, (c & 7) / 8.0
    wrong = np.where(e == 0, m * 2.0 ** -7, (1 + m) * np.exp2(e - 8.0))
    assert wrong[0x38] != 1.0 and not np.array_equal(wrong, oracle.e4m3_to_f64(ALL[:0x7F]))


def test_input_codes_round_to_nearest_even():
    """The workload encoder picks the nearest e4m3 value (ties to even code)."""
    vals = oracle.e4m3_to_f64(ALL[:0x7F])
    x = np.random.default_rng(3).uniform(-500, 500, 4000).astype(np.float32)
    x = np.concatenate([x, (vals[:-1] + vals[1:]) / 2]).astype(np.float32)   # exact ties
    codes = workloads.f32_to_e4m3_codes(x)
    got = oracle.e4m3_to_f64(codes)
    ax = np.minimum(np.abs(x.astype(np.float64)), 448.0)
    best = np.abs(vals[None, :] - ax[:, None]).min(axis=1)
    assert np.array_equal(np.abs(np.abs(got) - ax), best)
    ties = (codes[4000:] & 0x7F)
    assert np.all(ties % 2 == 0)


def _inputs(lengths, H=2, d=128, seed=0, prescale=(1.0, 1.0, 1.0)):
    inp = workloads.make_custom_inputs(lengths, H, d, d, seed=seed)
    return workloads.make_fp8_inputs(inp, prescale)


@pytest.mark.parametrize("causal", [False, True])
def test_zero_queries_closed_form(causal):
    f = _inputs([9, 17], prescale=(1.0, 1.0, 2.0))
    q8 = np.zeros_like(f["q8"])
    O, L = oracle.attention_fp8(q8, f["k8"], f["v8"], f["cu_seqlens"], causal, 0.3,
                                1.0, 1.0, f["v_descale"])
    v = oracle.e4m3_to_f64(f["v8"]) * f["v_descale"]
    cu = f["cu_seqlens"]
    for b in range(2):
        s, e = cu[b], cu[b + 1]
        for i in range(e - s):
            n = i + 1 if causal else e - s
            assert np.allclose(O[s + i], v[s:s + n].mean(axis=0), rtol=0, atol=1e-14)
            assert np.allclose(L[:, s + i], math.log(n), rtol=0, atol=1e-14)


def test_descale_algebra():
    f = _inputs([33, 70], seed=2, prescale=(8.0, 4.0, 16.0))
    cu, args = f["cu_seqlens"], (f["q8"], f["k8"], f["v8"])
    O1, L1 = oracle.attention_fp8(*args, cu, True, 0.1, f["q_descale"], f["k_descale"], f["v_descale"])
    # a factor moved between q_descale, k_descale and scale changes nothing
    O2, L2 = oracle.attention_fp8(*args, cu, True, 0.2, f["q_descale"] / 4, f["k_descale"] * 2, f["v_descale"])
    assert np.allclose(O1, O2, rtol=0, atol=1e-13) and np.allclose(L1, L2, rtol=0, atol=1e-13)
    # v_descale scales O linearly and leaves LSE alone
    O3, L3 = oracle.attention_fp8(*args, cu, True, 0.1, f["q_descale"], f["k_descale"], 3 * f["v_descale"])
    assert np.allclose(O3, 3 * O1, rtol=1e-13, atol=1e-13) and np.array_equal(L3, L1)


def test_single_key_returns_dequantised_v():
    f = _inputs([1, 4], seed=5, prescale=(2.0, 2.0, 2.0))
    O, L = oracle.attention_fp8(f["q8"], f["k8"], f["v8"], f["cu_seqlens"], True, 0.125,
                                f["q_descale"], f["k_descale"], f["v_descale"])
    q = oracle.e4m3_to_f64(f["q8"]) * f["q_descale"]
    k = oracle.e4m3_to_f64(f["k8"]) * f["k_descale"]
    v = oracle.e4m3_to_f64(f["v8"]) * f["v_descale"]
    for t in (0, 1):   # the one-token sequence and causal row 0 of the second
        assert np.array_equal(O[t], v[t])
        assert np.allclose(L[:, t], 0.125 * np.einsum("hd,hd->h", q[t], k[t]), rtol=0, atol=1e-13)


def test_rows_of_probabilities_sum_to_one_on_fp8_inputs():
    f = _inputs([40], H=1, seed=7)
    q = oracle.e4m3_to_f64(f["q8"][:, 0])
    k = oracle.e4m3_to_f64(f["k8"][:, 0])
    P = oracle.attention_probs_f64(q, k, True, 0.09)
    assert np.allclose(P.sum(axis=1), 1.0, rtol=0, atol=1e-12)
    # and O is P @ v, brute force
    v = oracle.e4m3_to_f64(f["v8"][:, 0])
    O, _ = oracle.attention_fp8(f["q8"], f["k8"], f["v8"], f["cu_seqlens"], True, 0.09)
    assert np.allclose(O[:, 0], P @ v, rtol=0, atol=1e-12)
