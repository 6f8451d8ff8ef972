"""Input generator checks (CPU): shapes, bf16 rounding, reproducibility, ramp strength."""
import math

import numpy as np

import workloads
from workloads import Workload, f32_to_bf16_bits, bf16_bits_to_f32, make_inputs


def test_bf16_rounding_is_round_to_nearest_even():
    x = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 1.0 + 2 ** -8 + 2 ** -20, -2.5, 0.0],
                 dtype=np.float32)
    got = bf16_bits_to_f32(f32_to_bf16_bits(x))
    want = np.array([1.0, 1.0, 1.0 + 2 ** -6, 1.0 + 2 ** -7, -2.5, 0.0], dtype=np.float32)
    assert np.array_equal(got, want)


def test_small_workload_shapes_and_seed():
    a = make_inputs(1)
    b = make_inputs("small_noncausal_b1h2n256d64")
    assert a["q"].shape == (256, 2, 64) and a["v"].shape == (256, 2, 64)
    assert np.array_equal(a["q"], b["q"]) and np.array_equal(a["v"], b["v"])
    assert a["cu_seqlens"].tolist() == [0, 256]
    assert abs(a["scale"] - 1 / 8) < 1e-15
    qf = bf16_bits_to_f32(a["q"])
    assert abs(qf.mean()) < 0.05 and abs(qf.std() - 1) < 0.05


def test_packed_lengths_are_seeded():
    rng = np.random.default_rng(0)
    lengths = rng.integers(512, 32768, size=16, endpoint=True)
    assert lengths.min() >= 512 and lengths.max() <= 32768
    assert len(lengths) == workloads.workload(5).B


def test_ramp_gives_logit_std_near_four():
    wl = Workload("ramp_small", B=3, H=2, N=4096, d_qk=128, d_v=128, causal=True,
                  varlen=True, len_lo=2048, len_hi=4096, ramp=True)
    x = make_inputs(wl, seed=3)
    q = bf16_bits_to_f32(x["q"]).astype(np.float64)
    k = bf16_bits_to_f32(x["k"]).astype(np.float64)
    cu = x["cu_seqlens"]
    rng = np.random.default_rng(0)
    vals = []
    for b in range(wl.B):
        s, e = int(cu[b]), int(cu[b + 1])
        i = rng.integers(0, e - s, 4000)
        j = (rng.random(4000) * (i + 1)).astype(np.int64)    # causal pairs j <= i
        h = rng.integers(0, wl.H, 4000)
        vals.append(np.einsum("nd,nd->n", q[s + i, h], k[s + j, h]) / math.sqrt(128))
    std = float(np.concatenate(vals).std())
    assert 3.6 < std < 4.4, std
