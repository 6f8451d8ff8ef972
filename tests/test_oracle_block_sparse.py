"""Pins for the fp64 block-sparse attention oracle (CPU only).

Checked against: the dense oracle (all-ones mask; a block-lower-triangular
mask under the causal flag), dense attention on separate sequences (a
block-diagonal mask), explicit scalar loops over each row's visible keys
(an asymmetric mask), and the empty-row convention.  Planted mistakes (a
transposed mask, a wrong block size, masked keys left in the normaliser)
each fail a pin.
"""
import importlib
import math

import numpy as np
import pytest

from oracle import attention_f64, block_sparse_attention, block_sparse_attention_f64

bs_mod = importlib.import_module("oracle.block_sparse")
RNG = np.random.default_rng(2024)
B128 = 128


def _cu(lengths):
    cu = np.zeros(len(lengths) + 1, dtype=np.int64)
    cu[1:] = np.cumsum(lengths)
    return cu


def _qkv(T, H, d, dv, rng=RNG):
    return rng.standard_normal((T, H, d)), rng.standard_normal((T, H, d)), rng.standard_normal((T, H, dv))


def _nb(n):
    return (n + B128 - 1) // B128


@pytest.mark.parametrize("causal", [False, True])
def test_all_ones_mask_is_dense(causal):
    lengths = [300, 129, 1]
    q, k, v = _qkv(sum(lengths), 2, 8, 6)
    nb = _nb(max(lengths))
    mask = np.ones((len(lengths), 2, nb, nb), dtype=np.uint8)
    O, L = block_sparse_attention_f64(q, k, v, _cu(lengths), causal, 0.3, mask)
    Od, Ld = attention_f64(q, k, v, _cu(lengths), causal, 0.3)
    assert np.max(np.abs(O - Od)) <= 1e-12 and np.max(np.abs(L - Ld)) <= 1e-12


def test_block_lower_triangle_with_causal_is_causal():
    L = 400
    q, k, v = _qkv(L, 1, 8, 4)
    nb = _nb(L)
    mask = np.tril(np.ones((nb, nb), dtype=np.uint8))[None, None]
    O, Ls = block_sparse_attention_f64(q, k, v, _cu([L]), True, 0.25, mask)
    Od, Ld = attention_f64(q, k, v, _cu([L]), True, 0.25)
    assert np.max(np.abs(O - Od)) <= 1e-12 and np.max(np.abs(Ls - Ld)) <= 1e-12


@pytest.mark.parametrize("causal", [False, True])
def test_block_diagonal_is_separate_sequences(causal):
    L = 350                                      # blocks of 128, 128, 94
    q, k, v = _qkv(L, 2, 8, 4)
    nb = _nb(L)
    mask = np.eye(nb, dtype=np.uint8)[None, None].repeat(2, axis=1)
    O, Ls = block_sparse_attention_f64(q, k, v, _cu([L]), causal, 0.4, mask)
    Od, Ld = attention_f64(q, k, v, _cu([128, 128, 94]), causal, 0.4)
    assert np.max(np.abs(O - Od)) <= 1e-12 and np.max(np.abs(Ls - Ld)) <= 1e-12


def _loops(q, k, v, L, causal, scale, m):
    """Scalar loops over each row's visible keys (one sequence, one head)."""
    d, dv = q.shape[1], v.shape[1]
    O = np.zeros((L, dv))
    LSE = np.full(L, -math.inf)
    for i in range(L):
        keys = [j for j in range(L) if m[i // B128][j // B128] and (not causal or j <= i)]
        if not keys:
            continue
        s = [scale * sum(q[i, c] * k[j, c] for c in range(d)) for j in keys]
        mx = max(s)
        w = [math.exp(x - mx) for x in s]
        tot = sum(w)
        for c in range(dv):
            O[i, c] = sum(wj * v[j, c] for wj, j in zip(w, keys)) / tot
        LSE[i] = mx + math.log(tot)
    return O, LSE


@pytest.mark.parametrize("causal", [False, True])
def test_scalar_loops_asymmetric_mask(causal):
    L = 300                                      # blocks 0, 1, 2 (2 is partial)
    q, k, v = _qkv(L, 1, 3, 2)
    m = np.array([[1, 0, 1], [1, 1, 0], [0, 1, 1]], dtype=np.uint8)
    O, Ls = block_sparse_attention_f64(q, k, v, _cu([L]), causal, 0.6, m[None, None])
    Or, Lr = _loops(q[:, 0], k[:, 0], v[:, 0], L, causal, 0.6, m)
    assert np.max(np.abs(O[:, 0] - Or)) <= 1e-12
    assert np.max(np.abs(Ls[0] - Lr)) <= 1e-12


def test_empty_rows_give_zero_and_minus_inf():
    L = 260
    q, k, v = _qkv(L, 1, 4, 3)
    m = np.array([[1, 1, 0], [0, 0, 0], [0, 0, 1]], dtype=np.uint8)[None, None]
    O, Ls = block_sparse_attention_f64(q, k, v, _cu([L]), False, 0.5, m)
    assert np.all(O[128:256] == 0.0) and np.all(np.isneginf(Ls[0, 128:256]))
    assert np.all(np.isfinite(Ls[0, :128])) and np.all(np.isfinite(Ls[0, 256:]))
    # causal: block row 2 only sees keys >= 256, so rows 256.. see themselves
    O, Ls = block_sparse_attention_f64(q, k, v, _cu([L]), True, 0.5, m)
    assert np.all(np.isfinite(Ls[0, 256:]))


def test_bf16_entry_point_matches_float_entry_point():
    rng = np.random.default_rng(5)
    T, H, d = 140, 1, 8
    bits = [(rng.integers(0x3C00, 0x4000, size=(T, H, d)) | (rng.integers(0, 2, size=(T, H, d)) << 15)).astype(np.uint16)
            for _ in range(3)]
    widen = lambda b: (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    m = np.array([[1, 0], [1, 1]], dtype=np.uint8)[None, None]
    a = block_sparse_attention(*bits, _cu([T]), True, 0.3, m)
    b = block_sparse_attention_f64(*[widen(x) for x in bits], _cu([T]), True, 0.3, m)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)


PLANTS = {
    "transposed_mask": ("vis = mask[b, h][np.ix_(blk, blk)] != 0", "vis = mask[b, h][np.ix_(blk, blk)].T != 0"),
    "block_64": ("blk = np.arange(L) // BLOCK", "blk = np.arange(L) // 64"),
    "hidden_keys_normalised": ("S[~vis] = -np.inf", "S[~vis] = S[~vis] - 0.0"),
}
_ORIG = block_sparse_attention_f64


@pytest.mark.parametrize("plant", sorted(PLANTS))
def test_pins_catch_planted_mistakes(plant):
    import inspect
    src = inspect.getsource(bs_mod)
    old, new = PLANTS[plant]
    assert old in src
    ns = dict(bs_mod.__dict__)
    ns["__name__"] = "planted"
    exec(compile(src.replace(old, new), "planted", "exec"), ns)
    failed = 0
    globals()["block_sparse_attention_f64"] = ns["block_sparse_attention_f64"]
    try:
        for test in (lambda: test_scalar_loops_asymmetric_mask(False),
                     lambda: test_block_diagonal_is_separate_sequences(False),
                     lambda: test_empty_rows_give_zero_and_minus_inf()):
            try:
                test()
            except (AssertionError, IndexError):     # a pin that fails or cannot even run
                failed += 1
    finally:
        globals()["block_sparse_attention_f64"] = _ORIG
    assert failed >= 1, plant
