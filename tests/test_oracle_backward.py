"""Pins for the fp64 attention-gradient oracle (CPU only).

The gradient formulas are checked against things other than themselves:
central finite differences of the (separately pinned) forward oracle, the
identities that softmax's Jacobian forces on column sums, invariance under a
shift of every key, and a closed form at Q = 0 written as scalar loops.
``test_pins_catch_planted_mistakes`` plants plausible slips in the oracle
(a dropped row term D, a wrong sign, a missing scale, P in place of P^T) and
checks that a pin fails for each.
"""
import importlib

import numpy as np
import pytest

from oracle import attention_backward, attention_backward_f64, attention_f64

bwd_mod = importlib.import_module("oracle.attention_backward")

RNG = np.random.default_rng(4321)


def _cu(lengths):
    cu = np.zeros(len(lengths) + 1, dtype=np.int64)
    cu[1:] = np.cumsum(lengths)
    return cu


def _inputs(lengths, H, d_qk, d_v, rng=RNG, qscale=1.0):
    T = int(sum(lengths))
    q = rng.standard_normal((T, H, d_qk)) * qscale
    k = rng.standard_normal((T, H, d_qk))
    v = rng.standard_normal((T, H, d_v))
    do = rng.standard_normal((T, H, d_v))
    return q, k, v, do, _cu(lengths)


def _loss(q, k, v, do, cu, causal, scale):
    O, _ = attention_f64(q, k, v, cu, causal, scale)
    return float(np.sum(O * do))


@pytest.mark.parametrize("causal", [False, True])
def test_finite_differences(causal):
    """d(sum dO*O)/dX by central differences of the forward oracle."""
    q, k, v, do, cu = _inputs([3, 5], 2, 3, 4)
    scale = 0.7
    dQ, dK, dV, _ = attention_backward_f64(q, k, v, do, cu, causal, scale)
    h = 1e-6
    for name, X, G in (("q", q, dQ), ("k", k, dK), ("v", v, dV)):
        num = np.zeros_like(X)
        for idx in np.ndindex(X.shape):
            Xp, Xm = X.copy(), X.copy()
            Xp[idx] += h
            Xm[idx] -= h
            args = {"q": q, "k": k, "v": v}
            args[name] = Xp
            fp = _loss(args["q"], args["k"], args["v"], do, cu, causal, scale)
            args[name] = Xm
            fm = _loss(args["q"], args["k"], args["v"], do, cu, causal, scale)
            num[idx] = (fp - fm) / (2 * h)
        assert np.max(np.abs(num - G)) <= 1e-7 * max(1.0, np.max(np.abs(G))), name


@pytest.mark.parametrize("causal", [False, True])
def test_column_sum_identities(causal):
    """Rows of dS sum to zero, so sum_j dK_j = 0; rows of P sum to one, so
    sum_j dV_j = sum_i dO_i (per sequence and head)."""
    q, k, v, do, cu = _inputs([40, 17, 1], 3, 8, 6)
    dQ, dK, dV, _ = attention_backward_f64(q, k, v, do, cu, causal, 0.35)
    for b in range(len(cu) - 1):
        s, e = cu[b], cu[b + 1]
        assert np.max(np.abs(dK[s:e].sum(axis=0))) <= 1e-12 * (e - s) * 10
        assert np.max(np.abs(dV[s:e].sum(axis=0) - do[s:e].sum(axis=0))) <= 1e-11


@pytest.mark.parametrize("causal", [False, True])
def test_key_shift_leaves_gradients_unchanged(causal):
    """k_j -> k_j + w moves every logit of row i by scale q_i.w, which softmax
    ignores; dQ gains scale w sum_j dS_ij = 0."""
    q, k, v, do, cu = _inputs([23, 9], 2, 5, 4)
    w = RNG.standard_normal(5)
    a = attention_backward_f64(q, k, v, do, cu, causal, 0.5)
    b = attention_backward_f64(q, k + w[None, None, :], v, do, cu, causal, 0.5)
    for x, y in zip(a, b):
        assert np.max(np.abs(x - y)) <= 1e-10


@pytest.mark.parametrize("causal", [False, True])
def test_zero_queries_closed_form(causal):
    """Q = 0: P is uniform over each row's visible keys.  Scalar loops:
    dV_j = sum_{i sees j} dO_i / n_i; dK = 0; dQ_i = scale/n_i sum_j (dO_i.v_j - D_i) k_j
    with D_i the mean of dO_i.v_j over the visible keys."""
    L, H, d, dv = 7, 1, 3, 2
    q = np.zeros((L, H, d))
    k = RNG.standard_normal((L, H, d))
    v = RNG.standard_normal((L, H, dv))
    do = RNG.standard_normal((L, H, dv))
    scale = 0.9
    dQ, dK, dV, D = attention_backward_f64(q, k, v, do, _cu([L]), causal, scale)
    for i in range(L):
        vis = list(range(i + 1)) if causal else list(range(L))
        n = len(vis)
        dots = [sum(do[i, 0, c] * v[j, 0, c] for c in range(dv)) for j in vis]
        Di = sum(dots) / n
        assert abs(D[0, i] - Di) <= 1e-13
        for c in range(d):
            want = scale / n * sum((dots[t] - Di) * k[j, 0, c] for t, j in enumerate(vis))
            assert abs(dQ[i, 0, c] - want) <= 1e-13
    assert np.all(dK == 0.0)
    for j in range(L):
        for c in range(dv):
            want = 0.0
            for i in range(L):
                vis = range(i + 1) if causal else range(L)
                if j in vis:
                    want += do[i, 0, c] / len(vis)
            assert abs(dV[j, 0, c] - want) <= 1e-13


@pytest.mark.parametrize("causal", [False, True])
def test_row_term_is_dO_dot_O(causal):
    q, k, v, do, cu = _inputs([31, 12], 2, 8, 8)
    _, _, _, D = attention_backward_f64(q, k, v, do, cu, causal, 0.4)
    O, _ = attention_f64(q, k, v, cu, causal, 0.4)
    want = np.einsum("thc,thc->ht", do, O)
    assert np.max(np.abs(D - want)) <= 1e-12


def test_single_key_gradients():
    """L = 1: O = v, so dV = dO, and the logit is irrelevant: dQ = dK = 0."""
    q, k, v, do, cu = _inputs([1], 2, 4, 3)
    dQ, dK, dV, D = attention_backward_f64(q, k, v, do, cu, False, 1.3)
    assert np.array_equal(dV, do)
    assert np.max(np.abs(dQ)) <= 1e-15 and np.max(np.abs(dK)) <= 1e-15


def test_bf16_entry_point_matches_float_entry_point():
    rng = np.random.default_rng(7)
    T, H, d = 20, 2, 8
    bits = [(rng.integers(0x3C00, 0x4000, size=(T, H, d)) | (rng.integers(0, 2, size=(T, H, d)) << 15)).astype(np.uint16)
            for _ in range(4)]
    widen = lambda b: (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    a = attention_backward(*bits, _cu([T]), True, 0.3)
    b = attention_backward_f64(*[widen(x) for x in bits], _cu([T]), True, 0.3)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)


PLANTS = {
    "no_row_term": ("dS = P * (dP - Di[:, None])", "dS = P * dP"),
    "sign": ("dS = P * (dP - Di[:, None])", "dS = P * (Di[:, None] - dP)"),
    "no_scale": ("dQ[s:e, hi, :] = scale * (dS @ kb)", "dQ[s:e, hi, :] = (dS @ kb)"),
    "p_not_transposed": ("dV[s:e, hi, :] = P.T @ dob", "dV[s:e, hi, :] = P @ dob"),
    "dk_uses_k": ("dK[s:e, hi, :] = scale * (dS.T @ qb)", "dK[s:e, hi, :] = scale * (dS.T @ kb)"),
}


_ORIG = attention_backward_f64


@pytest.mark.parametrize("plant", sorted(PLANTS))
def test_pins_catch_planted_mistakes(plant):
    import inspect
    src = inspect.getsource(bwd_mod)
    old, new = PLANTS[plant]
    assert old in src
    ns = dict(bwd_mod.__dict__)
    ns["__name__"] = "planted"
    exec(compile(src.replace(old, new), "planted", "exec"), ns)
    failed = 0
    globals()["attention_backward_f64"] = ns["attention_backward_f64"]
    try:
        for test in (lambda: test_finite_differences(True),
                     lambda: test_column_sum_identities(False),
                     lambda: test_zero_queries_closed_form(True)):
            try:
                test()
            except AssertionError:
                failed += 1
    finally:
        globals()["attention_backward_f64"] = _ORIG
    assert failed >= 1, plant
