"""Pins for the fp64 attention oracle (CPU only).

Each test checks the oracle against something other than itself: a closed
form, an invariant of softmax attention, or an independent mpmath brute
force in scalar loops.  Together they catch the plausible mistakes (a wrong
mask direction, a dropped scale, a wrong log/exp base, a transposed operand,
a missing max in the LSE): ``test_pins_catch_planted_mistakes`` plants some
of them in the oracle and checks that a pin fails.
"""
import math

import mpmath
import numpy as np
import pytest

import oracle
import importlib
oracle_attention_mod = importlib.import_module("oracle.attention")
from oracle import attention_f64, attention_probs_f64, online_softmax_attention_f64
import workloads

RNG = np.random.default_rng(1234)


def _rand(T, H, d, scale=1.0, rng=RNG):
    return rng.standard_normal((T, H, d)) * scale


def _cu(lengths):
    cu = np.zeros(len(lengths) + 1, dtype=np.int64)
    cu[1:] = np.cumsum(lengths)
    return cu


# --------------------------------------------------------------------------- basics

def test_bf16_widening_is_exact():
    bits = np.array([0x3F80, 0xC000, 0x0001, 0x7F7F, 0x8000, 0x3E80], dtype=np.uint16)
    want = np.array([1.0, -2.0, 2.0 ** -133, (2 - 2 ** -7) * 2.0 ** 127, -0.0, 0.25])
    got = oracle.bf16_bits_to_f64(bits)
    assert np.array_equal(got, want)
    assert np.signbit(got[4])


@pytest.mark.parametrize("causal", [False, True])
def test_probability_rows_sum_to_one(causal):
    q = RNG.standard_normal((37, 16))
    k = RNG.standard_normal((37, 16))
    P = attention_probs_f64(q, k, causal, 0.3)
    assert np.all(P >= 0)
    assert np.max(np.abs(P.sum(axis=1) - 1.0)) <= 1e-12
    if causal:
        assert np.all(P[np.triu_indices(37, 1)] == 0.0)
        assert P[0, 0] == 1.0


@pytest.mark.parametrize("causal", [False, True])
def test_constant_v_gives_constant_o(causal):
    T, H = 50, 3
    q, k = _rand(T, H, 8), _rand(T, H, 8)
    vrow = RNG.standard_normal((H, 5))
    v = np.broadcast_to(vrow, (T, H, 5)).copy()
    O, _ = attention_f64(q, k, v, _cu([T]), causal, 0.7)
    assert np.max(np.abs(O - vrow[None])) <= 1e-12


def test_key_permutation_leaves_output_unchanged():
    T, H = 64, 2
    q, k, v = _rand(T, H, 16), _rand(T, H, 16), _rand(T, H, 12)
    perm = RNG.permutation(T)
    O1, L1 = attention_f64(q, k, v, _cu([T]), False, 0.25)
    O2, L2 = attention_f64(q, k[perm], v[perm], _cu([T]), False, 0.25)
    assert np.max(np.abs(O1 - O2)) <= 1e-12
    assert np.max(np.abs(L1 - L2)) <= 1e-12


def test_single_key_returns_v():
    H = 2
    q, k, v = _rand(1, H, 8), _rand(1, H, 8), _rand(1, H, 4)
    O, L = attention_f64(q, k, v, _cu([1]), False, 0.5)
    assert np.array_equal(O, v)
    s00 = 0.5 * np.einsum("thd,thd->ht", q, k)
    assert np.max(np.abs(L - s00)) <= 1e-14
    # causal row 0 of a longer sequence sees only key 0
    T = 9
    q, k, v = _rand(T, H, 8), _rand(T, H, 8), _rand(T, H, 4)
    O, L = attention_f64(q, k, v, _cu([T]), True, 0.5)
    assert np.array_equal(O[0], v[0])
    assert np.max(np.abs(L[:, 0] - 0.5 * np.sum(q[0] * k[0], axis=-1))) <= 1e-14


@pytest.mark.parametrize("causal", [False, True])
def test_zero_queries_closed_form(causal):
    """Q = 0 makes every logit 0: O_i is the mean of the visible V rows and
    LSE_i = ln(number of visible keys).  Pins the mask direction, the
    normalisation and the natural-log base of the LSE."""
    T, H = 33, 2
    q = np.zeros((T, H, 8))
    k, v = _rand(T, H, 8), _rand(T, H, 6)
    O, L = attention_f64(q, k, v, _cu([T]), causal, 1.3)
    if causal:
        csum = np.cumsum(v, axis=0)
        cnt = np.arange(1, T + 1)[:, None, None]
        assert np.max(np.abs(O - csum / cnt)) <= 1e-12
        assert np.max(np.abs(L - np.log(np.arange(1, T + 1))[None, :])) <= 1e-12
    else:
        assert np.max(np.abs(O - v.mean(axis=0, keepdims=True))) <= 1e-12
        assert np.max(np.abs(L - math.log(T))) <= 1e-12


def _brute_force_mp(q, k, v, causal, scale, digits=50):
    """Independent scalar-loop attention in mpmath (one sequence, one head)."""
    mpmath.mp.dps = digits
    L, d = q.shape
    dv = v.shape[1]
    O = np.zeros((L, dv))
    LSE = np.zeros(L)
    for i in range(L):
        keys = range(i + 1) if causal else range(L)
        s = {}
        for j in keys:
            acc = mpmath.mpf(0)
            for c in range(d):
                acc += mpmath.mpf(float(q[i, c])) * mpmath.mpf(float(k[j, c]))
            s[j] = mpmath.mpf(float(scale)) * acc
        denom = mpmath.fsum(mpmath.exp(s[j]) for j in keys)
        for c in range(dv):
            num = mpmath.fsum(mpmath.exp(s[j]) * mpmath.mpf(float(v[j, c])) for j in keys)
            O[i, c] = float(num / denom)
        LSE[i] = float(mpmath.log(denom))
    return O, LSE


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("L,d,dv", [(1, 1, 1), (3, 2, 3), (5, 4, 2), (4, 3, 4)])
def test_mpmath_brute_force(causal, L, d, dv):
    rng = np.random.default_rng(L * 100 + d * 10 + dv)
    q = rng.standard_normal((L, 1, d)) * 2
    k = rng.standard_normal((L, 1, d)) * 2
    v = rng.standard_normal((L, 1, dv))
    scale = 0.37
    O, LSE = attention_f64(q, k, v, _cu([L]), causal, scale)
    Om, Lm = _brute_force_mp(q[:, 0], k[:, 0], v[:, 0], causal, scale)
    assert np.max(np.abs(O[:, 0] - Om)) <= 1e-13
    assert np.max(np.abs(LSE[0] - Lm)) <= 1e-13


def test_causal_row_equals_noncausal_prefix():
    T, H = 40, 2
    q, k, v = _rand(T, H, 8), _rand(T, H, 8), _rand(T, H, 8)
    Oc, Lc = attention_f64(q, k, v, _cu([T]), True, 0.4)
    for i in (0, 1, 17, T - 1):
        # non-causal attention of query i over the prefix 0..i
        qq = np.concatenate([np.zeros((i, H, 8)), q[i:i + 1]], axis=0)
        On, Ln = attention_f64(qq, k[:i + 1], v[:i + 1], _cu([i + 1]), False, 0.4,
                               rows=[i])
        assert np.max(np.abs(Oc[i] - On[0])) <= 1e-12
        assert np.max(np.abs(Lc[:, i] - Ln[:, 0])) <= 1e-12
    Onc, Lnc = attention_f64(q, k, v, _cu([T]), False, 0.4)
    assert np.max(np.abs(Oc[T - 1] - Onc[T - 1])) <= 1e-12


@pytest.mark.parametrize("causal", [False, True])
def test_varlen_equals_per_sequence(causal):
    lengths = [7, 0, 19, 1, 33]
    H = 2
    T = sum(lengths)
    q, k, v = _rand(T, H, 8), _rand(T, H, 8), _rand(T, H, 4)
    cu = _cu(lengths)
    O, L = attention_f64(q, k, v, cu, causal, 0.6)
    for b, n in enumerate(lengths):
        s, e = cu[b], cu[b + 1]
        if n == 0:
            continue
        Ob, Lb = attention_f64(q[s:e], k[s:e], v[s:e], _cu([n]), causal, 0.6)
        assert np.max(np.abs(O[s:e] - Ob)) <= 1e-13
        assert np.max(np.abs(L[:, s:e] - Lb)) <= 1e-13


def test_key_shift_changes_only_lse():
    """Adding w to every key adds scale*q_i.w to every logit of row i: P and O
    are unchanged and LSE_i grows by exactly that amount."""
    T, H, d = 30, 2, 8
    q, k, v = _rand(T, H, d), _rand(T, H, d), _rand(T, H, 5)
    w = RNG.standard_normal((H, d))
    for causal in (False, True):
        O1, L1 = attention_f64(q, k, v, _cu([T]), causal, 0.45)
        O2, L2 = attention_f64(q, k + w[None], v, _cu([T]), causal, 0.45)
        shift = 0.45 * np.einsum("thd,hd->ht", q, w)
        assert np.max(np.abs(O1 - O2)) <= 1e-11
        assert np.max(np.abs(L2 - L1 - shift)) <= 1e-11


def test_row_subset_matches_full():
    lengths = [100, 37]
    H = 2
    T = sum(lengths)
    q, k, v = _rand(T, H, 8), _rand(T, H, 8), _rand(T, H, 8)
    O, L = attention_f64(q, k, v, _cu(lengths), True, 0.5)
    rows = np.array([0, 5, 99, 100, 101, 136])
    Os, Ls = attention_f64(q, k, v, _cu(lengths), True, 0.5, rows=rows, block=2)
    assert np.max(np.abs(Os - O[rows])) <= 1e-14
    assert np.max(np.abs(Ls - L[:, rows])) <= 1e-14


def test_bf16_entry_point_matches_float_entry_point():
    inp = workloads.make_inputs(1)
    O, L = oracle.attention(inp["q"], inp["k"], inp["v"], inp["cu_seqlens"], False, inp["scale"])
    qf = oracle.bf16_bits_to_f64(inp["q"])
    kf = oracle.bf16_bits_to_f64(inp["k"])
    vf = oracle.bf16_bits_to_f64(inp["v"])
    O2, L2 = attention_f64(qf, kf, vf, inp["cu_seqlens"], False, inp["scale"])
    assert np.array_equal(O, O2) and np.array_equal(L, L2)
    assert O.shape == (256, 2, 64) and L.shape == (2, 256)


# ------------------------------------------------------------- online softmax model

@pytest.mark.parametrize("tau", [-1.0, 0.0, 8.0, 200.0])
@pytest.mark.parametrize("causal", [False, True])
def test_online_softmax_exact_for_any_threshold(tau, causal):
    lengths = [150, 64, 1, 97]
    H = 2
    T = sum(lengths)
    rng = np.random.default_rng(7)
    # growing logits along the sequence so that the max moves often
    ramp = np.concatenate([np.linspace(0, 3, n) for n in lengths])[:, None, None]
    q = rng.standard_normal((T, H, 16)) + 1.0
    k = rng.standard_normal((T, H, 16)) + ramp
    v = rng.standard_normal((T, H, 8))
    O, L = attention_f64(q, k, v, _cu(lengths), causal, 0.5)
    O2, L2, st = online_softmax_attention_f64(q, k, v, _cu(lengths), causal, 0.5, tau=tau, tile=32)
    assert np.max(np.abs(O - O2)) <= 1e-12
    assert np.max(np.abs(L - L2)) <= 1e-12
    assert 0 <= st["taken"] <= st["considered"]
    if tau >= 200:
        assert st["taken"] == 0


def test_online_softmax_threshold_zero_equals_unconditional_bitwise():
    T, H = 200, 2
    rng = np.random.default_rng(3)
    q = rng.standard_normal((T, H, 16))
    k = rng.standard_normal((T, H, 16)) + np.linspace(0, 2, T)[:, None, None]
    v = rng.standard_normal((T, H, 8))
    a = online_softmax_attention_f64(q, k, v, _cu([T]), True, 0.5, tau=0.0, tile=16)
    b = online_softmax_attention_f64(q, k, v, _cu([T]), True, 0.5, tau=-1.0, tile=16)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
    # a larger threshold skips at least as many rescales
    c = online_softmax_attention_f64(q, k, v, _cu([T]), True, 0.5, tau=8.0, tile=16)
    assert c[2]["taken"] <= a[2]["taken"]
    assert c[2]["considered"] == a[2]["considered"]


# Hand-built rescale counts.  scale = ln 2 makes c = scale * log2(e) exactly 1
# in fp64, so integer logits are exact in log2 units.  Query row 0 and row 1
# see ten keys in tiles of two; the tiles' maxima are
#     row 0: 0, 9, 16, 17, 10     (rises over the kept max: 9, 7, 8.0, 1)
#     row 1: 5, 5, 14, 20, 31     (rises: 0, 9, 6, 17)
# With the strict rule "rescale iff tile max - kept max > tau": tau = 8 takes
# row 0's first rise only (7 stays below and 8.0 is not above) and row 1's
# rises of 9 and 17; tau = 7 also takes row 0's 8.0; tau = 0 takes every
# strict increase; tau < 0 takes every tile after the first.
_HB_LOGITS = ([0, -3, 9, 2, 16, 1, 17, 0, 10, 5], [5, -1, 5, 4, 14, 3, 20, -7, 31, 0])
_HB_TAKEN = {8.0: (1, 2), 7.0: (2, 2), 0.0: (3, 3), -1.0: (4, 4)}


def _hand_built_counts(model, tau):
    """(taken, considered) of rows 0 and 1 (each repeated as 10 query rows), and the
    O, LSE of one row of each, from an online-softmax model function."""
    k = np.zeros((10, 1, 2))
    k[:, 0, 0], k[:, 0, 1] = _HB_LOGITS
    v = np.arange(20, dtype=np.float64).reshape(10, 1, 2)
    out = []
    for row in (0, 1):
        q = np.zeros((10, 1, 2))
        q[:, 0, row] = 1.0                                    # logits of every query row = column `row` of k
        O, L, st = model(q, k, v, np.array([0, 10]), False, math.log(2.0), tau=tau, tile=2)
        out.append((st["taken"] / 10, st["considered"] / 10, O[0, 0], L[0, 0]))
    return out


@pytest.mark.parametrize("tau", sorted(_HB_TAKEN))
def test_online_softmax_rescale_counts_hand_built(tau):
    assert math.log(2.0) * (1.0 / math.log(2.0)) == 1.0
    v = np.arange(20, dtype=np.float64).reshape(10, 2)
    for row, (taken, considered, O, L) in enumerate(_hand_built_counts(online_softmax_attention_f64, tau)):
        assert considered == 4
        assert taken == _HB_TAKEN[tau][row], (tau, row, taken)
        # whatever was skipped, the result is the plain definition
        w = np.array([2.0 ** x for x in _HB_LOGITS[row]])
        assert abs(L - math.log(w.sum())) <= 1e-12
        assert np.max(np.abs(O - (w / w.sum()) @ v)) <= 1e-10


_MODEL_PLANTS = {
    "non-strict rule": ("(m_t - m > tau)", "(m_t - m >= tau)"),
    "first tile counted": ("taken += int(np.count_nonzero(do & ~fresh))", "taken += int(np.count_nonzero(do))"),
    "max follows every tile": ("m_new = np.where(do, m_t, m)", "m_new = np.where(visible, np.maximum(m, m_t), m)"),
}


@pytest.mark.parametrize("plant", sorted(_MODEL_PLANTS))
def test_rescale_count_pin_catches_planted_mistakes(plant):
    """Each plausible mistake in the model's rescale rule, planted in a copy of
    its source, changes a hand-built count."""
    import inspect
    import oracle.online_softmax as mod
    old, new = _MODEL_PLANTS[plant]
    src = inspect.getsource(mod)
    assert src.count(old) == 1
    ns = {}
    exec(compile(src.replace(old, new), "<planted>", "exec"), ns)
    wrong = ns["online_softmax_attention_f64"]
    got = {tau: tuple(r[0] for r in _hand_built_counts(wrong, tau)) for tau in _HB_TAKEN}
    assert got != _HB_TAKEN, f"planted '{plant}' went unnoticed"


# ----------------------------------------------------------- planted mistakes

class _NpProxy:
    """numpy with selected functions replaced, to plant a mistake in the oracle."""

    def __init__(self, **over):
        self._over = over

    def __getattr__(self, name):
        return self._over.get(name, getattr(np, name))


_PLANTS = {
    "exp_base": dict(exp=np.exp2),                                    # softmax in base 2
    "log_base": dict(log=np.log2),                                    # LSE in log2
    "mask_flip": dict(arange=lambda n, *a, **kw: np.arange(n, *a, **kw)[::-1].copy()),
    "scale_dropped": dict(exp=lambda x: np.exp(x / 0.9)),             # logits without scale
}


@pytest.mark.parametrize("plant", sorted(_PLANTS))
def test_pins_catch_planted_mistakes(monkeypatch, plant):
    """Plant a mistake in the oracle module and check the brute-force pin fails."""
    monkeypatch.setattr(oracle_attention_mod, "np", _NpProxy(**_PLANTS[plant]))
    rng = np.random.default_rng(5)
    q = rng.standard_normal((4, 1, 3))
    k = rng.standard_normal((4, 1, 3))
    v = rng.standard_normal((4, 1, 2))
    O, L = attention_f64(q, k, v, _cu([4]), True, 0.9)
    monkeypatch.undo()
    Om, Lm = _brute_force_mp(q[:, 0], k[:, 0], v[:, 0], True, 0.9)
    err = max(np.max(np.abs(O[:, 0] - Om)), np.max(np.abs(L[0] - Lm)))
    assert err > 1e-6, "a planted mistake went unnoticed by the brute-force pin"


def test_head_subset_matches_full():
    T, H = 40, 4
    q, k, v = _rand(T, H, 8), _rand(T, H, 8), _rand(T, H, 8)
    O, L = attention_f64(q, k, v, _cu([T]), True, 0.5)
    Os, Ls = attention_f64(q, k, v, _cu([T]), True, 0.5, heads=[3, 1])
    assert np.array_equal(Os, O[:, [3, 1]]) and np.array_equal(Ls, L[[3, 1]])
