"""GPU parity of the FP8 (E4M3) forward against the fp64 oracle of the
dequantised inputs (``oracle.attention_fp8``), through the C ABI
(``exact_attention_57_amd.fwd_fp8`` -> ``attn_fwd_fp8``).

Tolerance, derived from the kernel's arithmetic.  The inputs are exact
(E4M3 values times fp32 descales) and both products accumulate in fp32; the
one rounding that matters is P -> E4M3 before the second product, with the row
sum l taken over the same rounded values.  With p_j the unrounded weights of a
row (relative to the kernel's kept max m, so max_j p_j >= 1 and l >= the
oracle's row sum relative to the true max) and p~_j the rounded ones,

    |p~_j - p_j| <= 2^-4 p_j + min(p_j, 2^-10)   (half an E4M3 step: 2^-4 p in
                                   the normal range, 2^-10 among the subnormals,
                                   p itself where p flushes to 0)
    O - O_ref = sum_j (p~_j - p_j)(v_j - O_ref) / sum_j p~_j          (exact)

and min(p_j, 2^-10) / l is largest with the true max (the kept max only scales
p and l up), so with P_j = exp(s_j - max s) and l = sum_j P_j from the oracle,
w_j = P_j / l, f_j = min(P_j, 2^-10) and F = sum_j f_j,

    |O - O_ref| <= [2^-4 (sum_j w_j |v_j| + |O_ref|) + (sum_j f_j |v_j| + F |O_ref|) / l] / den
                   + 2^-8 |O_ref| + 2e-4 max_j |v_j|,
    den = 1 - 2^-4 - F / l,
    |LSE - LSE_ref| <= -ln(den) + 1e-5,

the last terms covering the bf16 output rounding (2^-9 relative) and the fp32
sums.  The tests assert this bound element by element and report the mean
errors, which on N(0, 1) inputs are two orders of magnitude smaller.
"""
import math

import numpy as np
import pytest

import oracle
import workloads
from _gpu import lse_f64, o_f64, run, sample_rows, say, torch_cuda

pytestmark = pytest.mark.gpu

E4_REL = 2.0 ** -4
E4_ABS = 2.0 ** -10


def fp8_inputs(inp, prescale=(1.0, 1.0, 1.0)):
    f = workloads.make_fp8_inputs(inp, prescale)
    f["causal"] = inp.get("causal", False)
    f["scale"] = inp.get("scale", 1.0 / math.sqrt(inp["d_qk"]))
    return f


def run_fp8(f, causal=None, packed=None, scale=None, q8=None, **kw):
    torch = torch_cuda()
    import exact_attention_57_amd as ea
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    lengths = np.asarray(f["lengths"])
    if packed is None:
        packed = bool(len(lengths) == 0 or lengths.min() != lengths.max())
    cu = dev(np.asarray(f["cu_seqlens"], dtype=np.int32)) if packed else None
    causal = f["causal"] if causal is None else causal
    scale = f["scale"] if scale is None else scale
    args = dict(q_descale=f["q_descale"], k_descale=f["k_descale"], v_descale=f["v_descale"])
    args.update(kw)
    o, lse = ea.fwd_fp8(dev(f["q8"] if q8 is None else q8), dev(f["k8"]), dev(f["v8"]), cu_seqlens=cu,
                        max_seqlen=max(int(f["N"]), 1), causal=causal, scale=scale, **args)
    torch.cuda.synchronize()
    return o, lse


def bounds(f, causal, scale, rows=None, heads=None, q_descale=None, k_descale=None, v_descale=None):
    """(O_ref, LSE_ref, bound_O, bound_LSE) for the selected rows and heads (module docstring)."""
    qd = f["q_descale"] if q_descale is None else q_descale
    kd = f["k_descale"] if k_descale is None else k_descale
    vd = f["v_descale"] if v_descale is None else v_descale
    cu = np.asarray(f["cu_seqlens"], dtype=np.int64)
    T, H, _ = f["q8"].shape
    heads = list(range(H)) if heads is None else list(heads)
    rows = np.arange(T) if rows is None else np.asarray(rows)
    d_v = f["v8"].shape[2]
    O = np.empty((len(rows), len(heads), d_v))
    L = np.empty((len(heads), len(rows)))
    BO = np.empty_like(O)
    BL = np.empty_like(L)
    r0 = 0
    for b in range(len(cu) - 1):
        s, e = cu[b], cu[b + 1]
        sel = rows[(rows >= s) & (rows < e)]
        if len(sel) == 0:
            continue
        pos = sel - s
        for hi, h in enumerate(heads):
            q = oracle.e4m3_to_f64(f["q8"][sel, h]) * qd
            k = oracle.e4m3_to_f64(f["k8"][s:e, h]) * kd
            v = oracle.e4m3_to_f64(f["v8"][s:e, h]) * vd
            S = scale * (q @ k.T)
            if causal:
                S[np.arange(e - s)[None, :] > pos[:, None]] = -np.inf
            m = S.max(axis=1)
            P = np.exp(S - m[:, None])
            l = P.sum(axis=1)
            W = P / l[:, None]
            Oi = W @ v
            n = (pos + 1) if causal else np.full(len(sel), e - s)
            av = np.abs(v)
            vmax = np.array([av[:c].max(axis=0) for c in n]) if causal else np.broadcast_to(av.max(axis=0), Oi.shape)
            Fm = np.minimum(P, E4_ABS)                 # masked keys: P = 0
            F = Fm.sum(axis=1)
            den = 1.0 - E4_REL - F / l
            assert np.all(den > 0.5)
            bo = (E4_REL * (W @ av + np.abs(Oi)) + (Fm @ av + F[:, None] * np.abs(Oi)) / l[:, None]) / den[:, None]
            bo += 2.0 ** -8 * np.abs(Oi) + 2e-4 * vmax
            O[r0:r0 + len(sel), hi] = Oi
            L[hi, r0:r0 + len(sel)] = m + np.log(l)
            BO[r0:r0 + len(sel), hi] = bo
            BL[hi, r0:r0 + len(sel)] = -np.log(den) + 1e-5
        r0 += len(sel)
    return O, L, BO, BL


def check(f, o, lse, what, causal=None, scale=None, rows=None, heads=None, **descales):
    causal = f["causal"] if causal is None else causal
    scale = f["scale"] if scale is None else scale
    O_ref, L_ref, BO, BL = bounds(f, causal, scale, rows, heads, **descales)
    # the bound computation is an independent restatement; the reference
    # values themselves come from the oracle
    O_or, L_or = oracle.attention_fp8(f["q8"], f["k8"], f["v8"], f["cu_seqlens"], causal, scale,
                                      descales.get("q_descale", f["q_descale"]),
                                      descales.get("k_descale", f["k_descale"]),
                                      descales.get("v_descale", f["v_descale"]),
                                      rows=rows, heads=heads)
    assert np.allclose(O_ref, O_or, rtol=0, atol=1e-10) and np.allclose(L_ref, L_or, rtol=0, atol=1e-10)
    O = o_f64(o, rows, heads)
    L = lse_f64(lse, rows, heads)
    assert np.isfinite(O).all() and np.isfinite(L).all(), f"{what}: non-finite output"
    eo = np.abs(O - O_or)
    el = np.abs(L - L_or)
    say(f"  fp8 parity {what}: O max {eo.max():.3e} mean {eo.mean():.3e} (bound max {BO.max():.3e}, "
        f"worst err/bound {np.max(np.divide(eo, BO, out=np.zeros_like(eo), where=BO > 0)):.3f}); "
        f"LSE max {el.max():.3e} mean {el.mean():.3e} "
        f"(bound {BL.max():.3e})")
    assert np.all(eo <= BO), f"{what}: O outside the E4M3 rounding bound"
    assert np.all(el <= BL), f"{what}: LSE outside the E4M3 rounding bound"
    return eo, el


@pytest.mark.parametrize("d", [64, 128])
def test_fp8_small_all_elements(d):
    inp = workloads.make_custom_inputs([256], H=2, d_qk=d, d_v=d, seed=0)
    f = fp8_inputs(inp)
    say(f"case: fp8 B1 H2 N256 d{d} non-causal seed 0")
    o, lse = run_fp8(f)
    check(f, o, lse, f"small d={d}")


@pytest.mark.parametrize("dims", [(64, 64), (128, 128), (192, 128)])
@pytest.mark.parametrize("causal", [False, True])
def test_fp8_ragged_packed_all_elements(causal, dims):
    lengths = [1, 63, 64, 65, 127, 128, 129, 300, 777]
    inp = workloads.make_custom_inputs(lengths, H=3, d_qk=dims[0], d_v=dims[1], seed=11)
    inp["causal"] = causal
    f = fp8_inputs(inp, prescale=(4.0, 2.0, 8.0))
    say(f"case: fp8 ragged packed dims={dims} causal={causal} prescale (4, 2, 8)")
    o, lse = run_fp8(f)
    check(f, o, lse, f"ragged dims={dims} causal={causal}")


@pytest.mark.parametrize("causal", [False, True])
def test_fp8_many_heads_work_items_not_a_multiple_of_eight(causal):
    """37 heads over three sequences, the longest 1100 tokens: a grid of
    37 x 3 x 5 = 555 work items, not a multiple of the 8 XCDs the work order
    deals them to; every element within the derived bound."""
    inp = workloads.make_custom_inputs([1100, 97, 300], H=37, d_qk=128, d_v=128, seed=31)
    inp["causal"] = causal
    f = fp8_inputs(inp, prescale=(4.0, 2.0, 8.0))
    say(f"case: fp8 37 heads causal={causal}")
    o, lse = run_fp8(f)
    check(f, o, lse, f"37 heads causal={causal}")


@pytest.mark.parametrize("causal", [False, True])
def test_fp8_fixed_length_ragged_tail(causal):
    inp = workloads.make_custom_inputs([333, 333], H=2, d_qk=128, d_v=128, seed=12)
    inp["causal"] = causal
    f = fp8_inputs(inp)
    say(f"case: fp8 fixed length N=333 causal={causal}")
    o, lse = run_fp8(f, packed=False)
    check(f, o, lse, f"fixed N=333 causal={causal}")


def test_fp8_empty_and_single_token_sequences():
    inp = workloads.make_custom_inputs([0, 5, 0, 1, 0, 130, 0], H=2, d_qk=128, d_v=128, seed=13)
    f = fp8_inputs(inp, prescale=(0.5, 1.0, 2.0))
    for causal in (False, True):
        say(f"case: fp8 empty/single sequences causal={causal}")
        o, lse = run_fp8(f, causal=causal, packed=True)
        check(f, o, lse, f"empty+single causal={causal}", causal=causal)


def test_fp8_non_power_of_two_descales():
    """Descales that are not powers of two: the combined logit factor and the
    output factor are rounded to fp32 in the library."""
    inp = workloads.make_custom_inputs([300, 517], H=2, d_qk=128, d_v=128, seed=27)
    inp["causal"] = True
    f = fp8_inputs(inp, prescale=(3.7, 0.61, 11.3))
    say("case: fp8 descales 1/3.7, 1/0.61, 1/11.3")
    o, lse = run_fp8(f)
    check(f, o, lse, "non-power-of-two descales")


@pytest.mark.parametrize("causal", [False, True])
def test_fp8_large_logits_exercise_rescaling(causal):
    """Peaked rows: std-3 inputs at scale 0.3 (logits of order +-100) make the
    kept max stale by up to 8 (P up to 256, near E4M3's 448) and most weights
    flush below the E4M3 range."""
    inp = workloads.make_custom_inputs([200, 130, 1000], H=2, d_qk=128, d_v=128, seed=21, std=3.0)
    inp["causal"] = causal
    inp["scale"] = 0.3
    f = fp8_inputs(inp, prescale=(0.5, 0.5, 1.0))
    say(f"case: fp8 large logits causal={causal}")
    o, lse = run_fp8(f)
    check(f, o, lse, f"large logits causal={causal}")


def test_fp8_special_values():
    """Causal row 0 returns v_0 exactly (P = exp2(0) = 1); Q = 0 gives the mean of
    the visible V rows and LSE = ln(count); negative scale equals negated Q codes."""
    torch = torch_cuda()
    inp = workloads.make_custom_inputs([200, 260], H=2, d_qk=128, d_v=128, seed=14)
    f = fp8_inputs(inp, prescale=(1.0, 1.0, 4.0))
    say("case: fp8 special values")
    o, lse = run_fp8(f, causal=True, packed=True)
    v = oracle.e4m3_to_f64(f["v8"]) * f["v_descale"]
    O = o_f64(o)
    for s in (0, 200):
        assert np.array_equal(O[s], v[s]), "causal row 0 must return v_0"
    z = np.zeros_like(f["q8"])
    o0, lse0 = run_fp8(f, causal=True, packed=True, q8=z)
    O0, L0 = o_f64(o0), lse_f64(lse0)
    for s, e in ((0, 200), (200, 460)):
        cnt = np.arange(1, e - s + 1)
        ref = np.cumsum(v[s:e], axis=0) / cnt[:, None, None]
        assert np.max(np.abs(O0[s:e] - ref)) <= 2.0 ** -8 * np.abs(ref).max() + 1e-5
        assert np.max(np.abs(L0[:, s:e] - np.log(cnt)[None, :])) <= 1e-5
    neg = f["q8"] ^ np.uint8(0x80)
    o1, lse1 = run_fp8(f, causal=True, packed=True, scale=-f["scale"], q8=neg)
    assert torch.equal(o1, o) and torch.equal(lse1, lse)


def test_fp8_descales_fold_into_one_factor_and_runs_repeat_bitwise():
    torch = torch_cuda()
    inp = workloads.make_custom_inputs([500, 1000], H=2, d_qk=128, d_v=128, seed=15)
    f = fp8_inputs(inp)
    say("case: fp8 descale folding and determinism")
    a = run_fp8(f, causal=True, scale=0.25, q_descale=1.0, k_descale=1.0)
    b = run_fp8(f, causal=True, scale=0.125, q_descale=4.0, k_descale=0.5)
    c = run_fp8(f, causal=True, scale=0.25, q_descale=1.0, k_descale=1.0)
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])
    assert torch.equal(a[0], c[0]) and torch.equal(a[1], c[1])


def test_fp8_agrees_with_bf16_kernel_on_the_same_values():
    """E4M3 values are exact in bf16: the bf16 kernel on the dequantised inputs
    is a second reference, within the bf16 tolerance plus the E4M3 bound."""
    inp = workloads.make_custom_inputs([129, 700], H=2, d_qk=128, d_v=128, seed=16)
    f = fp8_inputs(inp)
    bf = dict(inp)
    for name in ("q", "k", "v"):
        x = oracle.e4m3_to_f64(f[name + "8"]).astype(np.float32)
        bf[name] = workloads.f32_to_bf16_bits(x)
    bf["causal"] = True
    bf["scale"] = f["scale"]
    say("case: fp8 vs bf16 kernel")
    o8, l8 = run_fp8(f, causal=True)
    ob, lb = run(bf, causal=True)
    _, _, BO, BL = bounds(f, True, f["scale"])
    assert np.all(np.abs(o_f64(o8) - o_f64(ob)) <= BO + 2e-2)
    assert np.all(np.abs(lse_f64(l8) - lse_f64(lb)) <= BL + 1e-3)


@pytest.mark.parametrize("key", ["noncausal_b4h16n4096d128", "causal_b2h16n16384d128", "causal_b2h32n8192dqk192dv128",
                                 "varlen_causal_16seq_h32d128_ramp"])
def test_fp8_full_size_sampled(key):
    inp = workloads.make_inputs(key)
    f = fp8_inputs(inp)
    say(f"case: fp8 full size {key}")
    o, lse = run_fp8(f)
    torch = torch_cuda()
    assert bool(torch.isfinite(o.float()).all()) and bool(torch.isfinite(lse).all())
    rows = sample_rows(f["cu_seqlens"], per_seq=8 if f["B"] > 4 else 24, seed=3)
    check(f, o, lse, key, rows=rows, heads=[0, 5, 10, 15])
