"""GPU parity of every method variant of the dense forward pass.

The kernel has 24 dense instances: (d_qk, d_v) in {(64,64), (128,128),
(192,128)} x causal in {0, 1} x the share of exponentials on the software
exp2 (poly in {0, 2, 4, 8} sixteenths), and each runs with any conditional-
rescale threshold tau (here -1: always rescale, 0, and the default 8).  For
every (dims, causal) pair one ragged packed input is drawn whose logits grow
steeply along each sequence, so that row maxima rise by more than 8 (log2
units) between tiles and rescales are both taken and skipped (checked through
the kernel's statistics counters).  Every variant's output is compared element
by element

  * with the fp64 oracle (O max 2e-2, mean 2e-3; LSE 1e-3), and
  * with the tau = -1 / poly = 0 run (the unconditional online softmax on the
    hardware exp2) at the same tolerance,

and tau = 0 must equal tau = -1 bit for bit at every poly share.

Sources: conditional rescaling, wittx news "FlashAttention-4", section on
skipping 90% of rescales; the software exp2, the same page's section on faking
a hardware instruction in software.

At full size, the packed causal ramp workload (16 sequences, H = 32, d = 128)
runs tau = 8 vs tau = -1 and poly = 2 vs poly = 0: each variant against the
oracle on sampled rows, and against the baseline variant on every element.
"""
import numpy as np
import pytest

import oracle
import workloads
from _gpu import assert_close, errors, lse_f64, o_f64, run, sample_rows, say, torch_cuda, TOL_LSE, TOL_O_MAX, TOL_O_MEAN

pytestmark = pytest.mark.gpu

DIMS = [(64, 64), (128, 128), (192, 128)]
TAUS = [-1.0, 0.0, 8.0]
POLYS = [0, 2, 4, 8]
LENGTHS = [1, 129, 300, 700]


def steep_ramp_inputs(lengths, H, d_qk, d_v, seed, strength=20.0):
    """Packed N(0,1) bf16 inputs plus a ramp: every query gets +strength/sqrt(d_qk)
    on each element and key j of a sequence of length L gets
    +strength/sqrt(d_qk) * j/(L-1), so the scaled logit grows by about
    strength^2/sqrt(d_qk) nats along each sequence (the packed workload's ramp,
    steeper: at strength 20 and L = 700 a 128-key tile raises the row max by
    about 6-13 in log2 units)."""
    inp = workloads.make_custom_inputs(lengths, H=H, d_qk=d_qk, d_v=d_v, seed=seed)
    a = np.float32(strength / np.sqrt(d_qk))
    q = workloads.bf16_bits_to_f32(inp["q"]) + a
    k = workloads.bf16_bits_to_f32(inp["k"])
    cu = inp["cu_seqlens"]
    for b, L in enumerate(lengths):
        t = np.arange(L, dtype=np.float32) / max(L - 1, 1)
        k[cu[b]:cu[b + 1]] += (a * t)[:, None, None]
    inp["q"] = workloads.f32_to_bf16_bits(q)
    inp["k"] = workloads.f32_to_bf16_bits(k)
    inp["scale"] = 1.0 / np.sqrt(d_qk)
    return inp


def bits(t):
    torch = torch_cuda()
    return t.view(torch.int16).cpu().numpy() if t.dtype == torch.bfloat16 else t.cpu().numpy().view(np.uint32)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("dims", DIMS)
def test_every_variant_against_oracle_and_baseline(dims, causal):
    torch = torch_cuda()
    inp = steep_ramp_inputs(LENGTHS, H=2, d_qk=dims[0], d_v=dims[1], seed=40 + dims[0] + int(causal))
    inp["causal"] = causal
    say(f"case: variants dims={dims} causal={causal} lengths={LENGTHS}")
    O_ref, L_ref = oracle.attention(inp["q"], inp["k"], inp["v"], inp["cu_seqlens"], causal, inp["scale"])
    out = {}
    for tau in TAUS:
        for poly in POLYS:
            stats = torch.zeros(4, dtype=torch.int64, device="cuda")
            o, lse = run(inp, packed=True, rescale_threshold_log2=tau, poly_exp_sixteenths=poly, stats=stats)
            st = stats.cpu().numpy()
            out[tau, poly] = (o, lse)
            if poly == 0:
                say(f"  tau={tau}: rescales taken {st[1]} of {st[0]} considered")
                assert st[0] > 0
                if tau == 8.0:
                    # the input forces some rescales past the threshold, and the threshold skips others
                    assert 0 < st[1] < st[0], st
            assert_close(o_f64(o), lse_f64(lse), O_ref, L_ref, f"tau={tau} poly={poly} vs oracle")
    base_o, base_l = out[-1.0, 0]
    for (tau, poly), (o, lse) in out.items():
        if (tau, poly) != (-1.0, 0):
            assert_close(o_f64(o), lse_f64(lse), o_f64(base_o), lse_f64(base_l),
                         f"tau={tau} poly={poly} vs tau=-1 poly=0")
    for poly in POLYS:
        assert np.array_equal(bits(out[0.0, poly][0]), bits(out[-1.0, poly][0])), f"tau 0 vs -1 O, poly {poly}"
        assert np.array_equal(bits(out[0.0, poly][1]), bits(out[-1.0, poly][1])), f"tau 0 vs -1 LSE, poly {poly}"


@pytest.fixture(scope="module")
def packed_ramp_full():
    wl = workloads.workload("varlen_causal_16seq_h32d128_ramp")
    say(f"case: full size {wl.key}: drawing inputs")
    return wl, workloads.make_inputs(wl, seed=0)


def _device_diff(a, b):
    """max and mean |a - b| over whole tensors, on the GPU (float32)."""
    d = (a.float() - b.float()).abs()
    return float(d.max()), float(d.mean())


@pytest.mark.slow
@pytest.mark.parametrize("variant", [dict(rescale_threshold_log2=8.0, poly_exp_sixteenths=0),
                                     dict(rescale_threshold_log2=8.0, poly_exp_sixteenths=2),
                                     dict(rescale_threshold_log2=-1.0, poly_exp_sixteenths=2)])
def test_full_size_packed_ramp_variants(packed_ramp_full, variant):
    """The packed causal ramp workload at full size: the variant against the oracle
    on sampled rows of 4 heads, and against tau = -1 / poly = 0 on every element."""
    torch = torch_cuda()
    wl, inp = packed_ramp_full
    say(f"  variant {variant}")
    base_o, base_l = run(inp, rescale_threshold_log2=-1.0, poly_exp_sixteenths=0)
    o, lse = run(inp, **variant)
    assert bool(torch.isfinite(o.float()).all()) and bool(torch.isfinite(lse).all())
    omax, omean = _device_diff(o, base_o)
    lmax, _ = _device_diff(lse, base_l)
    say(f"  vs tau=-1 poly=0 on all {o.numel()} outputs: O max {omax:.3e} mean {omean:.3e}, LSE max {lmax:.3e}")
    assert omax <= TOL_O_MAX and omean <= TOL_O_MEAN and lmax <= TOL_LSE
    del base_o, base_l
    rows = sample_rows(inp["cu_seqlens"], per_seq=16, seed=2)
    heads = [0, 7, 20, wl.H - 1]
    O_ref, L_ref = oracle.attention(inp["q"], inp["k"], inp["v"], inp["cu_seqlens"], True, inp["scale"],
                                    rows=rows, heads=heads)
    err = errors(o_f64(o, rows, heads), lse_f64(lse, rows, heads), O_ref, L_ref)
    say(f"  vs oracle on {len(rows)} rows x {len(heads)} heads: {err}")
    assert err["o_max"] <= TOL_O_MAX and err["o_mean"] <= TOL_O_MEAN and err["lse_max"] <= TOL_LSE
