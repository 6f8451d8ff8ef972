"""GPU parity: the HIP forward pass against the fp64 CPU oracle.

Calls go through the C ABI (``exact_attention_57_amd.fwd`` -> ``attn_fwd_ex``)
with the default options, the same launch configuration the benchmark times.
Small and mid-size cases compare every output element; the full-size
workloads compare sampled rows (tile and block boundaries, last rows,
random rows) on a subset of heads, and check the whole output is finite.
"""
import numpy as np
import pytest

import oracle
import workloads
from _gpu import assert_close, lse_f64, o_f64, run, sample_rows, say

pytestmark = pytest.mark.gpu


def full_check(inp, what, **kw):
    o, lse = run(inp, **kw)
    O_ref, L_ref = oracle.attention(inp["q"], inp["k"], inp["v"], inp["cu_seqlens"],
                                    kw.get("causal", inp["causal"]),
                                    kw.get("scale", inp["scale"]))
    return assert_close(o_f64(o), lse_f64(lse), O_ref, L_ref, what), o, lse


def test_small_workload_all_elements():
    inp = workloads.make_inputs(1)
    say("case: small_noncausal_b1h2n256d64 seed 0")
    full_check(inp, "small workload")


@pytest.mark.parametrize("dims", [(64, 64), (128, 128), (192, 128)])
@pytest.mark.parametrize("causal", [False, True])
def test_ragged_packed_all_elements(dims, causal):
    """Lengths around the 64-key tile and 128-row block sizes, several tiles, ragged tails."""
    lengths = [1, 63, 64, 65, 127, 128, 129, 300, 777]
    inp = workloads.make_custom_inputs(lengths, H=3, d_qk=dims[0], d_v=dims[1], seed=11)
    inp["causal"] = causal
    inp["scale"] = 1.0 / np.sqrt(dims[0])
    say(f"case: ragged packed dims={dims} causal={causal}")
    full_check(inp, f"ragged {dims} causal={causal}")


@pytest.mark.parametrize("dims", [(128, 128), (192, 128)])
@pytest.mark.parametrize("causal", [False, True])
def test_many_heads_work_items_not_a_multiple_of_eight(dims, causal):
    """37 heads over three sequences, the longest 1100 tokens: a grid of
    37 x 3 x 5 = 555 work items of 256 rows (the grid follows the longest
    sequence), not a multiple of the 8 XCDs the default order deals them to,
    with several (sequence, head) pairs per XCD; every item must run once."""
    inp = workloads.make_custom_inputs([1100, 97, 300], H=37, d_qk=dims[0], d_v=dims[1], seed=31)
    inp["causal"] = causal
    inp["scale"] = 1.0 / np.sqrt(dims[0])
    say(f"case: 37 heads dims={dims} causal={causal}")
    full_check(inp, f"37 heads {dims} causal={causal}", packed=True)


@pytest.mark.parametrize("causal", [False, True])
def test_fixed_length_ragged_tail(causal):
    inp = workloads.make_custom_inputs([333, 333], H=2, d_qk=128, d_v=128, seed=12)
    inp["causal"] = causal
    inp["scale"] = 1.0 / np.sqrt(128)
    say(f"case: fixed length N=333 causal={causal}")
    full_check(inp, f"fixed N=333 causal={causal}", packed=False)


def test_empty_and_single_token_sequences():
    inp = workloads.make_custom_inputs([0, 5, 0, 1, 0, 130, 0], H=2, d_qk=64, d_v=64, seed=13)
    inp["scale"] = 0.125
    for causal in (False, True):
        inp["causal"] = causal
        say(f"case: empty/single sequences causal={causal}")
        full_check(inp, f"empty+single causal={causal}", packed=True)


def test_single_token_fixed_length():
    inp = workloads.make_custom_inputs([1, 1, 1], H=4, d_qk=128, d_v=128, seed=14)
    inp["scale"] = 0.3
    inp["causal"] = True
    say("case: B=3 N=1")
    _, o, _ = full_check(inp, "N=1", packed=False)
    # a single key returns its value exactly
    torch = pytest.importorskip("torch")
    assert np.array_equal(o.view(torch.int16).cpu().numpy().view(np.uint16), inp["v"])


def test_no_tokens_is_a_noop():
    torch = pytest.importorskip("torch")
    import exact_attention_57_amd as ea
    assert ea.fwd_raw(None, None, None, None, None, None, 2, 4, 0, 128, 128, 1.0, 1, None) == 0
    torch.cuda.synchronize()


def test_negative_and_tiny_scale():
    inp = workloads.make_custom_inputs([200, 57], H=2, d_qk=128, d_v=128, seed=15)
    for scale in (-0.09, 1e-35, 0.0):
        for causal in (False, True):
            inp["causal"] = causal
            inp["scale"] = scale
            say(f"case: scale={scale} causal={causal}")
            full_check(inp, f"scale={scale} causal={causal}", scale=scale, packed=True)


FULL = ["noncausal_b4h16n4096d128", "causal_b2h16n16384d128", "causal_b2h32n8192dqk192dv128",
        "varlen_causal_16seq_h32d128_ramp"]


@pytest.mark.slow
@pytest.mark.parametrize("key", FULL)
def test_full_size_sampled(key):
    wl = workloads.workload(key)
    say(f"case: full size {key}: drawing inputs")
    inp = workloads.make_inputs(wl, seed=0)
    say(f"  T={inp['T']} running GPU")
    o, lse = run(inp)
    torch = pytest.importorskip("torch")
    assert bool(torch.isfinite(o.float()).all()) and bool(torch.isfinite(lse).all())
    rows = sample_rows(inp["cu_seqlens"], per_seq=24 if wl.varlen else 48, seed=1)
    H = wl.H
    heads = sorted({0, H // 2, H - 1, 5 % H})
    say(f"  oracle on {len(rows)} rows x {len(heads)} heads")
    O_ref, L_ref = oracle.attention(inp["q"], inp["k"], inp["v"], inp["cu_seqlens"], wl.causal,
                                    inp["scale"], rows=rows, heads=heads)
    assert_close(o_f64(o, rows, heads), lse_f64(lse, rows, heads), O_ref, L_ref, key)
