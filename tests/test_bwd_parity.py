"""GPU parity of the backward pass (attn_bwd) against the fp64 gradient oracle.

Every gradient element must lie within the bound derived from the kernels'
arithmetic in ``_bwd_bound`` (bf16 rounding of P, dS and the outputs, fp32
sums, the forward's o and lse as given): |G_gpu - G_ref| <= bound element by
element, small entries included.  The relative RMS error is reported beside
the largest error-to-bound ratio.
"""
import numpy as np
import pytest

import oracle
import workloads
from _bwd_bound import check_within, grad_bounds
from _gpu import say, to_dev, torch_cuda

pytestmark = pytest.mark.gpu


def gpu_fwd_bwd(inp, causal, scale, dout_bits, packed):
    """(o, lse, dq, dk, dv) of the GPU forward and backward passes."""
    torch = torch_cuda()
    import exact_attention_57_amd as ea
    q, k, v = to_dev(inp["q"]), to_dev(inp["k"]), to_dev(inp["v"])
    do = to_dev(dout_bits)
    cu = torch.from_numpy(np.asarray(inp["cu_seqlens"], dtype=np.int32)).cuda() if packed else None
    N = max(int(inp["N"]), 1)
    o, lse = ea.fwd(q, k, v, cu_seqlens=cu, max_seqlen=N, causal=causal, scale=scale)
    dq, dk, dv = ea.bwd(q, k, v, o, lse, do, cu_seqlens=cu, max_seqlen=N, causal=causal, scale=scale)
    torch.cuda.synchronize()
    return o, lse, dq, dk, dv


def f64(t, heads=None):
    a = t.float().cpu().numpy().astype(np.float64)
    return a if heads is None else a[:, heads]


def check_grads(sub, dout, causal, scale, o, lse, grads, heads=None, rows=None):
    """Compare GPU gradients with the oracle within the derived bound.

    sub: input dict of the sequences compared (q, k, v bf16 bits, cu_seqlens);
    dout: its dO bits; o, lse, grads: GPU tensors for the same tokens
    (``rows`` selects them from larger GPU tensors); heads: head subset."""
    sel = slice(None) if rows is None else rows
    lse_np = lse.cpu().numpy().astype(np.float64)
    lse_np = lse_np[:, sel] if heads is None else lse_np[heads][:, sel]
    o_np = f64(o[sel], heads)
    O_ref, L_ref = oracle.attention(sub["q"], sub["k"], sub["v"], sub["cu_seqlens"], causal, scale, heads=heads)
    rq, rk, rv, _ = oracle.attention_backward(sub["q"], sub["k"], sub["v"], dout, sub["cu_seqlens"], causal,
                                              scale, heads=heads)
    bq, bk, bv = grad_bounds(sub["q"], sub["k"], sub["v"], dout, o_np, lse_np, O_ref, L_ref, rq, rk, rv,
                             sub["cu_seqlens"], causal, scale, heads=heads)
    for name, g, ref, bnd in zip(("dq", "dk", "dv"), grads, (rq, rk, rv), (bq, bk, bv)):
        check_within(name, f64(g[sel], heads), ref, bnd, say=say)


def full_check(inp, causal, scale, what, packed=None, seed=0):
    lengths = np.asarray(inp["lengths"])
    if packed is None:
        packed = bool(len(lengths) == 0 or lengths.min() != lengths.max())
    inp = dict(inp)
    dout = workloads.make_output_grad(inp, seed)
    say(f"[bwd parity] {what}: lengths {list(lengths)[:8]} H={inp['H']} d=({inp['d_qk']},{inp['d_v']}) "
        f"causal={causal} packed={packed}")
    o, lse, dq, dk, dv = gpu_fwd_bwd(inp, causal, scale, dout, packed)
    check_grads(inp, dout, causal, scale, o, lse, (dq, dk, dv))


@pytest.mark.parametrize("causal", [False, True])
def test_small_workload_all_elements(causal):
    inp = workloads.make_custom_inputs([256], 2, 64, 64, seed=0)
    full_check(inp, causal, 0.125, "B1 H2 N256 d64")


@pytest.mark.parametrize("dims", [(64, 64), (128, 128), (192, 128)])
@pytest.mark.parametrize("causal", [False, True])
def test_ragged_packed_all_elements(dims, causal):
    inp = workloads.make_custom_inputs([1, 77, 300, 129], 2, dims[0], dims[1], seed=3)
    full_check(inp, causal, 1.0 / np.sqrt(dims[0]), f"packed ragged d{dims}")


@pytest.mark.parametrize("dims", [(64, 64), (128, 128), (192, 128)])
@pytest.mark.parametrize("causal", [False, True])
def test_sequences_ending_on_tile_and_block_boundaries(dims, causal):
    """Sequence ends exactly at multiples of the key tiles (32, 64), the
    128-key dK/dV block and the 256-query dQ block, so the tile after a
    sequence's last one lies wholly past its end."""
    inp = workloads.make_custom_inputs([256, 32, 64, 512, 128], 2, dims[0], dims[1], seed=21)
    full_check(inp, causal, 1.0 / np.sqrt(dims[0]), f"boundary-length sequences d{dims}", packed=True)


@pytest.mark.parametrize("dims", [(128, 128), (192, 128)])
@pytest.mark.parametrize("causal", [False, True])
def test_many_heads_work_items_not_a_multiple_of_eight(dims, causal):
    """37 heads over three sequences, the longest 1100 tokens: grids of
    37 x 3 x 9 = 999 dK/dV blocks of 128 keys and 37 x 3 x 5 = 555 dQ blocks
    of 256 queries, neither a multiple of the 8 XCDs the work order deals
    them to; every gradient element is checked."""
    inp = workloads.make_custom_inputs([1100, 97, 300], 37, dims[0], dims[1], seed=31)
    full_check(inp, causal, 1.0 / np.sqrt(dims[0]), f"37 heads d{dims}", packed=True)


@pytest.mark.parametrize("causal", [False, True])
def test_fixed_length_ragged_tail(causal):
    inp = workloads.make_custom_inputs([300, 300], 2, 128, 128, seed=5)
    full_check(inp, causal, 1.0 / np.sqrt(128), "fixed N300 d128", packed=False)


@pytest.mark.parametrize("dims", [(64, 64), (128, 128), (192, 128)])
def test_empty_and_single_token_sequences(dims):
    inp = workloads.make_custom_inputs([0, 1, 0, 64, 5], 3, dims[0], dims[1], seed=7)
    full_check(inp, True, 1.0 / np.sqrt(dims[0]), f"empty and single-token sequences d{dims}", packed=True)


def test_split_dims_negative_scale_and_large_logits():
    inp = workloads.make_custom_inputs([200, 130], 2, 192, 128, seed=12, std=3.0)
    full_check(inp, True, 0.25, "(192,128) std 3 inputs, scale 0.25", packed=True)
    full_check(inp, False, -0.04, "(192,128) negative scale", packed=True)


def test_large_logits_and_negative_scale():
    inp = workloads.make_custom_inputs([200, 130], 2, 128, 128, seed=11, std=3.0)
    full_check(inp, True, 0.3, "std 3 inputs, scale 0.3 (large logits)", packed=True)
    full_check(inp, False, -0.05, "negative scale", packed=True)


def test_deterministic():
    """No atomics: two runs give the same bits."""
    torch = torch_cuda()
    inp = workloads.make_custom_inputs([700, 333], 4, 128, 128, seed=13)
    dout = workloads.make_output_grad(inp, 1)
    a = gpu_fwd_bwd(inp, True, 0.088, dout, True)[2:]
    b = gpu_fwd_bwd(inp, True, 0.088, dout, True)[2:]
    for x, y in zip(a, b):
        assert torch.equal(x.view(torch.int16), y.view(torch.int16))


def test_column_sum_identities_mid_size():
    """sum_j dk_j = 0 and sum_j dv_j = sum_i dO_i per (sequence, head), at a
    size where the full oracle would be slow to compare element by element."""
    inp = workloads.make_custom_inputs([2048, 1500], 4, 128, 128, seed=17)
    dout = workloads.make_output_grad(inp, 2)
    _, _, dq, dk, dv = gpu_fwd_bwd(inp, True, 1.0 / np.sqrt(128), dout, True)
    dk, dv = f64(dk), f64(dv)
    do = workloads.bf16_bits_to_f32(dout).astype(np.float64)
    cu = inp["cu_seqlens"]
    for b in range(len(cu) - 1):
        s, e = int(cu[b]), int(cu[b + 1])
        sk = np.abs(dk[s:e].sum(axis=0)) / np.abs(dk[s:e]).sum(axis=0)
        sv = np.abs(dv[s:e].sum(axis=0) - do[s:e].sum(axis=0)) / np.abs(dv[s:e]).sum(axis=0)
        say(f"  seq {b}: max |sum dk| / sum |dk| = {sk.max():.2e}, max |sum dv - sum dO| / sum |dv| = {sv.max():.2e}")
        assert sk.max() <= 1e-2 and sv.max() <= 1e-2


def _last_sequence(inp, dout):
    cu = inp["cu_seqlens"]
    b = inp["B"] - 1
    s, e = int(cu[b]), int(cu[b + 1])
    sub = dict(q=inp["q"][s:e], k=inp["k"][s:e], v=inp["v"][s:e], cu_seqlens=np.array([0, e - s]))
    return sub, dout[s:e], slice(s, e)


@pytest.mark.slow
@pytest.mark.parametrize("causal", [False, True])
def test_full_size_all_heads_of_one_sequence(causal):
    """At the benchmark shape (B4 H16 N4096 d128): every head of the last
    sequence, every element, against the oracle within the derived bound."""
    wl = workloads.workload("noncausal_b4h16n4096d128")
    inp = workloads.make_inputs(wl, seed=0)
    dout = workloads.make_output_grad(inp, 0)
    say(f"[bwd parity] full size {wl.key} causal={causal}: all {inp['H']} heads of the last sequence")
    o, lse, dq, dk, dv = gpu_fwd_bwd(inp, causal, inp["scale"], dout, False)
    sub, dsub, rows = _last_sequence(inp, dout)
    check_grads(sub, dsub, causal, inp["scale"], o, lse, (dq, dk, dv), rows=rows)


@pytest.mark.slow
@pytest.mark.parametrize("causal", [False, True])
def test_split_dims_full_size_sampled_heads(causal):
    """The split head dims of the causal (192, 128) workload (B2 H32 N8192):
    four whole (sequence, head) pairs of the last sequence, every element,
    within the derived bound (non-causal too: the kernels serve both)."""
    wl = workloads.workload("causal_b2h32n8192dqk192dv128")
    inp = workloads.make_inputs(wl, seed=0)
    dout = workloads.make_output_grad(inp, 0)
    say(f"[bwd parity] full size {wl.key} causal={causal}")
    o, lse, dq, dk, dv = gpu_fwd_bwd(inp, causal, inp["scale"], dout, False)
    sub, dsub, rows = _last_sequence(inp, dout)
    check_grads(sub, dsub, causal, inp["scale"], o, lse, (dq, dk, dv), heads=[0, 3, 17, inp["H"] - 1], rows=rows)
