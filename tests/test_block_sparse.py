"""GPU parity of the block-sparse forward pass (attn_fwd_ex with a block mask)
against the fp64 block-sparse oracle.

Tolerances as for the dense forward pass (O max abs <= 2e-2, mean abs <=
2e-3; LSE max abs <= 1e-3), on rows that see at least one key; rows that see
none must give O = 0 and LSE = -inf exactly.  With an all-ones mask the
block-sparse kernel visits the same tiles with the same arithmetic as the
dense kernel, so its stored outputs must equal the dense ones bit for bit.
"""
import numpy as np
import pytest

import oracle
import workloads
from _gpu import TOL_LSE, TOL_O_MAX, TOL_O_MEAN, say, to_dev, torch_cuda

pytestmark = pytest.mark.gpu


def gpu_run(inp, causal, scale, mask, packed):
    torch = torch_cuda()
    import exact_attention_57_amd as ea
    q, k, v = to_dev(inp["q"]), to_dev(inp["k"]), to_dev(inp["v"])
    cu = torch.from_numpy(np.asarray(inp["cu_seqlens"], dtype=np.int32)).cuda() if packed else None
    bm = torch.from_numpy(np.ascontiguousarray(mask)).cuda() if mask is not None else None
    o, lse = ea.fwd(q, k, v, cu_seqlens=cu, max_seqlen=max(int(inp["N"]), 1), causal=causal, scale=scale,
                    block_mask=bm)
    torch.cuda.synchronize()
    return o, lse


def check(inp, causal, scale, mask, what, packed):
    say(f"[block-sparse] {what}: lengths {list(np.asarray(inp['lengths']))[:6]} H={inp['H']} "
        f"d=({inp['d_qk']},{inp['d_v']}) causal={causal} kept {mask.mean():.2f}")
    o, lse = gpu_run(inp, causal, scale, mask, packed)
    O_ref, L_ref = oracle.block_sparse_attention(inp["q"], inp["k"], inp["v"], inp["cu_seqlens"], causal, scale, mask)
    O = o.float().cpu().numpy().astype(np.float64)
    L = lse.cpu().numpy().astype(np.float64)
    empty = np.isneginf(L_ref)                                 # [H, T]: rows with no visible key
    say(f"  empty rows {int(empty.sum())} of {empty.size}")
    assert np.array_equal(np.isneginf(L), empty), "rows without keys must get LSE = -inf, and only they"
    assert np.all(O.transpose(1, 0, 2)[empty] == 0.0), "rows without keys must get O = 0"
    full = ~empty.T                                           # [T, H]
    e = np.abs(O - O_ref)[full]
    le = np.abs(L[~empty] - L_ref[~empty])
    say(f"  O max {e.max() if e.size else 0:.3e} mean {e.mean() if e.size else 0:.3e}  LSE max {le.max() if le.size else 0:.3e}")
    if e.size:
        assert e.max() <= TOL_O_MAX and e.mean() <= TOL_O_MEAN and le.max() <= TOL_LSE


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("density", [0.3, 0.7])
def test_random_masks_d128(causal, density):
    inp = workloads.make_custom_inputs([1000], 4, 128, 128, seed=21)
    mask = workloads.make_block_mask(1, 4, 1000, density, seed=int(density * 10) + causal)
    check(inp, causal, 1.0 / np.sqrt(128), mask, "random mask d128", packed=False)


@pytest.mark.parametrize("causal", [False, True])
def test_packed_ragged_d64(causal):
    inp = workloads.make_custom_inputs([1, 300, 0, 700, 129], 2, 64, 64, seed=22)
    mask = workloads.make_block_mask(5, 2, int(inp["N"]), 0.5, seed=3)
    check(inp, causal, 0.125, mask, "packed ragged d64", packed=True)


@pytest.mark.parametrize("causal", [False, True])
def test_split_dims_two_tiles_per_block(causal):
    """(192, 128): 64-key tiles, two per 128-key mask block; lengths with an
    odd tile count, so the last kept block holds a single tile."""
    inp = workloads.make_custom_inputs([300, 1, 0, 700, 129], 2, 192, 128, seed=25)
    mask = workloads.make_block_mask(5, 2, int(inp["N"]), 0.5, seed=5 + causal)
    check(inp, causal, 1.0 / np.sqrt(192), mask, "packed ragged (192,128)", packed=True)


@pytest.mark.parametrize("dims", [(128, 128), (192, 128)])
def test_empty_query_blocks(dims):
    """Whole query blocks with no kept key block, and a causal mask that hides
    the only kept block from some rows."""
    inp = workloads.make_custom_inputs([600], 2, dims[0], dims[1], seed=23)
    nb = 5
    mask = np.zeros((1, 2, nb, nb), dtype=np.uint8)
    mask[0, 0, 0, 0] = 1          # block row 0 keeps block 0
    mask[0, 0, 2, 3] = 1          # block row 2 keeps only key block 3: hidden under causal
    mask[0, 1, 4, 0] = 1
    mask[0, 1, 1, :] = 1
    check(inp, False, 0.09, mask, "empty query blocks, non-causal", packed=False)
    check(inp, True, 0.09, mask, "empty query blocks, causal", packed=False)


@pytest.mark.parametrize("dims", [(128, 128), (192, 128)])
@pytest.mark.parametrize("causal", [False, True])
def test_all_ones_mask_equals_dense_bitwise(causal, dims):
    torch = torch_cuda()
    inp = workloads.make_custom_inputs([777, 1200], 4, dims[0], dims[1], seed=24)
    nb = (int(inp["N"]) + 127) // 128
    mask = np.ones((2, 4, nb, nb), dtype=np.uint8)
    o1, l1 = gpu_run(inp, causal, 0.088, mask, packed=True)
    o0, l0 = gpu_run(inp, causal, 0.088, None, packed=True)
    assert torch.equal(o1.view(torch.int16), o0.view(torch.int16))
    assert torch.equal(l1, l0)


def test_full_size_sampled():
    """The benchmark shape (B4 H16 N4096 d128) at half density, two heads of
    one sequence against the oracle."""
    wl = workloads.workload("noncausal_b4h16n4096d128")
    inp = workloads.make_inputs(wl, seed=0)
    mask = workloads.make_block_mask(4, 16, 4096, 0.5, seed=0)
    say("[block-sparse] full size, density 0.5")
    o, lse = gpu_run(inp, False, inp["scale"], mask, packed=False)
    b, heads = 2, [3, 12]
    s, e = 2 * 4096, 3 * 4096
    sub = np.ascontiguousarray(mask[b:b + 1])
    O_ref, L_ref = oracle.block_sparse_attention(inp["q"][s:e], inp["k"][s:e], inp["v"][s:e], np.array([0, 4096]),
                                                 False, inp["scale"], sub, heads=heads)
    O = o[s:e][:, heads].float().cpu().numpy().astype(np.float64)
    L = lse[heads][:, s:e].cpu().numpy().astype(np.float64)
    ok = ~np.isneginf(L_ref)
    assert np.array_equal(np.isneginf(L), ~ok)
    err = np.abs(O - O_ref)[ok.T]
    say(f"  O max {err.max():.3e} mean {err.mean():.3e}  LSE max {np.abs(L - L_ref)[ok].max():.3e}")
    assert err.max() <= TOL_O_MAX and err.mean() <= TOL_O_MEAN
    assert np.abs(L - L_ref)[ok].max() <= TOL_LSE
