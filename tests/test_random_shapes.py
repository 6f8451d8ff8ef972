"""GPU parity over a seeded sweep of small random configurations, for every
entry point: ragged packed lengths (including empty and one-token
sequences), every supported head-dim pair, causal or not, scales of either
sign, block masks of random density and FP8 descales.  Each case is compared
element by element with the fp64 oracle at the tolerance of its row (forward:
O max 2e-2, mean 2e-3, LSE 1e-3; backward: the derived per-element bound of
_bwd_bound; FP8: the derived E4M3 bound of test_fp8_parity).
The draws come from their own seed, so the sweep is the same on every run."""
import numpy as np
import pytest

import oracle
import workloads
from _gpu import TOL_LSE, TOL_O_MAX, TOL_O_MEAN, say, to_dev, torch_cuda

pytestmark = pytest.mark.gpu

DIMS = [(64, 64), (128, 128), (192, 128)]
N_CASES = 24


def draw_case(i):
    rng = np.random.default_rng(np.random.SeedSequence(2024, spawn_key=(i,)))
    nseq = int(rng.integers(1, 5))
    lengths = [int(x) for x in rng.choice([0, 1, 2, 31, 64, 65, 127, 200, 256, 333, 511], size=nseq)]
    if sum(lengths) == 0:
        lengths[0] = 97
    dims = DIMS[int(rng.integers(0, 3))]
    H = int(rng.integers(1, 4))
    causal = bool(rng.integers(0, 2))
    scale = float(rng.choice([1.0, -1.0])) * float(rng.uniform(0.03, 0.2))
    return dict(lengths=lengths, dims=dims, H=H, causal=causal, scale=scale, seed=100 + i,
                density=float(rng.uniform(0.2, 0.9)), prescale=tuple(float(x) for x in rng.uniform(0.3, 6.0, 3)))


def _dev_run(c, inp):
    torch = torch_cuda()
    cu = torch.from_numpy(np.asarray(inp["cu_seqlens"], dtype=np.int32)).cuda()
    return torch, cu, max(int(inp["N"]), 1)


@pytest.mark.parametrize("i", range(N_CASES))
def test_forward_and_backward(i):
    import exact_attention_57_amd as ea
    c = draw_case(i)
    say(f"case {i}: {c}")
    inp = workloads.make_custom_inputs(c["lengths"], c["H"], c["dims"][0], c["dims"][1], seed=c["seed"])
    torch, cu, N = _dev_run(c, inp)
    q, k, v = to_dev(inp["q"]), to_dev(inp["k"]), to_dev(inp["v"])
    o, lse = ea.fwd(q, k, v, cu_seqlens=cu, max_seqlen=N, causal=c["causal"], scale=c["scale"])
    dout = workloads.make_output_grad(inp, c["seed"])
    dq, dk, dv = ea.bwd(q, k, v, o, lse, to_dev(dout), cu_seqlens=cu, max_seqlen=N, causal=c["causal"],
                        scale=c["scale"])
    torch.cuda.synchronize()
    O_ref, L_ref = oracle.attention(inp["q"], inp["k"], inp["v"], inp["cu_seqlens"], c["causal"], c["scale"])
    O = o.float().cpu().numpy().astype(np.float64)
    L = lse.cpu().numpy().astype(np.float64)
    e = np.abs(O - O_ref)
    say(f"  fwd: O max {e.max():.3e} mean {e.mean():.3e} LSE max {np.abs(L - L_ref).max():.3e}")
    assert e.max() <= TOL_O_MAX and e.mean() <= TOL_O_MEAN and np.abs(L - L_ref).max() <= TOL_LSE
    from test_bwd_parity import check_grads
    check_grads(inp, dout, c["causal"], c["scale"], o, lse, (dq, dk, dv))


@pytest.mark.parametrize("i", range(N_CASES))
def test_block_sparse(i):
    import exact_attention_57_amd as ea
    c = draw_case(i)
    inp = workloads.make_custom_inputs(c["lengths"], c["H"], c["dims"][0], c["dims"][1], seed=c["seed"])
    torch, cu, N = _dev_run(c, inp)
    mask = workloads.make_block_mask(len(c["lengths"]), c["H"], N, c["density"], seed=c["seed"])
    say(f"case {i}: {c['lengths']} dims {c['dims']} causal {c['causal']} kept {mask.mean():.2f}")
    o, lse = ea.fwd(to_dev(inp["q"]), to_dev(inp["k"]), to_dev(inp["v"]), cu_seqlens=cu, max_seqlen=N,
                    causal=c["causal"], scale=c["scale"], block_mask=torch.from_numpy(mask).cuda())
    torch.cuda.synchronize()
    O_ref, L_ref = oracle.block_sparse_attention(inp["q"], inp["k"], inp["v"], inp["cu_seqlens"], c["causal"],
                                                 c["scale"], mask)
    O = o.float().cpu().numpy().astype(np.float64)
    L = lse.cpu().numpy().astype(np.float64)
    empty = np.isneginf(L_ref)
    assert np.array_equal(np.isneginf(L), empty)
    assert np.all(O.transpose(1, 0, 2)[empty] == 0.0)
    full = ~empty.T
    e = np.abs(O - O_ref)[full]
    if e.size:
        le = np.abs(L[~empty] - L_ref[~empty])
        say(f"  O max {e.max():.3e} mean {e.mean():.3e} LSE max {le.max():.3e}")
        assert e.max() <= TOL_O_MAX and e.mean() <= TOL_O_MEAN and le.max() <= TOL_LSE


@pytest.mark.parametrize("i", range(N_CASES))
def test_fp8(i):
    import test_fp8_parity as t8
    c = draw_case(i)
    inp = workloads.make_custom_inputs(c["lengths"], c["H"], c["dims"][0], c["dims"][1], seed=c["seed"])
    inp["causal"] = c["causal"]
    inp["scale"] = c["scale"]
    f = t8.fp8_inputs(inp, prescale=c["prescale"])
    say(f"case {i}: {c['lengths']} dims {c['dims']} causal {c['causal']} prescale {c['prescale']}")
    o, lse = t8.run_fp8(f, packed=True)
    t8.check(f, o, lse, f"random case {i}")
