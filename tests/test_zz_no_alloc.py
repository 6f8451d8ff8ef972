"""The allocation-free backward entry point (attn_bwd_noalloc) through the C ABI.

Its D workspace is the library's static scratch array instead of a caller
buffer; the kernels are attn_bwd's.  Two calls in a row on one GPU, the
second smaller than the first (so a stale first-call D in the shared array
would be read if the second call's D pass missed a row): each call's dq, dk,
dv must equal attn_bwd's on the same inputs bit for bit, and lie within the
derived per-element bound of the fp64 gradient oracle.
"""
import numpy as np
import pytest

import workloads
from _gpu import say, to_dev, torch_cuda

pytestmark = pytest.mark.gpu

CALLS = [   # lengths, H, d_qk, d_v, causal
    ([700, 333, 1, 129], 4, 128, 128, True),
    ([100, 17], 2, 64, 64, False),
    ([300, 65], 3, 192, 128, True),
]


def _one(ea, torch, lengths, H, d_qk, d_v, causal, seed):
    from test_bwd_parity import check_grads
    inp = workloads.make_custom_inputs(lengths, H, d_qk, d_v, seed=seed)
    cu = torch.from_numpy(inp["cu_seqlens"]).cuda()
    N = max(lengths)
    scale = 1.0 / np.sqrt(d_qk)
    q, k, v = to_dev(inp["q"]), to_dev(inp["k"]), to_dev(inp["v"])
    dout_bits = workloads.make_output_grad(inp, seed)
    dout = to_dev(dout_bits)
    o, lse = ea.fwd(q, k, v, cu_seqlens=cu, max_seqlen=N, causal=causal, scale=scale)
    ref = ea.bwd(q, k, v, o, lse, dout, cu_seqlens=cu, max_seqlen=N, causal=causal, scale=scale)
    got = tuple(torch.empty_like(t) for t in (q, k, v))
    ea.bwd_noalloc(q, k, v, o, lse, dout, *got, cu_seqlens=cu, max_seqlen=N, causal=causal, scale=scale)
    torch.cuda.synchronize()
    for name, a, b in zip(("dq", "dk", "dv"), ref, got):
        assert torch.equal(a.view(torch.int16), b.view(torch.int16)), f"{name}: attn_bwd_noalloc != attn_bwd"
    check_grads(inp, dout_bits, causal, scale, o, lse, got)


def test_noalloc_matches_attn_bwd_on_consecutive_calls():
    torch = torch_cuda()
    import exact_attention_57_amd as ea
    for i, (lengths, H, d_qk, d_v, causal) in enumerate(CALLS):
        say(f"case: noalloc call {i}: lengths {lengths} H={H} d=({d_qk},{d_v}) causal={causal}")
        _one(ea, torch, lengths, H, d_qk, d_v, causal, seed=110 + i)


def test_noalloc_rejects_beyond_scratch_before_any_work():
    torch = torch_cuda()
    import exact_attention_57_amd as ea
    st = ea.bwd_noalloc_raw(1 << 16, 1 << 16, 1 << 16, 1 << 16, 1 << 16, 1 << 16, 1 << 16, 1 << 16, 1 << 16, None,
                            1, 1, ea.NOALLOC_MAX_ROWS + 1, 64, 64, 0.125, 0, None)
    torch.cuda.synchronize()
    assert st == ea.ATTN_ERR_SCRATCH
