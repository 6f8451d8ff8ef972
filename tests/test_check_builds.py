"""The checking builds against the default build, through the C ABI.

* Race check (``libattn_racecheck.so``, ATTN_RACE_CHECK): every workgroup
  barrier first drains all of the wave's memory traffic (LDS DMAs and LDS
  reads) and is passed twice, so no tile transfer or LDS access overlaps a
  barrier.  A tile read before its DMA landed, or a buffer refilled while a
  wave still reads it, would give the default build different bits; so for
  every entry point (forward at all head-dim pairs with and without the
  causal mask, a software-exp2 share, block-sparse, FP8, backward) the outputs
  of both builds must be equal bit for bit on ragged packed inputs.
* Instrumented build (``libattn_stamps.so``, ATTN_STAMPS): the same outputs bit
  for bit, and its per-workgroup records must be complete and consistent with
  the work decomposition: every (head, sequence, query block) exactly once,
  tile-loop iterations equal to the closed form, start before end; the four
  counters stay zero (this build keeps only the records).
"""
import numpy as np
import pytest

import workloads
from _gpu import say, to_dev, torch_cuda

pytestmark = pytest.mark.gpu

LENGTHS = [1, 100, 0, 513, 256, 777]
STAMP_WORDS = 16


def bits(t):
    torch = torch_cuda()
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)


def same(a, b):
    torch = torch_cuda()
    return bool(torch.equal(bits(a), bits(b)))


def _inputs(dims, seed, H=3):
    torch = torch_cuda()
    inp = workloads.make_custom_inputs(LENGTHS, H=H, d_qk=dims[0], d_v=dims[1], seed=seed)
    cu = torch.from_numpy(inp["cu_seqlens"]).cuda()
    return inp, cu, max(LENGTHS)


@pytest.mark.parametrize("dims", [(64, 64), (128, 128), (192, 128)])
def test_race_check_forward_and_backward_bitwise(dims):
    torch = torch_cuda()
    import exact_attention_57_amd as ea
    rc = ea.check_build("racecheck")
    inp, cu, N = _inputs(dims, seed=80 + dims[0])
    q, k, v = to_dev(inp["q"]), to_dev(inp["k"]), to_dev(inp["v"])
    dout = to_dev(workloads.make_output_grad(inp, 3))
    scale = 1.0 / np.sqrt(dims[0])
    for causal in (False, True):
        for poly in (0, 4):
            say(f"case: race check fwd dims={dims} causal={causal} poly={poly}")
            a = ea.fwd(q, k, v, cu_seqlens=cu, max_seqlen=N, causal=causal, scale=scale, poly_exp_sixteenths=poly)
            b = ea.fwd(q, k, v, cu_seqlens=cu, max_seqlen=N, causal=causal, scale=scale, poly_exp_sixteenths=poly,
                       _lib=rc)
            torch.cuda.synchronize()
            assert same(a[0], b[0]) and same(a[1], b[1]), f"forward differs: causal={causal} poly={poly}"
        say(f"case: race check bwd dims={dims} causal={causal}")
        o, lse = ea.fwd(q, k, v, cu_seqlens=cu, max_seqlen=N, causal=causal, scale=scale)
        ga = ea.bwd(q, k, v, o, lse, dout, cu_seqlens=cu, max_seqlen=N, causal=causal, scale=scale)
        gb = ea.bwd(q, k, v, o, lse, dout, cu_seqlens=cu, max_seqlen=N, causal=causal, scale=scale, _lib=rc)
        torch.cuda.synchronize()
        for name, x, y in zip(("dq", "dk", "dv"), ga, gb):
            assert same(x, y), f"{name} differs: causal={causal}"


@pytest.mark.parametrize("dims", [(64, 64), (128, 128), (192, 128)])
def test_race_check_block_sparse_and_fp8_bitwise(dims):
    torch = torch_cuda()
    import exact_attention_57_amd as ea
    rc = ea.check_build("racecheck")
    inp, cu, N = _inputs(dims, seed=90 + dims[0])
    q, k, v = to_dev(inp["q"]), to_dev(inp["k"]), to_dev(inp["v"])
    mask = torch.from_numpy(workloads.make_block_mask(len(LENGTHS), 3, N, 0.5, seed=9)).cuda()
    f8 = workloads.make_fp8_inputs(inp, (2.0, 2.0, 2.0))
    q8, k8, v8 = (torch.from_numpy(f8[n]).cuda() for n in ("q8", "k8", "v8"))
    scale = 1.0 / np.sqrt(dims[0])
    for causal in (False, True):
        say(f"case: race check block-sparse and fp8 dims={dims} causal={causal}")
        a = ea.fwd(q, k, v, cu_seqlens=cu, max_seqlen=N, causal=causal, scale=scale, block_mask=mask)
        b = ea.fwd(q, k, v, cu_seqlens=cu, max_seqlen=N, causal=causal, scale=scale, block_mask=mask, _lib=rc)
        c = ea.fwd_fp8(q8, k8, v8, cu_seqlens=cu, max_seqlen=N, causal=causal, scale=scale, q_descale=0.5,
                       k_descale=0.5, v_descale=0.5)
        d = ea.fwd_fp8(q8, k8, v8, cu_seqlens=cu, max_seqlen=N, causal=causal, scale=scale, q_descale=0.5,
                       k_descale=0.5, v_descale=0.5, _lib=rc)
        torch.cuda.synchronize()
        assert same(a[0], b[0]) and same(a[1], b[1]), f"block-sparse differs: causal={causal}"
        assert same(c[0], d[0]) and same(c[1], d[1]), f"fp8 differs: causal={causal}"


@pytest.mark.parametrize("schedule", [0, 1])
@pytest.mark.parametrize("causal", [False, True])
def test_stamps_build_records(causal, schedule):
    torch = torch_cuda()
    import exact_attention_57_amd as ea
    st = ea.check_build("stamps")
    dims = (128, 128)
    inp, cu, N = _inputs(dims, seed=95, H=4)
    q, k, v = to_dev(inp["q"]), to_dev(inp["k"]), to_dev(inp["v"])
    geo = ea.geometry(*dims)
    rows, tile = geo["rows_per_item"], geo["keys_per_tile"]
    B, H = len(LENGTHS), 4
    nqb = -(-N // rows)
    W = B * H * nqb
    say(f"case: stamps causal={causal} schedule={schedule} W={W}")
    buf = torch.zeros(4 + STAMP_WORDS * W, dtype=torch.int64, device="cuda")
    a = ea.fwd(q, k, v, cu_seqlens=cu, max_seqlen=N, causal=causal, schedule=schedule)
    b = ea.fwd(q, k, v, cu_seqlens=cu, max_seqlen=N, causal=causal, schedule=schedule, stats=buf, _lib=st)
    torch.cuda.synchronize()
    assert same(a[0], b[0]) and same(a[1], b[1])
    rec = buf[4:].cpu().numpy().view(np.uint64).reshape(W, STAMP_WORDS)
    assert np.all(rec[:, 1] >= rec[:, 0]) and np.all(rec[:, 0] > 0)
    items = {(int(x) >> 40, (int(x) >> 20) & 0xFFFFF, int(x) & 0xFFFFF): i for i, x in enumerate(rec[:, 3])}
    assert len(items) == W, "every (head, sequence, query block) exactly once"
    for (h, bb, qb), i in items.items():
        L = LENGTHS[bb]
        q0 = qb * rows
        if q0 >= L:
            assert rec[i, 4] == 0
            continue
        kend = min(L, q0 + rows) if causal else L
        assert rec[i, 4] == -(-kend // tile) + 1, (h, bb, qb, rec[i, 4])
        assert rec[i, 6] > 0 and rec[i, 8] > 0 and rec[i, 12] > 0        # loop, matrix phases of waves 0 and 4
    xcc = (rec[:, 2] >> np.uint64(32)).astype(np.int64)
    assert np.all((xcc >= 0) & (xcc < 8))
    say(f"  XCC id = workgroup index mod 8 for {np.mean(xcc == np.arange(W) % 8):.3f} of the workgroups")
    assert not buf[:4].any(), "the instrumented build keeps no counters"
