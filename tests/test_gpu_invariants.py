"""GPU invariants and variant parity.

* closed forms: Q = 0 gives the mean of the visible V rows and LSE = ln(count);
  causal row 0 (and a single key) returns V exactly;
* determinism: two runs, the two schedules, and packed vs fixed-length
  launches of the same data are bitwise equal;
* conditional rescaling: threshold 0 is bitwise the always-rescale path and
  threshold 8 stays within tolerance of it (and of the oracle);
* software exp2 fractions stay within tolerance of the hardware-only path;
* out-of-bounds writes: guard regions around O and LSE are untouched;
* the optional statistics match closed forms (tiles, work items) and the
  oracle's tile-by-tile model (rescales considered and applied).
"""
import numpy as np
import pytest

import oracle
import workloads
from _gpu import TOL_O_MAX, TOL_O_MEAN, assert_close, lse_f64, o_f64, run, say, torch_cuda

pytestmark = pytest.mark.gpu


def ramp_inputs(lengths, H=4, d=128, seed=21, strength=13.255):
    """Packed inputs whose logits grow along each sequence (frequent max updates)."""
    wl = workloads.Workload("ramp_test", B=len(lengths), H=H, N=max(lengths), d_qk=d, d_v=d,
                            causal=True, varlen=True, ramp=True)
    inp = workloads.make_custom_inputs(lengths, H=H, d_qk=d, d_v=d, seed=seed)
    # add the same ramp the packed workload uses
    q = workloads.bf16_bits_to_f32(inp["q"]) + np.float32(strength / np.sqrt(d))
    k = workloads.bf16_bits_to_f32(inp["k"])
    cu = inp["cu_seqlens"]
    for b, L in enumerate(lengths):
        t = np.arange(L, dtype=np.float32) / max(L - 1, 1)
        k[cu[b]:cu[b + 1]] += (strength / np.sqrt(d) * t)[:, None, None].astype(np.float32)
    inp["q"] = workloads.f32_to_bf16_bits(q)
    inp["k"] = workloads.f32_to_bf16_bits(k)
    inp["causal"] = True
    inp["scale"] = 1.0 / np.sqrt(d)
    del wl
    return inp


def bits(t):
    torch = torch_cuda()
    return t.view(torch.int16).cpu().numpy() if t.dtype == torch.bfloat16 else t.cpu().numpy().view(np.uint32)


@pytest.mark.parametrize("causal", [False, True])
def test_zero_queries_closed_form(causal):
    lengths = [200, 77]
    inp = workloads.make_custom_inputs(lengths, H=2, d_qk=128, d_v=128, seed=31)
    inp["q"][:] = 0
    inp["causal"] = causal
    inp["scale"] = 0.7
    o, lse = run(inp, packed=True)
    v = workloads.bf16_bits_to_f32(inp["v"]).astype(np.float64)
    cu = inp["cu_seqlens"]
    O_ref = np.empty_like(v)
    L_ref = np.empty((2, cu[-1]))
    for b, L in enumerate(lengths):
        s, e = cu[b], cu[b + 1]
        if causal:
            O_ref[s:e] = np.cumsum(v[s:e], axis=0) / np.arange(1, L + 1)[:, None, None]
            L_ref[:, s:e] = np.log(np.arange(1, L + 1))[None]
        else:
            O_ref[s:e] = v[s:e].mean(axis=0, keepdims=True)
            L_ref[:, s:e] = np.log(L)
    assert_close(o_f64(o), lse_f64(lse), O_ref, L_ref, f"Q=0 causal={causal}")


@pytest.mark.parametrize("poly", [0, 4])
def test_causal_first_row_returns_v_exactly(poly):
    lengths = [130, 64, 1, 300]
    inp = workloads.make_custom_inputs(lengths, H=3, d_qk=192, d_v=128, seed=32)
    inp["causal"] = True
    inp["scale"] = 1 / np.sqrt(192)
    o, _ = run(inp, packed=True, poly_exp_sixteenths=poly)
    ob = bits(o)
    firsts = inp["cu_seqlens"][:-1]
    assert np.array_equal(ob[firsts], inp["v"][firsts].view(np.int16))


def test_runs_schedules_and_launch_forms_bitwise_equal():
    inp = workloads.make_custom_inputs([700, 700, 700], H=4, d_qk=128, d_v=128, seed=33)
    inp["causal"] = True
    inp["scale"] = 1 / np.sqrt(128)
    a = run(inp, packed=False)
    b = run(inp, packed=False)
    c = run(inp, packed=False, schedule=1)
    d = run(inp, packed=True)
    for other, what in ((b, "rerun"), (c, "natural schedule"), (d, "packed launch")):
        assert np.array_equal(bits(a[0]), bits(other[0])), what
        assert np.array_equal(bits(a[1]), bits(other[1])), what


def test_packed_equals_separate_fixed_length_runs():
    lengths = [256, 384, 128]
    inp = workloads.make_custom_inputs(lengths, H=2, d_qk=64, d_v=64, seed=34)
    inp["causal"] = True
    inp["scale"] = 0.125
    o, lse = run(inp, packed=True)
    cu = inp["cu_seqlens"]
    for b, L in enumerate(lengths):
        s, e = cu[b], cu[b + 1]
        sub = dict(q=inp["q"][s:e], k=inp["k"][s:e], v=inp["v"][s:e], cu_seqlens=np.array([0, L]),
                   lengths=np.array([L]), N=L, causal=True, scale=0.125)
        ob, lb = run(sub, packed=False)
        assert np.array_equal(bits(o)[s:e], bits(ob))
        assert np.array_equal(bits(lse)[:, s:e], bits(lb))


def test_threshold_zero_is_bitwise_always_rescale_and_eight_is_close():
    inp = ramp_inputs([1500, 700, 2048])
    o_always, l_always = run(inp, packed=True, rescale_threshold_log2=-1.0)
    o_zero, l_zero = run(inp, packed=True, rescale_threshold_log2=0.0)
    o_eight, l_eight = run(inp, packed=True, rescale_threshold_log2=8.0)
    assert np.array_equal(bits(o_always), bits(o_zero))
    assert np.array_equal(bits(l_always), bits(l_zero))
    assert_close(o_f64(o_eight), lse_f64(l_eight), o_f64(o_always), lse_f64(l_always),
                 "tau=8 vs always-rescale")
    O_ref, L_ref = oracle.attention(inp["q"], inp["k"], inp["v"], inp["cu_seqlens"], True, inp["scale"])
    assert_close(o_f64(o_eight), lse_f64(l_eight), O_ref, L_ref, "tau=8 vs oracle")
    assert_close(o_f64(o_always), lse_f64(l_always), O_ref, L_ref, "always vs oracle")


@pytest.mark.parametrize("poly", [2, 4, 8])
def test_software_exp2_fractions_close_to_hardware(poly):
    inp = ramp_inputs([1000, 333], seed=35)
    o0, l0 = run(inp, packed=True, poly_exp_sixteenths=0)
    o1, l1 = run(inp, packed=True, poly_exp_sixteenths=poly)
    assert_close(o_f64(o1), lse_f64(l1), o_f64(o0), lse_f64(l0), f"poly {poly}/16 vs hw")
    O_ref, L_ref = oracle.attention(inp["q"], inp["k"], inp["v"], inp["cu_seqlens"], True, inp["scale"])
    assert_close(o_f64(o1), lse_f64(l1), O_ref, L_ref, f"poly {poly}/16 vs oracle")


def test_guard_regions_untouched():
    torch = torch_cuda()
    import exact_attention_57_amd as ea
    from _gpu import to_dev
    lengths = [5, 129, 0, 67]
    H, d = 3, 128
    inp = workloads.make_custom_inputs(lengths, H=H, d_qk=d, d_v=d, seed=36)
    T = int(inp["cu_seqlens"][-1])
    guard = 4096
    obuf = torch.full((guard + T * H * d + guard,), -12345, dtype=torch.int16, device="cuda")
    lbuf = torch.full((guard + H * T + guard,), -7.25, dtype=torch.float32, device="cuda")
    o = obuf[guard:guard + T * H * d].view(torch.bfloat16).view(T, H, d)
    lse = lbuf[guard:guard + H * T].view(H, T)
    cu = torch.from_numpy(inp["cu_seqlens"]).cuda()
    for causal in (False, True):
        ea.fwd(to_dev(inp["q"]), to_dev(inp["k"]), to_dev(inp["v"]), o=o, lse=lse, cu_seqlens=cu,
               max_seqlen=max(lengths), causal=causal, scale=0.1)
        torch.cuda.synchronize()
        assert bool((obuf[:guard] == -12345).all()) and bool((obuf[-guard:] == -12345).all())
        assert bool((lbuf[:guard] == -7.25).all()) and bool((lbuf[-guard:] == -7.25).all())


def expected_counts(lengths, causal, H, d=128):
    """Closed forms for the statistics counters: wave-tiles computed, work items, and the
    number of (valid row, tile) pairs after each row's first tile, over H heads."""
    import exact_attention_57_amd as ea
    geo = ea.geometry(d, d)
    block_m, tile, rw = geo["rows_per_item"], geo["keys_per_tile"], geo["rows_per_wave"]
    waves = block_m // rw
    tiles = items = considered = 0
    for L in lengths:
        for q0 in range(0, L, block_m):
            items += 1
            kend = min(L, q0 + block_m) if causal else L
            nt = -(-kend // tile)
            for w in range(waves):
                qw0 = q0 + rw * w
                done = sum(1 for t in range(nt) if (not causal) or t * tile <= qw0 + rw - 1)
                tiles += done
                valid_rows = max(0, min(rw, L - qw0))
                considered += valid_rows * (done - 1)
    return tiles * H, items * H, considered * H


@pytest.mark.parametrize("causal", [False, True])
def test_statistics_match_closed_forms_and_oracle_model(causal):
    torch = torch_cuda()
    lengths = [1500, 700, 2048, 1]
    inp = ramp_inputs(lengths, seed=37)
    inp["causal"] = causal
    for tau in (8.0, 0.0, -1.0):
        stats = torch.zeros(4, dtype=torch.int64, device="cuda")
        run(inp, packed=True, rescale_threshold_log2=tau, stats=stats)
        st = stats.cpu().numpy()
        tiles, items, considered = expected_counts(lengths, causal, H=inp["H"])
        assert st[2] == tiles and st[3] == items and st[0] == considered, (st, tiles, items, considered)
        qf = workloads.bf16_bits_to_f32(inp["q"]).astype(np.float64)
        kf = workloads.bf16_bits_to_f32(inp["k"]).astype(np.float64)
        vf = workloads.bf16_bits_to_f32(inp["v"]).astype(np.float64)
        import exact_attention_57_amd as ea
        tile = ea.geometry(128, 128)["keys_per_tile"]
        _, _, ost = oracle.online_softmax_attention_f64(qf, kf, vf, inp["cu_seqlens"], causal,
                                                        inp["scale"], tau=tau, tile=tile)
        say(f"  tau={tau} causal={causal}: gpu taken {st[1]} / considered {st[0]}; "
            f"oracle model taken {ost['taken']} / {ost['considered']}")
        assert ost["considered"] == considered
        assert abs(int(st[1]) - ost["taken"]) <= max(3, 0.01 * ost["taken"])
