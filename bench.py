#!/usr/bin/env python3
"""Benchmark of the fused attention forward pass on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload KEY]
                    [--tau 8.0] [--poly 0] [--schedule 0|1] [--no-cpu-baseline]
                    [--bwd] [--block-density D] [--fp8] [--stamps] [--stats]
    python bench.py --ramp N | --gemm-ceiling N | --copy-calibration MIB

A step is one call of attn_fwd over the whole workload (all query blocks of
all heads and sequences).  Default workload: non-causal B=4 H=16 N=4096
d=128 (bf16 inputs, fp32 accumulation).  Inputs are seeded synthetic bf16
draws resident in HBM before timing starts.

Printed (one JSON line on stdout):
  value      whole-job TFLOP/s = algorithmic FLOP * K / wall time of the K steps
             (bracketed by device synchronisations)
  roofline   the kernel's per-launch average duration from HIP events recorded
             on the launch stream over the timed region; achieved TFLOP/s
             against the dense bf16 MFMA peak; HBM traffic per launch from
             committed rocprofv3 counter summaries when they match the current
             kernel source, else null
  cpu_baseline  the fp64 CPU oracle timed on a bounded sample of the same
             workload (whole (sequence, head) pairs until ~10 s have elapsed),
             scaled to TFLOP/s with the same FLOP convention

FLOP convention: 4*B*H*N^2*d (non-causal, d_qk = d_v = d), 2*B*H*N^2*(d_qk+d_v)
in general, halved when causal; packed sequences sum the per-sequence counts.

--bwd times the backward pass (attn_bwd: the D pass, the dK/dV kernel and the
dQ kernel) instead, on the forward's o and lse and a seeded dO; its
algorithmic FLOP are 2.5x the forward's (five products of the forward's
size: S, dP, dV, dK, dQ; the kernels recompute S and dP once more, seven
products in all).

--block-density D runs the block-sparse forward pass with a seeded random
128 x 128 block mask keeping each block with probability D; its algorithmic
FLOP count only the kept blocks, clipped to the sequences (under the causal
mask a diagonal block counts half and a block above the diagonal nothing, so
an all-ones mask counts exactly the dense figure).

--fp8 runs the FP8 forward pass (attn_fwd_fp8) on the same draws rounded to
E4M3 (descales 1); same FLOP convention, roofline against the dense FP8
MFMA peak (5.0 PFLOP/s), with the percentage of the bf16 peak alongside.

--stamps times the instrumented build of the bf16 forward pass
(libattn_stamps.so: the same kernels plus per-workgroup clock stamps), then
runs it ~50 ms more with a record buffer and adds a "stamps" summary of the
last launch: the XCD each workgroup ran on against its grid index, per-XCD
and per-CU busy time and last finish, workgroups per CU and the gaps between
them, the finish-time tail (last workgroup end minus the median end), the
start order against the grid index and against the work per item, and the
shader cycles per tile iteration of each phase (matrix, barrier, softmax,
barrier) for one wave of each ping-pong group.

--ramp N only times the first N launches of the instrumented bf16 forward in
this process one by one, and reads the shader clock and cycles per workgroup
of selected launches from their records (the clock dip of the first launches).
--gemm-ceiling N only times the vendor bf16 GEMM (torch.matmul, N^3);
--copy-calibration MIB only runs a plain copy kernel over MIB MiB, for scaling
the FETCH_SIZE / WRITE_SIZE counters.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6      # MI355X dense bf16 MFMA: 256 CU x 4096 flop/clk x 2.4 GHz
PEAK_FP8_TFLOPS = 5033.2       # MI355X dense fp8 MFMA: 256 CU x 8192 flop/clk x 2.4 GHz
HBM_PEAK_GBS = 8000.0
DEFAULT_WORKLOAD = "noncausal_b4h16n4096d128"
KERNEL_SOURCES = {   # sources whose hash keys a stored traffic record, per kernel family
    "bf16": ["exact_attention_57_amd/csrc/attn_fwd_kernel.hip", "exact_attention_57_amd/csrc/attn_fwd_common.h"],
    "fp8": ["exact_attention_57_amd/csrc/attn_fwd_fp8_kernel.hip", "exact_attention_57_amd/csrc/attn_fwd_common.h"],
}
BWD_FLOP_FACTOR = 2.5          # backward algorithmic FLOP / forward (5 products vs 2)


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def algorithmic_flops(lengths, H, d_qk, d_v, causal) -> float:
    tot = 0.0
    for L in lengths:
        f = 2.0 * H * float(L) * float(L) * (d_qk + d_v)
        tot += f / 2 if causal else f
    return tot


def block_sparse_flops(lengths, H, d_qk, d_v, causal, mask) -> float:
    """Algorithmic FLOP of the kept 128 x 128 blocks (mask [B, H, nb, nb])."""
    import numpy as np
    tot = 0.0
    for b, L in enumerate(lengths):
        nb = (L + 127) // 128
        if nb == 0:
            continue
        size = np.minimum(128, L - 128 * np.arange(nb)).astype(np.float64)      # rows (keys) per block
        pair = np.outer(size, size)
        if causal:
            pair = np.tril(pair, -1) + np.diag(np.diag(pair)) / 2.0
        kept = mask[b, :, :nb, :nb].astype(np.float64)                           # [H, nb, nb]
        tot += 2.0 * (d_qk + d_v) * float((kept * pair[None]).sum())
    return tot


def compulsory_bytes(T, H, d_qk, d_v) -> float:
    """Read Q, K, V once, write O (bf16) and LSE (fp32) once."""
    return T * H * (2 * d_qk * 2 + d_v * 2 + d_v * 2 + 4)


def kernel_source_hash(family: str = "bf16") -> str:
    """sha256[:16] of the kernel sources with comments and blank lines removed,
    so that a change of wording leaves the traffic records valid."""
    import re
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES[family]:
        with open(os.path.join(ROOT, rel)) as f:
            text = f.read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        lines = [re.sub(r"//.*$", "", line).rstrip() for line in text.splitlines()]
        h.update("\n".join(line for line in lines if line).encode())
    return h.hexdigest()[:16]


def load_traffic(workload: str, variant: str):
    """HBM bytes per launch from profiles/traffic_<workload>.json, if the kernel is unchanged."""
    name = f"traffic_{workload}" + ("_fp8" if variant == "fp8" else "")
    path = os.path.join(ROOT, "profiles", name + ".json")
    if not os.path.exists(path):
        return None
    try:
        rec = json.load(open(path))
    except (OSError, ValueError):
        return None
    family = "fp8" if variant == "fp8" else "bf16"
    if rec.get("kernel_source_sha256_16") != kernel_source_hash(family) or rec.get("variant") != variant:
        return None
    return rec.get("hbm_bytes_per_launch")


def cpu_baseline(inp, budget_s: float = 10.0, backward_dout=None, block_mask=None, fp8=None) -> dict:
    """Time the fp64 oracle on whole (sequence, head) pairs until the budget is
    spent (the gradient oracle when ``backward_dout`` is given)."""
    import numpy as np
    import oracle
    blas = "unknown"
    try:
        from threadpoolctl import threadpool_info
        info = threadpool_info()
        threads = max([p.get("num_threads", 1) for p in info] or [1])
        blas = ", ".join(sorted({f"{p.get('internal_api')} {p.get('version')}" for p in info if p.get("user_api") == "blas"})) or blas
    except Exception:  # pragma: no cover - threadpoolctl is optional
        threads = os.cpu_count() or 1
    cu = inp["cu_seqlens"]
    H = inp["H"]
    pairs = [(b, h) for b in range(len(cu) - 1) for h in range(H) if cu[b + 1] > cu[b]]
    rng = np.random.default_rng(0)
    order = rng.permutation(len(pairs))
    done_flops = 0.0
    n = 0
    t0 = time.perf_counter()
    for idx in order:
        b, h = pairs[idx]
        s, e = int(cu[b]), int(cu[b + 1])
        sub_cu = np.array([0, e - s])
        if fp8 is not None:
            oracle.attention_fp8(fp8["q8"][s:e, h:h + 1], fp8["k8"][s:e, h:h + 1], fp8["v8"][s:e, h:h + 1],
                                 sub_cu, inp["causal"], inp["scale"])
            done_flops += algorithmic_flops([e - s], 1, inp["d_qk"], inp["d_v"], inp["causal"])
        elif block_mask is not None:
            oracle.block_sparse_attention(inp["q"][s:e, h:h + 1], inp["k"][s:e, h:h + 1], inp["v"][s:e, h:h + 1],
                                          sub_cu, inp["causal"], inp["scale"],
                                          np.ascontiguousarray(block_mask[b:b + 1, h:h + 1]))
            done_flops += block_sparse_flops([e - s], 1, inp["d_qk"], inp["d_v"], inp["causal"],
                                             block_mask[b:b + 1, h:h + 1])
        elif backward_dout is None:
            oracle.attention(inp["q"][s:e, h:h + 1], inp["k"][s:e, h:h + 1], inp["v"][s:e, h:h + 1],
                             sub_cu, inp["causal"], inp["scale"])
            done_flops += algorithmic_flops([e - s], 1, inp["d_qk"], inp["d_v"], inp["causal"])
        else:
            oracle.attention_backward(inp["q"][s:e, h:h + 1], inp["k"][s:e, h:h + 1], inp["v"][s:e, h:h + 1],
                                      backward_dout[s:e, h:h + 1], sub_cu, inp["causal"], inp["scale"])
            done_flops += BWD_FLOP_FACTOR * algorithmic_flops([e - s], 1, inp["d_qk"], inp["d_v"], inp["causal"])
        n += 1
        if time.perf_counter() - t0 >= budget_s:
            break
    dt = time.perf_counter() - t0
    return {"value": done_flops / dt / 1e12, "unit": "TFLOP/s", "cores": int(threads),
            "kind": "oracle",
            "sample": f"{n} of {len(pairs)} (sequence, head) pairs, fp64 NumPy/BLAS, {dt:.1f} s",
            "seconds": round(dt, 3), "cpu": _cpu_model(), "blas": blas, "host_cpus": os.cpu_count()}


STAMP_WORDS = 16              # uint64 per workgroup record of the instrumented build
REALTIME_HZ = 100e6           # s_memrealtime rate


def stamp_summary(ea, q, k, v, o, lse, cu, inp, wl, args, bmask_dev, stream, fwd_lib, kernel_ms) -> dict:
    """The last of about 50 ms of launches of the instrumented build with a record buffer, summarised.

    Record words (per workgroup, at its linear grid index): [0] real-time clock
    at entry, [1] at the end, [2] (XCC id << 32) | HW_ID, [3] work item, [4]
    tile-loop iterations, [5..7] shader cycles of the prologue, the loop and
    the epilogue (wave 0), [8..11] wave 0's loop cycles in its matrix phases,
    the barrier after them, its softmax phases and the barrier after those,
    [12..15] the same for wave 4."""
    import numpy as np
    import torch
    geo = ea.geometry(wl.d_qk, wl.d_v)
    nqb = -(-inp["N"] // geo["rows_per_item"])
    W = inp["B"] * inp["H"] * nqb
    buf = torch.zeros(4 + STAMP_WORDS * W, dtype=torch.int64, device="cuda")
    def launch():
        ea.fwd(q, k, v, o=o, lse=lse, cu_seqlens=cu, max_seqlen=inp["N"], causal=wl.causal, scale=inp["scale"],
               rescale_threshold_log2=args.tau, poly_exp_sixteenths=args.poly, schedule=args.schedule,
               block_mask=bmask_dev, stats=buf, stream=stream, _lib=fwd_lib)
    # about 50 ms of launches back to back (each overwrites the records), so that
    # the recorded last one runs at the clock of the timed launches, not at the
    # lower one the chip drops to after an idle gap; the last launch starts
    # after the one before it has ended, so its span covers it alone
    for _ in range(max(5, min(200, int(50.0 / max(kernel_ms, 1e-3))))):
        launch()
    torch.cuda.synchronize()
    launch()
    torch.cuda.synchronize()
    r = buf[4:].cpu().numpy().view(np.uint64).reshape(W, STAMP_WORDS).astype(np.float64)
    ran = r[:, 4] > 0                                        # workgroups with a query block to compute
    t0 = r[:, 0].min()
    start = (r[:, 0] - t0) / REALTIME_HZ * 1e6               # us
    end = (r[:, 1] - t0) / REALTIME_HZ * 1e6
    span = float(end.max())
    hw = buf[4:].cpu().numpy().view(np.uint64).reshape(W, STAMP_WORDS)[:, 2]
    xcc = (hw >> np.uint64(32)).astype(np.int64)
    cu_key = xcc * 256 + ((hw >> np.uint64(8)) & np.uint64(0xff)).astype(np.int64)   # XCC, SE, SH, CU
    ids = np.arange(W)
    dur = end - start
    per_cu, cu_last, cu_n = {}, {}, {}
    for key, d, e in zip(cu_key[ran], dur[ran], end[ran]):
        per_cu[key] = per_cu.get(key, 0.0) + d
        cu_last[key] = max(cu_last.get(key, 0.0), e)
        cu_n[key] = cu_n.get(key, 0) + 1
    cu_busy = np.array(list(per_cu.values()))
    cu_end = np.array(list(cu_last.values()))
    cu_count = np.array(list(cu_n.values()))
    # idle time on a CU between one workgroup's end stamp and the next one's start stamp
    gaps, first_start = [], []
    for key in per_cu:
        sel = ran & (cu_key == key)
        order = np.argsort(start[sel])
        st_, en_ = start[sel][order], end[sel][order]
        first_start.append(st_[0])
        gaps.extend((st_[1:] - en_[:-1]).tolist())
    gaps = np.array(gaps) if gaps else np.zeros(1)
    xcds = {}
    for x in range(8):
        sel = ran & (xcc == x)
        if sel.any():
            xcds[str(x)] = {"workgroups": int(sel.sum()), "first_start_us": round(float(start[sel].min()), 2),
                            "last_end_us": round(float(end[sel].max()), 2),
                            "busy_us": round(float(dur[sel].sum()), 1)}
    e_ran = np.sort(end[ran])
    iters = r[ran, 4]
    loop = r[ran, 6]
    ph = r[ran, 8:16] / iters[:, None]                       # cycles per loop iteration
    cyc = r[ran, 5] + r[ran, 6] + r[ran, 7]
    clock_ghz = cyc / np.maximum((r[ran, 1] - r[ran, 0]) / REALTIME_HZ, 1e-12) / 1e9

    def rank_corr(a, b):
        ra, rb = np.argsort(np.argsort(a)), np.argsort(np.argsort(b))
        return float(np.corrcoef(ra, rb)[0, 1]) if len(a) > 2 else None

    # longest first: within each XCD, do workgroups with more tile iterations start earlier?
    lf = [rank_corr(start[ran & (xcc == x)], r[ran & (xcc == x), 4]) for x in range(8)
          if (ran & (xcc == x)).sum() > 2 and np.ptp(r[ran & (xcc == x), 4]) > 0]
    names = ["matrix", "barrier_after_matrix", "softmax", "barrier_after_softmax"]
    return {
        "workgroups": int(W), "workgroups_with_work": int(ran.sum()),
        "kernel_ms_instrumented": round(kernel_ms, 4),
        "span_us": round(span, 1),
        "xcc_equals_index_mod_8": round(float(np.mean(xcc == ids % 8)), 4),
        "per_xcd": xcds,
        "cus_used": int(len(per_cu)),
        "cu_busy_us": {"max": round(float(cu_busy.max()), 1), "mean": round(float(cu_busy.mean()), 1),
                       "min": round(float(cu_busy.min()), 1)},
        "workgroups_per_cu": {"min": int(cu_count.min()), "max": int(cu_count.max())},
        "cu_first_start_us": {"median": round(float(np.median(first_start)), 2),
                              "max": round(float(np.max(first_start)), 2)},
        "gap_between_workgroups_us": {"median": round(float(np.median(gaps)), 2),
                                      "p90": round(float(np.percentile(gaps, 90)), 2),
                                      "max": round(float(gaps.max()), 2)},
        # when each compute unit finished its last workgroup: a balanced schedule keeps these close
        "cu_last_end_us": {"min": round(float(cu_end.min()), 1), "median": round(float(np.median(cu_end)), 1),
                           "max": round(float(cu_end.max()), 1)},
        "finish_us": {"median": round(float(np.median(e_ran)), 1), "last": round(float(e_ran[-1]), 1),
                      "tail_last_minus_median": round(float(e_ran[-1] - np.median(e_ran)), 1),
                      "p90": round(float(np.percentile(e_ran, 90)), 1)},
        "start_order_vs_index_rank_corr": rank_corr(start[ran], ids[ran]),
        "start_vs_tiles_rank_corr_per_xcd": [round(x, 3) for x in lf] if lf else None,
        "workgroup_us": {"median": round(float(np.median(dur[ran])), 2), "max": round(float(dur[ran].max()), 2)},
        "tile_iterations": {"median": float(np.median(iters)), "max": float(iters.max())},
        "cycles_per_iteration": {
            "wave0_group0": {n: round(float(np.mean(ph[:, i])), 1) for i, n in enumerate(names)},
            "wave4_group1": {n: round(float(np.mean(ph[:, 4 + i])), 1) for i, n in enumerate(names)},
            "loop_total": round(float(np.mean(loop / iters)), 1),
        },
        "cycles_per_workgroup": {"prologue": round(float(np.mean(r[ran, 5])), 0),
                                 "loop": round(float(np.mean(loop)), 0),
                                 "epilogue": round(float(np.mean(r[ran, 7])), 0)},
        "shader_clock_ghz": {"median": round(float(np.median(clock_ghz)), 3)},
    }


def _cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    # in a fresh process the chip's clock dips to ~1.3 GHz around launches 5-10
    # of this kernel and recovers after ~30 (--ramp shows it); 100 untimed
    # warm-up launches get past the dip
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--tau", type=float, default=8.0, help="rescale threshold (log2); <0 = always")
    ap.add_argument("--poly", type=int, default=0, help="sixteenths of exps on the software exp2")
    ap.add_argument("--schedule", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--stats", action="store_true",
                    help="after timing, run one launch with the kernel's counters and report the rescale "
                         "skip rate and tile counts")
    ap.add_argument("--cpu-budget", type=float, default=10.0)
    ap.add_argument("--bwd", action="store_true", help="time the backward pass (attn_bwd) instead")
    ap.add_argument("--block-density", type=float, default=None,
                    help="block-sparse forward with a seeded random 128x128 block mask of this density")
    ap.add_argument("--block-aligned", action="store_true",
                    help="with --block-density: query-block rows 2i+1 copy rows 2i (the 256-row work items "
                         "then keep exactly the drawn fraction of key tiles)")
    ap.add_argument("--fp8", action="store_true", help="time the FP8 (E4M3) forward pass (attn_fwd_fp8)")
    ap.add_argument("--stamps", action="store_true",
                    help="time the instrumented build (libattn_stamps.so) of the bf16 forward pass and summarise "
                         "its per-workgroup records: dispatch order, XCD mapping, per-CU balance, finish tail, "
                         "cycles per phase")
    ap.add_argument("--ramp", type=int, default=0, metavar="N",
                    help="only time the first N launches of the bf16 forward pass in this process one by one "
                         "(instrumented build, no warm-up) and report, for some of them, the shader clock and the "
                         "cycles per workgroup from the per-workgroup records")
    ap.add_argument("--gemm-ceiling", type=int, default=0, metavar="N",
                    help="only time the vendor library's bf16 GEMM (torch.matmul, N x N x N, fp32 accumulation) "
                         "with --warmup and --steps launches, as a practical matrix-core ceiling on this chip")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain elementwise copy kernel (negation) over MIB MiB 5 times "
                         "(for scaling FETCH_SIZE/WRITE_SIZE counters) and print the byte counts")
    args = ap.parse_args()
    if args.stats and (args.bwd or args.fp8):
        raise SystemExit("--stats reads the bf16 forward kernel's counters; the backward and FP8 entry points have none")

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures the single-GPU kernel only: the attention forward pass shards "
              "over (sequence, head) pairs with no exchange, so run it with --gpus 1 "
              f"(got --gpus {args.gpus}, WORLD_SIZE={world}).", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    if args.gemm_ceiling:
        n = args.gemm_ceiling
        gen = torch.Generator(device="cuda").manual_seed(0)
        a = torch.randn(n, n, dtype=torch.bfloat16, device="cuda", generator=gen)
        b = torch.randn(n, n, dtype=torch.bfloat16, device="cuda", generator=gen)
        c = torch.empty(n, n, dtype=torch.bfloat16, device="cuda")
        for _ in range(args.warmup):
            torch.matmul(a, b, out=c)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(args.steps):
            torch.matmul(a, b, out=c)
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / args.steps
        tf = 2.0 * n ** 3 / (ms * 1e-3) / 1e12
        print(json.dumps({"gemm_ceiling": f"torch.matmul bf16 {n}x{n}x{n}", "steps": args.steps,
                          "warmup": args.warmup, "kernel_ms": round(ms, 4), "tflops": round(tf, 1),
                          "pct_of_dense_bf16_peak": round(100 * tf / PEAK_BF16_TFLOPS, 2)}), flush=True)
        return

    if args.copy_calibration:
        n = args.copy_calibration << 20
        src = torch.ones(n // 2, dtype=torch.bfloat16, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(5):
            torch.neg(src, out=dst)     # one elementwise kernel: reads n bytes, writes n bytes
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes_read": n, "copy_calibration_bytes_written": n,
                          "launches": 5}), flush=True)
        return

    import exact_attention_57_amd as ea
    import workloads

    wl = workloads.workload(args.workload)
    log(f"bench: drawing inputs for {wl.key}")
    inp = workloads.make_inputs(wl, seed=0)
    T, H = inp["T"], inp["H"]
    lengths = [int(x) for x in inp["lengths"]]
    flops = algorithmic_flops(lengths, H, wl.d_qk, wl.d_v, wl.causal)

    def dev(bits):
        return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).cuda()

    q, k, v = dev(inp["q"]), dev(inp["k"]), dev(inp["v"])
    cu = torch.from_numpy(inp["cu_seqlens"]).cuda() if wl.varlen else None
    o = torch.empty((T, H, wl.d_v), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((H, T), dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()

    bmask = bmask_dev = None
    if args.block_density is not None:
        if args.bwd:
            raise SystemExit("--block-density applies to the forward pass")
        bmask = workloads.make_block_mask(inp["B"], H, inp["N"], args.block_density, seed=0)
        if args.block_aligned:
            bmask[:, :, 1::2, :] = bmask[:, :, 0:bmask.shape[2] // 2 * 2:2, :]
        bmask_dev = torch.from_numpy(bmask).cuda()
        flops = block_sparse_flops(lengths, H, wl.d_qk, wl.d_v, wl.causal, bmask)

    fwd_lib = None
    if args.stamps:
        if args.bwd or args.fp8:
            raise SystemExit("--stamps instruments the bf16 forward pass")
        fwd_lib = ea.check_build("stamps")

    def step():
        ea.fwd(q, k, v, o=o, lse=lse, cu_seqlens=cu, max_seqlen=inp["N"], causal=wl.causal,
               scale=inp["scale"], rescale_threshold_log2=args.tau,
               poly_exp_sixteenths=args.poly, schedule=args.schedule, block_mask=bmask_dev, stream=stream,
               _lib=fwd_lib)

    if args.ramp:
        if args.bwd or args.fp8 or args.block_density is not None:
            raise SystemExit("--ramp follows the dense bf16 forward pass")
        st_lib = ea.check_build("stamps")
        geo = ea.geometry(wl.d_qk, wl.d_v)
        W = inp["B"] * H * (-(-inp["N"] // geo["rows_per_item"]))
        n = args.ramp
        rec_at = [i for i in (1, 2, 3, 4, 5, 6, 8, 10, 15, 20, 25, 30, 40, 60, 80, 120, 160, 200, 300, 400) if i <= n]
        bufs = {i: torch.zeros(4 + STAMP_WORDS * W, dtype=torch.int64, device="cuda") for i in rec_at}
        torch.cuda.synchronize()
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(n + 1)]
        evs[0].record(stream)
        for i in range(1, n + 1):
            ea.fwd(q, k, v, o=o, lse=lse, cu_seqlens=cu, max_seqlen=inp["N"], causal=wl.causal,
                   scale=inp["scale"], rescale_threshold_log2=args.tau, poly_exp_sixteenths=args.poly,
                   schedule=args.schedule, stats=bufs.get(i), stream=stream, _lib=st_lib)
            evs[i].record(stream)
        torch.cuda.synchronize()
        ms = [evs[i - 1].elapsed_time(evs[i]) for i in range(1, n + 1)]
        recs = {}
        for i in rec_at:
            r = bufs[i][4:].cpu().numpy().view(np.uint64).reshape(W, STAMP_WORDS).astype(np.float64)
            ran = r[:, 4] > 0
            cyc = r[ran, 5] + r[ran, 6] + r[ran, 7]
            dur = (r[ran, 1] - r[ran, 0]) / REALTIME_HZ
            recs[str(i)] = {"ms": round(ms[i - 1], 4), "cycles_per_workgroup": int(np.median(cyc)),
                            "shader_clock_ghz": round(float(np.median(cyc / dur)) / 1e9, 3)}
        win = ms[5:25]                            # the launches a run with 5 warm-ups and 20 timed steps times
        print(json.dumps({"ramp": wl.key, "launches": n, "ms_per_launch": [round(x, 4) for x in ms],
                          "recorded": recs,
                          "mean_ms_launches_6_to_25": round(sum(win) / len(win), 4) if len(win) == 20 else None,
                          "mean_ms_last_20": round(sum(ms[-20:]) / 20, 4) if n >= 20 else None,
                          "flop_per_launch": flops}), flush=True)
        return

    f8 = None
    if args.fp8:
        if args.bwd or args.block_density is not None:
            raise SystemExit("--fp8 times the dense forward pass only")
        f8 = workloads.make_fp8_inputs(inp)
        q8, k8, v8 = (torch.from_numpy(f8[n]).cuda() for n in ("q8", "k8", "v8"))

        def step():                              # noqa: F811 - the FP8 step replaces the bf16 one
            ea.fwd_fp8(q8, k8, v8, o=o, lse=lse, cu_seqlens=cu, max_seqlen=inp["N"], causal=wl.causal,
                       scale=inp["scale"], stream=stream)

    if args.bwd:
        step()                                   # o and lse for the backward pass
        dout_bits = workloads.make_output_grad(inp, 0)
        dout = dev(dout_bits)
        dq, dk, dvv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
        delta = torch.empty(H * inp["B"] * inp["N"], dtype=torch.float32, device="cuda")
        flops = BWD_FLOP_FACTOR * flops

        def step():                              # noqa: F811 - the backward step replaces the forward one
            ea.bwd(q, k, v, o, lse, dout, cu_seqlens=cu, max_seqlen=inp["N"], causal=wl.causal,
                   scale=inp["scale"], dq=dq, dk=dk, dv=dvv, delta=delta, stream=stream)

    log(f"bench: warmup {args.warmup}")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    log(f"bench: timing {args.steps} steps")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(args.steps):
        step()
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ev_ms = ev0.elapsed_time(ev1) / args.steps

    # per-launch spread, in a separate pass after the timed region (the events
    # between launches would otherwise sit inside it)
    n_each = min(args.steps, 100)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n_each)]
    for e0, e1 in evs:
        e0.record(stream)
        step()
        e1.record(stream)
    torch.cuda.synchronize()
    each = sorted(e0.elapsed_time(e1) for e0, e1 in evs)
    launch_ms = {"median": round(each[len(each) // 2], 4), "min": round(each[0], 4),
                 "max": round(each[-1], 4), "launches": n_each}

    value = flops * args.steps / wall / 1e12
    achieved = flops / (ev_ms * 1e-3) / 1e12
    variant = "bwd" if args.bwd else "fp8" if args.fp8 else f"tau={args.tau},poly={args.poly},schedule={args.schedule}"
    if bmask is not None:
        variant += f",block_density={args.block_density}" + (",aligned" if args.block_aligned else "")
    traffic = None if args.bwd or bmask is not None else load_traffic(wl.key, variant)
    out = {
        "metric": ("attention bwd" if args.bwd else "attention fwd (FP8 E4M3 inputs)" if args.fp8
                   else "attention fwd" if bmask is None else "block-sparse attention fwd")
                  + " TFLOP/s and % of BF16 MFMA peak on 1 MI355X"
                  + (f", d={wl.d_qk}" if wl.d_qk == wl.d_v else f", d_qk={wl.d_qk} d_v={wl.d_v}"),
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall * 1e3 / args.steps, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8e4m3" if args.fp8 else "bf16",
        "data": "synthetic",
        "pct_of_peak": round(100.0 * value / PEAK_BF16_TFLOPS, 2),
        "config": {"workload": wl.key, "B": wl.B, "H": H, "N": inp["N"], "T": T,
                   "d_qk": wl.d_qk, "d_v": wl.d_v, "causal": wl.causal,
                   "packed": wl.varlen, "variant": variant, "flop_per_step": flops},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                     "traffic": traffic, "kernel_ms": round(ev_ms, 4), "launch_ms": launch_ms,
                     "compulsory_bytes": compulsory_bytes(T, H, wl.d_qk, wl.d_v)},
    }
    if args.fp8:
        out["roofline"]["peak"] = PEAK_FP8_TFLOPS
        out["roofline"]["frac"] = round(achieved / PEAK_FP8_TFLOPS, 4)
        out["roofline"]["compulsory_bytes"] = T * H * (2 * wl.d_qk + wl.d_v + 2 * wl.d_v + 4)
    if bmask is not None:
        out["config"]["kept_blocks"] = round(float(bmask.mean()), 4)
    if args.bwd:
        out["roofline"]["note"] = "kernel_ms spans the D pass, the dK/dV kernel and the dQ kernel"
        # read q, k, v, o, dO, lse; write dq, dk, dv; D written and read back
        out["roofline"]["compulsory_bytes"] = T * H * (4 * 2 * wl.d_qk + 4 * 2 * wl.d_v + 4 + 8)
    if args.stats and not args.bwd:
        st = torch.zeros(4, dtype=torch.int64, device="cuda")
        ea.fwd(q, k, v, o=o, lse=lse, cu_seqlens=cu, max_seqlen=inp["N"], causal=wl.causal,
               scale=inp["scale"], rescale_threshold_log2=args.tau, poly_exp_sixteenths=args.poly,
               schedule=args.schedule, stats=st, block_mask=bmask_dev, stream=stream)
        torch.cuda.synchronize()
        considered, taken, tiles, items = (int(x) for x in st.cpu())
        out["stats"] = {"rescale_considered": considered, "rescale_taken": taken,
                        "skip_rate": round(1.0 - taken / considered, 4) if considered else None,
                        "wave_tiles": tiles, "work_items": items}
    if args.stamps:
        out["metric"] = "instrumented build: " + out["metric"]
        out["stamps"] = stamp_summary(ea, q, k, v, o, lse, cu, inp, wl, args, bmask_dev, stream, fwd_lib,
                                      ev_ms)
    if not args.no_cpu_baseline:
        log(f"bench: cpu baseline (~{args.cpu_budget:.0f} s of oracle work)")
        out["cpu_baseline"] = cpu_baseline(inp, args.cpu_budget, dout_bits if args.bwd else None, bmask, f8)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
