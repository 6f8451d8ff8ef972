"""Helpers for the GPU tests: device transfer, a call through the C ABI, and
the comparison against the CPU oracle with the stated tolerances.

Tolerances (bf16 inputs, fp32 accumulation, bf16 output):
  O:   max |gpu - oracle| <= 2e-2 and mean |gpu - oracle| <= 2e-3
  LSE: max |gpu - oracle| <= 1e-3
"""
from __future__ import annotations

import sys

import numpy as np

TOL_O_MAX = 2e-2
TOL_O_MEAN = 2e-3
TOL_LSE = 1e-3


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def torch_cuda():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    return torch


def to_dev(bits: np.ndarray):
    torch = torch_cuda()
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def run(inp: dict, causal=None, packed=None, scale=None, o=None, lse=None, **opts):
    """Run the GPU forward pass on a ``workloads`` input dict; returns (o, lse) torch tensors.

    packed=None: use cu_seqlens only when the lengths differ (else fixed length).
    """
    torch = torch_cuda()
    import exact_attention_57_amd as ea
    q, k, v = to_dev(inp["q"]), to_dev(inp["k"]), to_dev(inp["v"])
    lengths = np.asarray(inp["lengths"])
    if packed is None:
        packed = bool(len(lengths) == 0 or lengths.min() != lengths.max())
    cu = torch.from_numpy(np.asarray(inp["cu_seqlens"], dtype=np.int32)).cuda() if packed else None
    causal = inp["causal"] if causal is None else causal
    scale = inp["scale"] if scale is None else scale
    out = ea.fwd(q, k, v, o=o, lse=lse, cu_seqlens=cu, max_seqlen=max(int(inp["N"]), 1),
                 causal=causal, scale=scale, **opts)
    torch.cuda.synchronize()
    return out


def o_f64(o, rows=None, heads=None) -> np.ndarray:
    t = o
    if rows is not None:
        import torch
        t = t[torch.as_tensor(np.asarray(rows), device=o.device)]
    if heads is not None:
        import torch
        t = t[:, torch.as_tensor(np.asarray(heads), device=o.device)]
    return t.float().cpu().numpy().astype(np.float64)


def lse_f64(lse, rows=None, heads=None) -> np.ndarray:
    a = lse.cpu().numpy().astype(np.float64)
    if heads is not None:
        a = a[np.asarray(heads)]
    if rows is not None:
        a = a[:, np.asarray(rows)]
    return a


def errors(O, L, O_ref, L_ref) -> dict:
    e = np.abs(O - O_ref)
    le = np.abs(L - L_ref)
    i = np.unravel_index(int(np.argmax(e)), e.shape) if e.size else None
    return dict(o_max=float(e.max()) if e.size else 0.0, o_mean=float(e.mean()) if e.size else 0.0,
                lse_max=float(le.max()) if le.size else 0.0,
                o_at_max=float(O_ref[i]) if i is not None else 0.0)


def assert_close(O, L, O_ref, L_ref, what="") -> dict:
    err = errors(O, L, O_ref, L_ref)
    say(f"  parity {what}: {err}")
    assert np.isfinite(O).all() and np.isfinite(L).all(), f"{what}: non-finite output"
    assert err["o_max"] <= TOL_O_MAX, f"{what}: O max abs err {err['o_max']}"
    assert err["o_mean"] <= TOL_O_MEAN, f"{what}: O mean abs err {err['o_mean']}"
    assert err["lse_max"] <= TOL_LSE, f"{what}: LSE max abs err {err['lse_max']}"
    return err


def sample_rows(cu, per_seq: int, seed: int = 0, extra=(0, 1, 63, 64, 127, 128, 129)) -> np.ndarray:
    """Query rows to check per sequence: tile/block boundaries, the last rows, and random ones."""
    rng = np.random.default_rng(seed)
    rows = []
    for b in range(len(cu) - 1):
        s, e = int(cu[b]), int(cu[b + 1])
        L = e - s
        if L == 0:
            continue
        pick = {x for x in extra if x < L} | {L - 1, max(0, L - 2), L // 2}
        pick |= set(rng.integers(0, L, per_seq).tolist())
        rows.extend(s + np.array(sorted(pick)))
    return np.array(sorted(rows), dtype=np.int64)
