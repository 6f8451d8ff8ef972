"""Seeded synthetic inputs for the attention-forward workloads.

This module only *draws* inputs: random bf16 tensors, sequence lengths and
the packed-sequence offsets.  It contains none of the attention arithmetic,
so both the CPU oracle (``oracle/``) and the HIP path's tests and benchmark
may use it without sharing any of the method.

bf16 tensors are returned as ``numpy.uint16`` arrays holding the raw bf16
bit patterns (numpy has no bf16 type).  Values are drawn in float32 with
``standard_normal(dtype=float32)`` from PCG64 generators and rounded to bf16
with round-to-nearest-even.  Sequence lengths (packed workload) come from
``numpy.random.default_rng(seed)``; Q, K, V are streams 0, 1, 2, each cut
into chunks of about 2^20 elements drawn from
``default_rng(SeedSequence(seed, spawn_key=(stream, chunk)))`` so that
threads can fill them in parallel with the same result.

Layouts: q, k are ``[T, H, d_qk]``, v is ``[T, H, d_v]`` (token-major, heads
interleaved), where T is the total token count; ``cu_seqlens`` is int32
``[B+1]`` with ``cu_seqlens[b]`` the first token of sequence b.
"""
from __future__ import annotations

import math
import os
import threading
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np

__all__ = [
    "make_output_grad",
    "make_block_mask",
    "Workload",
    "WORKLOADS",
    "workload",
    "f32_to_bf16_bits",
    "bf16_bits_to_f32",
    "make_inputs",
    "make_custom_inputs",
    "ramp_strength",
]


@dataclass(frozen=True)
class Workload:
    """One attention-forward workload (shapes and value distribution)."""

    key: str
    B: int                 # number of sequences
    H: int                 # heads
    N: int                 # (max) sequence length
    d_qk: int
    d_v: int
    causal: bool
    varlen: bool = False   # lengths drawn uniformly in [len_lo, len_hi]
    len_lo: int = 0
    len_hi: int = 0
    ramp: bool = False     # per-key linear ramp on Q/K (logits grow along the sequence)
    description: str = ""
    scale: float = field(default=0.0)

    def softmax_scale(self) -> float:
        return self.scale if self.scale else 1.0 / math.sqrt(self.d_qk)


# The five workloads the forward pass is checked and timed on.
WORKLOADS = {
    "small_noncausal_b1h2n256d64": Workload(
        "small_noncausal_b1h2n256d64", B=1, H=2, N=256, d_qk=64, d_v=64, causal=False,
        description="non-causal, B=1 H=2 N=256 d=64, N(0,1), scale 1/8"),
    "noncausal_b4h16n4096d128": Workload(
        "noncausal_b4h16n4096d128", B=4, H=16, N=4096, d_qk=128, d_v=128, causal=False,
        description="non-causal, B=4 H=16 N=4096 d=128, N(0,1), scale 1/sqrt(128)"),
    "causal_b2h16n16384d128": Workload(
        "causal_b2h16n16384d128", B=2, H=16, N=16384, d_qk=128, d_v=128, causal=True,
        description="causal, B=2 H=16 N=16384 d=128, N(0,1), scale 1/sqrt(128)"),
    "causal_b2h32n8192dqk192dv128": Workload(
        "causal_b2h32n8192dqk192dv128", B=2, H=32, N=8192, d_qk=192, d_v=128, causal=True,
        description="causal split head dims d_qk=192 d_v=128, B=2 H=32 N=8192, scale 1/sqrt(192)"),
    "varlen_causal_16seq_h32d128_ramp": Workload(
        "varlen_causal_16seq_h32d128_ramp", B=16, H=32, N=32768, d_qk=128, d_v=128, causal=True,
        varlen=True, len_lo=512, len_hi=32768, ramp=True,
        description="packed causal, 16 sequences with lengths U[512,32768], H=32 d=128, "
                    "Q/K N(0,1) plus a per-key linear ramp (logit std ~4)"),
}

_ORDER = list(WORKLOADS)


def workload(key_or_index) -> Workload:
    """Look a workload up by key or by its 1-based position in ``WORKLOADS``."""
    if isinstance(key_or_index, int):
        return WORKLOADS[_ORDER[key_or_index - 1]]
    return WORKLOADS[key_or_index]


def f32_to_bf16_bits(x: np.ndarray, out: np.ndarray | None = None,
                     scratch: np.ndarray | None = None) -> np.ndarray:
    """Round float32 values to bf16 (round-to-nearest-even); return uint16 bit patterns.

    ``out`` (uint16) and ``scratch`` (uint32, same size) may be passed to avoid
    fresh allocations when converting in chunks.
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = np.empty(u.shape, dtype=np.uint32) if scratch is None else scratch.reshape(u.shape)
    np.right_shift(u, np.uint32(16), out=r)
    np.bitwise_and(r, np.uint32(1), out=r)
    np.add(r, np.uint32(0x7FFF), out=r)
    np.add(r, u, out=r)
    np.right_shift(r, np.uint32(16), out=r)
    if out is None:
        return r.astype(np.uint16)
    out[...] = r.reshape(out.shape)
    return out


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns to float32 (exact)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


_CHUNK_ELEMS = 1 << 20
_TLS = threading.local()


def _threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def _fill_normal(out2d: np.ndarray, seed: int, stream: int, add_rows: np.ndarray | None = None):
    """Fill uint16 [rows, cols] with bf16(N(0,1) + add_rows[row]).

    Rows are cut into chunks of about 2^20 elements; chunk c of stream s is
    drawn from ``default_rng(SeedSequence(seed, spawn_key=(s, c)))``, so the
    values do not depend on how many threads fill them.
    """
    rows, cols = out2d.shape
    per = max(1, _CHUNK_ELEMS // max(cols, 1))
    starts = list(range(0, rows, per))

    def work(ci):
        t0 = starts[ci]
        t1 = min(rows, t0 + per)
        n = (t1 - t0) * cols
        buf = getattr(_TLS, "f", None)
        if buf is None or buf.size < per * cols:
            _TLS.f = buf = np.empty(per * cols, dtype=np.float32)
            _TLS.s = np.empty(per * cols, dtype=np.uint32)
        z = buf[:n].reshape(t1 - t0, cols)
        rng = np.random.default_rng(np.random.SeedSequence(seed, spawn_key=(stream, ci)))
        rng.standard_normal(dtype=np.float32, out=z)
        if add_rows is not None:
            z += add_rows[t0:t1, None]
        f32_to_bf16_bits(z, out=out2d[t0:t1], scratch=_TLS.s[:n])

    if len(starts) <= 1:
        for ci in range(len(starts)):
            work(ci)
    else:
        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(work, range(len(starts))))


def _normal_bf16(seed: int, stream: int, shape, add_rows=None) -> np.ndarray:
    T = shape[0]
    row = int(np.prod(shape[1:]))
    out = np.empty((T, row), dtype=np.uint16)
    _fill_normal(out, seed, stream, add_rows)
    return out.reshape(shape)


def ramp_strength(d: int) -> float:
    """Ramp coefficient beta = gamma for the packed workload.

    With u = 1/sqrt(d) * ones(d), queries get +beta*u and key j of a sequence
    of length L gets +gamma*t_j*u, t_j = j/(L-1).  The scaled logit of a causal
    pair then has variance 1 + (beta^2 + gamma^2 E[t^2] + beta^2 gamma^2 Var t)/d
    with E[t^2] = 1/6 and Var t = 1/18 over causal pairs; beta = gamma = 13.255
    gives a logit standard deviation of about 4 at d = 128.
    """
    del d
    return 13.255


def make_inputs(wl, seed: int = 0) -> dict:
    """Draw the seeded inputs of a workload.

    Returns a dict with keys q, k, v (uint16 bf16 bits), cu_seqlens (int32
    [B+1]), lengths (int64 [B]), B, H, N (max length), d_qk, d_v, causal,
    scale, T.
    """
    if not isinstance(wl, Workload):
        wl = workload(wl)
    rng = np.random.default_rng(seed)
    if wl.varlen:
        lengths = rng.integers(wl.len_lo, wl.len_hi, size=wl.B, endpoint=True).astype(np.int64)
    else:
        lengths = np.full(wl.B, wl.N, dtype=np.int64)
    cu = np.zeros(wl.B + 1, dtype=np.int64)
    cu[1:] = np.cumsum(lengths)
    T = int(cu[-1])
    H = wl.H
    qadd = kadd = None
    if wl.ramp:
        beta = ramp_strength(wl.d_qk)
        u = 1.0 / math.sqrt(wl.d_qk)
        qadd = np.full(T, beta * u, dtype=np.float32)
        kadd = np.empty(T, dtype=np.float32)
        for b in range(wl.B):
            L = int(lengths[b])
            kadd[cu[b]:cu[b + 1]] = beta * u * np.arange(L, dtype=np.float64) / max(L - 1, 1)
    q = _normal_bf16(seed, 0, (T, H, wl.d_qk), qadd)
    k = _normal_bf16(seed, 1, (T, H, wl.d_qk), kadd)
    v = _normal_bf16(seed, 2, (T, H, wl.d_v))
    return dict(q=q, k=k, v=v, cu_seqlens=cu.astype(np.int32), lengths=lengths,
                B=wl.B, H=H, N=int(lengths.max()) if wl.B else 0, d_qk=wl.d_qk, d_v=wl.d_v,
                causal=wl.causal, scale=wl.softmax_scale(), T=T, key=wl.key)


def make_custom_inputs(lengths, H: int, d_qk: int, d_v: int, seed: int = 0,
                       std: float = 1.0, mean: float = 0.0) -> dict:
    """Seeded N(mean, std^2) bf16 inputs for arbitrary (ragged) sequence lengths.

    Used for edge cases: empty sequences, lengths that are not a multiple of
    any tile size, single-token sequences.
    """
    lengths = np.asarray(lengths, dtype=np.int64)
    cu = np.zeros(len(lengths) + 1, dtype=np.int64)
    cu[1:] = np.cumsum(lengths)
    T = int(cu[-1])

    def draw(stream, d):
        bits = _normal_bf16(seed, stream, (T, H, d))
        if std == 1.0 and mean == 0.0:
            return bits
        x = bf16_bits_to_f32(bits) * np.float32(std) + np.float32(mean)
        return f32_to_bf16_bits(x)

    q = draw(0, d_qk)
    k = draw(1, d_qk)
    v = draw(2, d_v)
    return dict(q=q, k=k, v=v, cu_seqlens=cu.astype(np.int32), lengths=lengths,
                B=len(lengths), H=H, N=int(lengths.max()) if len(lengths) else 0,
                d_qk=d_qk, d_v=d_v, T=T)


def make_output_grad(inp: dict, seed: int = 0) -> np.ndarray:
    """Seeded N(0, 1) bf16 output gradient dO [T, H, d_v] for an input dict
    (its own random stream, independent of q, k, v)."""
    return _normal_bf16(seed, 3, (int(inp["T"]), int(inp["H"]), int(inp["d_v"])))


def make_block_mask(B: int, H: int, N: int, density: float, seed: int = 0) -> np.ndarray:
    """Seeded random uint8 block mask [B, H, nb, nb], nb = ceil(N / 128): each
    128 x 128 (query block, key block) pair is kept with probability
    ``density`` (independent draws from their own random stream)."""
    nb = (int(N) + 127) // 128
    rng = np.random.default_rng(np.random.SeedSequence(seed, spawn_key=(4,)))
    return (rng.random((B, H, nb, nb)) < density).astype(np.uint8)



def f32_to_e4m3_codes(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the OCP E4M3 8-bit float (nearest even; values
    beyond 448 saturate to +-448) and return the uint8 bit patterns.  Input
    preparation only: torch's own float8_e4m3fn conversion on the CPU."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    t = torch.clamp(t, -448.0, 448.0)
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def make_fp8_inputs(inp: dict, prescale=(1.0, 1.0, 1.0)) -> dict:
    """FP8 copies of an input dict's bf16 q, k, v: each tensor is multiplied
    by its ``prescale`` factor, rounded to E4M3 codes, and paired with the
    dequantisation factor 1/prescale.  Returns a new dict with q8, k8, v8
    (uint8) and q_descale, k_descale, v_descale, plus the shape fields."""
    out = {key: val for key, val in inp.items() if key not in ("q", "k", "v")}
    for name, f in zip(("q", "k", "v"), prescale):
        x = bf16_bits_to_f32(inp[name]) * np.float32(f)
        out[name + "8"] = f32_to_e4m3_codes(x)
        out[name + "_descale"] = float(np.float32(1.0) / np.float32(f))
    return out
