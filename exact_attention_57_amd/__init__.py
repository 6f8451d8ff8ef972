"""Python binding of libattn.so, the MI355X fused attention forward and backward passes.

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI declared in ``include/attn.h``.  Torch is used for
device memory (``data_ptr``) and for the current HIP stream.

The library must be built first (``python exact_attention_57_amd/build.py``);
importing this package without it raises ImportError -- there is no fallback
of any kind.
"""
from __future__ import annotations

import ctypes
import math
import os

__all__ = [
    "AttnError", "lib", "fwd", "fwd_raw", "fwd_fp8", "fwd_fp8_raw", "bwd", "bwd_raw", "debug_exp2", "strerror", "version", "geometry",
    "ATTN_OK", "ATTN_ERR_NULL", "ATTN_ERR_SHAPE", "ATTN_ERR_UNSUPPORTED", "ATTN_ERR_ALIGN",
    "ATTN_ERR_VALUE", "ATTN_ERR_LAUNCH", "ATTN_ERR_SCRATCH", "NOALLOC_MAX_ROWS", "bwd_noalloc", "bwd_noalloc_raw", "SCHEDULE_LONGEST_FIRST", "SCHEDULE_NATURAL",
    "SUPPORTED_DIMS", "BWD_SUPPORTED_DIMS", "FP8_SUPPORTED_DIMS", "LIB_PATH", "CHECK_BUILDS", "check_build",
]

# The library built in-tree next to this file; no other copy is ever loaded.
LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libattn.so")

ATTN_OK = 0
ATTN_ERR_NULL = -1
ATTN_ERR_SHAPE = -2
ATTN_ERR_UNSUPPORTED = -3
ATTN_ERR_ALIGN = -4
ATTN_ERR_VALUE = -5
ATTN_ERR_LAUNCH = -6
ATTN_ERR_SCRATCH = -7
NOALLOC_MAX_ROWS = 16 * 1024 * 1024      # H * B * N limit of attn_bwd_noalloc
SCHEDULE_LONGEST_FIRST = 0
SCHEDULE_NATURAL = 1
SUPPORTED_DIMS = ((64, 64), (128, 128), (192, 128))
BWD_SUPPORTED_DIMS = ((64, 64), (128, 128), (192, 128))
FP8_SUPPORTED_DIMS = ((64, 64), (128, 128), (192, 128))


class AttnError(RuntimeError):
    def __init__(self, status: int, where: str = "attn_fwd"):
        self.status = status
        super().__init__(f"{where} failed with status {status}: {strerror(status)}")


class FwdOpts(ctypes.Structure):
    _fields_ = [
        ("rescale_threshold_log2", ctypes.c_float),
        ("poly_exp_sixteenths", ctypes.c_int),
        ("schedule", ctypes.c_int),
        ("stats", ctypes.c_void_p),
        ("block_mask", ctypes.c_void_p),
    ]


def _hip_runtimes_mapped():
    """Distinct libamdhip64 files mapped into this process (Linux /proc/self/maps)."""
    found = set()
    try:
        with open("/proc/self/maps") as f:
            for line in f:
                if "libamdhip64" in line:
                    found.add(os.path.realpath(line.split()[-1]))
    except OSError:
        pass
    return found


CHECK_BUILDS = ("racecheck", "stamps")


def _load(path=LIB_PATH):
    if not os.path.exists(path):
        raise ImportError(
            f"{path} is missing: build it with `python exact_attention_57_amd/build.py`")
    # torch ships its own HIP runtime.  Load it first so that libattn.so's
    # dependency on libamdhip64.so.7 resolves to that same, already-loaded
    # copy: two HIP runtimes in one process cannot share streams or memory.
    import torch  # noqa: F401
    L = ctypes.CDLL(path)
    runtimes = _hip_runtimes_mapped()
    if len(runtimes) > 1:
        raise ImportError(f"more than one HIP runtime is loaded: {sorted(runtimes)}")
    vp, i32, f32 = ctypes.c_void_p, ctypes.c_int, ctypes.c_float
    fwd_args = [vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, f32, i32, vp]
    L.attn_fwd.argtypes = fwd_args
    L.attn_fwd.restype = i32
    L.attn_fwd_ex.argtypes = fwd_args + [ctypes.POINTER(FwdOpts)]
    L.attn_fwd_ex.restype = i32
    L.attn_fwd_opts_default.argtypes = [ctypes.POINTER(FwdOpts)]
    L.attn_fwd_opts_default.restype = None
    L.attn_fwd_fp8.argtypes = fwd_args[:12] + [f32, f32, f32, i32, vp]
    L.attn_fwd_fp8.restype = i32
    L.attn_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, f32, i32, vp]
    L.attn_bwd.restype = i32
    L.attn_bwd_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, f32, i32, vp]
    L.attn_bwd_noalloc.restype = i32
    L.attn_strerror.argtypes = [i32]
    L.attn_strerror.restype = ctypes.c_char_p
    L.attn_debug_exp2.argtypes = [vp, vp, i32, i32, vp]
    L.attn_debug_exp2.restype = i32
    L.attn_version.argtypes = []
    L.attn_version.restype = i32
    L.attn_fwd_geometry.argtypes = [i32, i32, ctypes.POINTER(i32), ctypes.POINTER(i32), ctypes.POINTER(i32)]
    L.attn_fwd_geometry.restype = i32
    return L


lib = _load()
_check_libs = {}


def check_build(name: str):
    """ctypes handle of one of the checking builds compiled next to libattn.so
    from the same sources: ``"racecheck"`` (every barrier drains all memory
    traffic and is passed twice) or ``"stamps"`` (the forward kernels write
    per-workgroup timing records after the statistics counters).  Pass it as
    ``_lib`` to ``fwd``, ``fwd_fp8`` or ``bwd``."""
    if name not in CHECK_BUILDS:
        raise ValueError(f"unknown checking build {name!r}; one of {CHECK_BUILDS}")
    if name not in _check_libs:
        _check_libs[name] = _load(os.path.join(os.path.dirname(LIB_PATH), f"libattn_{name}.so"))
    return _check_libs[name]


def strerror(status: int) -> str:
    return lib.attn_strerror(int(status)).decode()


def version() -> int:
    return int(lib.attn_version())


def geometry(d_qk: int, d_v: int) -> dict:
    """Work decomposition of the forward kernels: rows per work item, keys per tile, rows per wave."""
    a, b, c = ctypes.c_int(), ctypes.c_int(), ctypes.c_int()
    st = int(lib.attn_fwd_geometry(int(d_qk), int(d_v), ctypes.byref(a), ctypes.byref(b), ctypes.byref(c)))
    if st != ATTN_OK:
        raise AttnError(st, "attn_fwd_geometry")
    return {"rows_per_item": a.value, "keys_per_tile": b.value, "rows_per_wave": c.value}


def _check_tensor(name, t, dtypes, device, shape=None, min_numel=None):
    """Raise ValueError unless ``t`` is a contiguous tensor of one of ``dtypes`` on
    ``device`` with exactly ``shape`` (or at least ``min_numel`` elements): the
    kernels read and write these buffers at the sizes the C ABI states, so a
    smaller or strided buffer would be accessed past its end."""
    if t.dtype not in dtypes:
        raise ValueError(f"{name} must have dtype {' or '.join(str(d) for d in dtypes)}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if min_numel is not None and t.numel() < min_numel:
        raise ValueError(f"{name} needs at least {min_numel} elements, got {t.numel()}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, the inputs on {device}")


def _check_inputs(names_tensors, dtypes, what):
    """Inputs of ``what``: contiguous GPU tensors of ``dtypes``, all on the first one's device."""
    first = names_tensors[0][1]
    if not first.is_cuda:
        raise ValueError(f"{what}: {names_tensors[0][0]} must be a CUDA tensor")
    for name, t in names_tensors:
        _check_tensor(name, t, dtypes, first.device)
    return first.device


# uint64 words per workgroup record that the instrumented build (check_build
# ("stamps")) writes after the four counters of ``stats``
STAMP_RECORD_WORDS = 16


def _check_stats(stats, device, min_numel=4):
    import torch
    _check_tensor("stats", stats, (torch.int64, torch.uint64), device, min_numel=min_numel)


def default_opts() -> FwdOpts:
    o = FwdOpts()
    lib.attn_fwd_opts_default(ctypes.byref(o))
    return o


def fwd_raw(q_ptr, k_ptr, v_ptr, o_ptr, lse_ptr, cu_ptr, B, H, N, d_qk, d_v, scale, causal,
            stream, opts: FwdOpts | None = None, _lib=None) -> int:
    """Call attn_fwd_ex with raw integer pointers; returns the status code."""
    return int((_lib or lib).attn_fwd_ex(q_ptr, k_ptr, v_ptr, o_ptr, lse_ptr, cu_ptr, int(B), int(H), int(N),
                               int(d_qk), int(d_v), float(scale), int(bool(causal)), stream,
                               ctypes.byref(opts) if opts is not None else None))


def _stream_handle(stream):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def _fwd_shape(q, cu_seqlens, max_seqlen):
    """(B, N, H, T, d_qk) of a forward call's q: [B, N, H, d] fixed length, or
    [T, H, d] with max_seqlen (fixed length, T = B * N) or with cu_seqlens."""
    if q.dim() == 4:
        B, N, H, d_qk = q.shape
        if cu_seqlens is not None:
            raise ValueError("4-D inputs are fixed length; pass [T, H, d] with cu_seqlens")
        T = B * N
    elif q.dim() == 3:
        T, H, d_qk = q.shape
        if cu_seqlens is None:
            if max_seqlen is None:
                B, N = 1, T
            else:
                N = int(max_seqlen)
                if N <= 0 or T % N:
                    raise ValueError("fixed-length [T, H, d] input needs T = B * max_seqlen")
                B = T // N
        else:
            if max_seqlen is None:
                raise ValueError("packed input needs max_seqlen")
            B = cu_seqlens.numel() - 1
            N = int(max_seqlen)
    else:
        raise ValueError("q must be [B, N, H, d] or [T, H, d]")
    return B, N, H, T, d_qk


def fwd(q, k, v, o=None, lse=None, cu_seqlens=None, *, max_seqlen=None, causal=False,
        scale=None, rescale_threshold_log2=8.0, poly_exp_sixteenths=0,
        schedule=SCHEDULE_LONGEST_FIRST, stats=None, block_mask=None, stream=None, _lib=None):
    """Fused attention forward on torch tensors.

    Fixed length: q, k [B, N, H, d_qk], v [B, N, H, d_v] (or [T, H, d] with
    ``cu_seqlens=None`` and ``max_seqlen`` = N, T = B*N).  Packed: q, k
    [T, H, d_qk], v [T, H, d_v] with ``cu_seqlens`` (int32 device [B+1]) and
    ``max_seqlen`` (>= longest sequence).  bf16, contiguous, on the GPU.

    Returns (o, lse): o bf16 shaped like v, lse fp32 [H, T].  Outputs are
    allocated with torch when not given.  ``stats``: optional uint64/int64
    device tensor of 4 counters that the kernel adds to.  ``block_mask``:
    optional uint8/bool device tensor [B, H, nb, nb], nb = ceil(N / 128), for
    block-sparse attention (see attn_fwd_opts in include/attn.h).  Every
    buffer given is checked for dtype, shape (o like v, lse [H, T]),
    contiguity and device before the call; ValueError otherwise.
    """
    import torch
    B, N, H, T, d_qk = _fwd_shape(q, cu_seqlens, max_seqlen)
    d_v = v.shape[-1]
    dev = _check_inputs((("q", q), ("k", k), ("v", v)), (torch.bfloat16,), "fwd")
    if k.shape != q.shape or v.shape[:-1] != q.shape[:-1]:
        raise ValueError("q, k, v shapes disagree")
    if cu_seqlens is not None:
        _check_tensor("cu_seqlens", cu_seqlens, (torch.int32,), dev, shape=(B + 1,))
    if o is None:
        o = torch.empty(v.shape, dtype=torch.bfloat16, device=q.device)
    _check_tensor("o", o, (torch.bfloat16,), dev, shape=v.shape)
    if lse is None:
        lse = torch.empty((H, T), dtype=torch.float32, device=q.device)
    _check_tensor("lse", lse, (torch.float32,), dev, shape=(H, T))
    if stats is not None:
        words = 4
        if _lib is not None and _lib is _check_libs.get("stamps"):
            # one record per workgroup of the grid (B * H * query blocks)
            words += STAMP_RECORD_WORDS * B * H * (-(-N // geometry(d_qk, d_v)["rows_per_item"]))
        _check_stats(stats, dev, words)
    if scale is None:
        scale = 1.0 / math.sqrt(d_qk)
    if block_mask is not None:
        nb = (N + 127) // 128
        _check_tensor("block_mask", block_mask, (torch.uint8, torch.bool), dev, shape=(B, H, nb, nb))
    opts = FwdOpts(float(rescale_threshold_log2), int(poly_exp_sixteenths), int(schedule),
                   stats.data_ptr() if stats is not None else None,
                   block_mask.data_ptr() if block_mask is not None else None)
    st = fwd_raw(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                 cu_seqlens.data_ptr() if cu_seqlens is not None else None,
                 B, H, N, d_qk, d_v, scale, causal, _stream_handle(stream), opts, _lib=_lib)
    if st != ATTN_OK:
        raise AttnError(st)
    return o, lse


def fwd_fp8_raw(q_ptr, k_ptr, v_ptr, o_ptr, lse_ptr, cu_ptr, B, H, N, d_qk, d_v, scale,
                q_descale, k_descale, v_descale, causal, stream, _lib=None) -> int:
    """Call attn_fwd_fp8 with raw integer pointers; returns the status code."""
    return int((_lib or lib).attn_fwd_fp8(q_ptr, k_ptr, v_ptr, o_ptr, lse_ptr, cu_ptr, int(B), int(H), int(N),
                                int(d_qk), int(d_v), float(scale), float(q_descale), float(k_descale),
                                float(v_descale), int(bool(causal)), stream))


def fwd_fp8(q8, k8, v8, o=None, lse=None, cu_seqlens=None, *, max_seqlen=None, causal=False,
            scale=None, q_descale=1.0, k_descale=1.0, v_descale=1.0, stream=None, _lib=None):
    """FP8 attention forward: q8, k8, v8 hold OCP E4M3 values (torch.float8_e4m3fn
    or uint8 bit patterns), contiguous CUDA tensors shaped as for ``fwd``, each
    multiplied by its descale factor.  Returns (o bf16 shaped like v8, lse fp32
    [H, T]); see attn_fwd_fp8 in include/attn.h."""
    import torch
    B, N, H, T, d_qk = _fwd_shape(q8, cu_seqlens, max_seqlen)
    d_v = v8.shape[-1]
    dev = _check_inputs((("q8", q8), ("k8", k8), ("v8", v8)), (torch.float8_e4m3fn, torch.uint8), "fwd_fp8")
    if k8.shape != q8.shape or v8.shape[:-1] != q8.shape[:-1]:
        raise ValueError("q8, k8, v8 shapes disagree")
    if cu_seqlens is not None:
        _check_tensor("cu_seqlens", cu_seqlens, (torch.int32,), dev, shape=(B + 1,))
    if o is None:
        o = torch.empty(v8.shape, dtype=torch.bfloat16, device=q8.device)
    _check_tensor("o", o, (torch.bfloat16,), dev, shape=v8.shape)
    if lse is None:
        lse = torch.empty((H, T), dtype=torch.float32, device=q8.device)
    _check_tensor("lse", lse, (torch.float32,), dev, shape=(H, T))
    if scale is None:
        scale = 1.0 / math.sqrt(d_qk)
    st = fwd_fp8_raw(q8.data_ptr(), k8.data_ptr(), v8.data_ptr(), o.data_ptr(), lse.data_ptr(),
                     cu_seqlens.data_ptr() if cu_seqlens is not None else None,
                     B, H, N, d_qk, d_v, scale, q_descale, k_descale, v_descale, causal, _stream_handle(stream),
                     _lib=_lib)
    if st != ATTN_OK:
        raise AttnError(st, "attn_fwd_fp8")
    return o, lse


def bwd_raw(q_ptr, k_ptr, v_ptr, o_ptr, do_ptr, lse_ptr, dq_ptr, dk_ptr, dv_ptr, delta_ptr, cu_ptr,
            B, H, N, d_qk, d_v, scale, causal, stream, _lib=None) -> int:
    """Call attn_bwd with raw integer pointers; returns the status code."""
    return int((_lib or lib).attn_bwd(q_ptr, k_ptr, v_ptr, o_ptr, do_ptr, lse_ptr, dq_ptr, dk_ptr, dv_ptr, delta_ptr, cu_ptr,
                            int(B), int(H), int(N), int(d_qk), int(d_v), float(scale), int(bool(causal)), stream))


def bwd(q, k, v, o, lse, dout, cu_seqlens=None, *, max_seqlen=None, causal=False, scale=None,
        dq=None, dk=None, dv=None, delta=None, stream=None, _lib=None):
    """Attention backward on torch tensors: gradients of the forward's o with
    respect to q, k, v for the output gradient ``dout``.

    Shapes and layouts as ``fwd`` (o and dout shaped like v; lse [H, T] as
    ``fwd`` returned it); the same cu_seqlens / max_seqlen / causal / scale
    as the forward call.  Returns (dq, dk, dv), bf16, allocated with torch
    when not given; ``delta`` (contiguous fp32, at least H*T elements, T the
    total token count) is the workspace for the row terms D = rowsum(dout * o).
    Every buffer is checked for dtype, shape (dq, dk, dv like q, k, v; lse
    [H, T]), contiguity and device before the call; ValueError otherwise.
    """
    import torch
    if q.dim() == 4:
        B, N, H, d_qk = q.shape
        if cu_seqlens is not None:
            raise ValueError("4-D inputs are fixed length; pass [T, H, d] with cu_seqlens")
    elif q.dim() == 3:
        T, H, d_qk = q.shape
        if cu_seqlens is None:
            N = T if max_seqlen is None else int(max_seqlen)
            if N <= 0 or T % N:
                raise ValueError("fixed-length [T, H, d] input needs T = B * max_seqlen")
            B = T // N
        else:
            if max_seqlen is None:
                raise ValueError("packed input needs max_seqlen")
            B = cu_seqlens.numel() - 1
            N = int(max_seqlen)
    else:
        raise ValueError("q must be [B, N, H, d] or [T, H, d]")
    d_v = v.shape[-1]
    T = B * N if q.dim() == 4 else q.shape[0]
    dev = _check_inputs((("q", q), ("k", k), ("v", v), ("o", o), ("dout", dout)), (torch.bfloat16,), "bwd")
    if k.shape != q.shape or v.shape[:-1] != q.shape[:-1] or o.shape != v.shape or dout.shape != v.shape:
        raise ValueError("q, k, v, o, dout shapes disagree")
    _check_tensor("lse", lse, (torch.float32,), dev, shape=(H, T))
    if cu_seqlens is not None:
        _check_tensor("cu_seqlens", cu_seqlens, (torch.int32,), dev, shape=(B + 1,))
    dq = torch.empty(q.shape, dtype=torch.bfloat16, device=q.device) if dq is None else dq
    dk = torch.empty(k.shape, dtype=torch.bfloat16, device=q.device) if dk is None else dk
    dv = torch.empty(v.shape, dtype=torch.bfloat16, device=q.device) if dv is None else dv
    _check_tensor("dq", dq, (torch.bfloat16,), dev, shape=q.shape)
    _check_tensor("dk", dk, (torch.bfloat16,), dev, shape=k.shape)
    _check_tensor("dv", dv, (torch.bfloat16,), dev, shape=v.shape)
    if delta is None:
        delta = torch.empty(H * T, dtype=torch.float32, device=q.device)
    _check_tensor("delta", delta, (torch.float32,), dev, min_numel=H * T)
    if scale is None:
        scale = 1.0 / math.sqrt(d_qk)
    st = bwd_raw(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), dout.data_ptr(), lse.data_ptr(),
                 dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), delta.data_ptr(),
                 cu_seqlens.data_ptr() if cu_seqlens is not None else None,
                 B, H, N, d_qk, d_v, scale, causal, _stream_handle(stream), _lib=_lib)
    if st != ATTN_OK:
        raise AttnError(st, "attn_bwd")
    return dq, dk, dv


def bwd_noalloc_raw(q_ptr, k_ptr, v_ptr, o_ptr, do_ptr, lse_ptr, dq_ptr, dk_ptr, dv_ptr, cu_ptr,
                    B, H, N, d_qk, d_v, scale, causal, stream) -> int:
    """Call attn_bwd_noalloc with raw integer pointers; returns the status code."""
    return int(lib.attn_bwd_noalloc(q_ptr, k_ptr, v_ptr, o_ptr, do_ptr, lse_ptr, dq_ptr, dk_ptr, dv_ptr, cu_ptr,
                                    int(B), int(H), int(N), int(d_qk), int(d_v), float(scale), int(bool(causal)),
                                    stream))


def bwd_noalloc(q, k, v, o, lse, dout, dq, dk, dv, cu_seqlens=None, *, max_seqlen=None, causal=False, scale=None,
                stream=None):
    """The backward pass without any allocation (attn_bwd_noalloc): as ``bwd``,
    but the caller passes dq, dk, dv, and the D workspace is the library's
    static scratch array (H * B * N <= NOALLOC_MAX_ROWS).  Calls that overlap
    in time on one GPU share that array and must not be issued.  Returns
    (dq, dk, dv)."""
    import torch
    if q.dim() == 4:
        B, N, H, d_qk = q.shape
        if cu_seqlens is not None:
            raise ValueError("4-D inputs are fixed length; pass [T, H, d] with cu_seqlens")
    elif q.dim() == 3:
        T, H, d_qk = q.shape
        if cu_seqlens is None:
            N = T if max_seqlen is None else int(max_seqlen)
            if N <= 0 or T % N:
                raise ValueError("fixed-length [T, H, d] input needs T = B * max_seqlen")
            B = T // N
        else:
            if max_seqlen is None:
                raise ValueError("packed input needs max_seqlen")
            B = cu_seqlens.numel() - 1
            N = int(max_seqlen)
    else:
        raise ValueError("q must be [B, N, H, d] or [T, H, d]")
    d_v = v.shape[-1]
    T = B * N if q.dim() == 4 else q.shape[0]
    dev = _check_inputs((("q", q), ("k", k), ("v", v), ("o", o), ("dout", dout)), (torch.bfloat16,), "bwd_noalloc")
    if k.shape != q.shape or v.shape[:-1] != q.shape[:-1] or o.shape != v.shape or dout.shape != v.shape:
        raise ValueError("q, k, v, o, dout shapes disagree")
    _check_tensor("lse", lse, (torch.float32,), dev, shape=(H, T))
    if cu_seqlens is not None:
        _check_tensor("cu_seqlens", cu_seqlens, (torch.int32,), dev, shape=(B + 1,))
    _check_tensor("dq", dq, (torch.bfloat16,), dev, shape=q.shape)
    _check_tensor("dk", dk, (torch.bfloat16,), dev, shape=k.shape)
    _check_tensor("dv", dv, (torch.bfloat16,), dev, shape=v.shape)
    if scale is None:
        scale = 1.0 / math.sqrt(d_qk)
    st = bwd_noalloc_raw(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), dout.data_ptr(), lse.data_ptr(),
                         dq.data_ptr(), dk.data_ptr(), dv.data_ptr(),
                         cu_seqlens.data_ptr() if cu_seqlens is not None else None,
                         B, H, N, d_qk, d_v, scale, causal, _stream_handle(stream))
    if st != ATTN_OK:
        raise AttnError(st, "attn_bwd_noalloc")
    return dq, dk, dv


def debug_exp2(x, use_poly: bool, y=None, stream=None):
    """The kernels' own exp2 (hardware or software cubic) over a fp32 CUDA tensor."""
    import torch
    dev = _check_inputs((("x", x),), (torch.float32,), "debug_exp2")
    if y is None:
        y = torch.empty_like(x)
    _check_tensor("y", y, (torch.float32,), dev, shape=x.shape)
    st = int(lib.attn_debug_exp2(x.data_ptr(), y.data_ptr(), x.numel(), int(bool(use_poly)),
                                 _stream_handle(stream)))
    if st != ATTN_OK:
        raise AttnError(st, "attn_debug_exp2")
    return y
