"""C-ABI checks that need no GPU.

The library must load, export every function include/attn.h declares, and
reject invalid arguments with the documented status codes before any HIP
call (so these calls are safe on a machine without a GPU: none of them
reaches a launch).
"""
import ctypes
import math
import os
import re

import pytest

import exact_attention_57_amd as ea

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "attn.h")
P = 0x10000          # a 16-byte-aligned fake device address: never dereferenced here


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\*?\s*(attn_[a-z0-9_]+)\s*\(",
                       text, flags=re.M)
    return sorted(set(names))


def test_header_declares_expected_entry_points():
    names = declared_functions()
    for want in ("attn_fwd", "attn_fwd_ex", "attn_fwd_opts_default", "attn_strerror",
                 "attn_debug_exp2", "attn_version", "attn_fwd_geometry", "attn_bwd", "attn_fwd_fp8",
                 "attn_bwd_noalloc"):
        assert want in names


def test_library_exports_every_declared_symbol():
    raw = ctypes.CDLL(ea.LIB_PATH)
    for name in declared_functions():
        assert hasattr(raw, name), f"libattn.so does not export {name}"


def test_strerror_covers_every_code():
    codes = [ea.ATTN_OK, ea.ATTN_ERR_NULL, ea.ATTN_ERR_SHAPE, ea.ATTN_ERR_UNSUPPORTED,
             ea.ATTN_ERR_ALIGN, ea.ATTN_ERR_VALUE, ea.ATTN_ERR_LAUNCH, ea.ATTN_ERR_SCRATCH]
    msgs = [ea.strerror(c) for c in codes]
    assert all(msgs) and len(set(msgs)) == len(msgs)
    assert "unknown" in ea.strerror(-99)
    assert ea.version() >= 100


def test_default_options():
    o = ea.default_opts()
    assert o.rescale_threshold_log2 == 8.0
    assert o.poly_exp_sixteenths == 0
    assert o.schedule == ea.SCHEDULE_LONGEST_FIRST
    assert not o.stats


def call(**kw):
    args = dict(q=P, k=P, v=P, o=P, lse=P, cu=None, B=1, H=1, N=1, d_qk=128, d_v=128,
                scale=1.0, causal=0, stream=None, opts=None)
    args.update(kw)
    return ea.fwd_raw(args["q"], args["k"], args["v"], args["o"], args["lse"], args["cu"],
                      args["B"], args["H"], args["N"], args["d_qk"], args["d_v"], args["scale"],
                      args["causal"], args["stream"], args["opts"])


@pytest.mark.parametrize("kw,code", [
    (dict(B=0), ea.ATTN_ERR_SHAPE),
    (dict(H=0), ea.ATTN_ERR_SHAPE),
    (dict(N=-1), ea.ATTN_ERR_SHAPE),
    (dict(B=70000), ea.ATTN_ERR_SHAPE),
    (dict(N=65535 * ea.geometry(128, 128)["rows_per_item"] + 1), ea.ATTN_ERR_SHAPE),
    (dict(H=64, N=262144), ea.ATTN_ERR_SHAPE),            # 4 GiB of K rows in one sequence
    (dict(H=64, N=262000), ea.ATTN_ERR_SHAPE),            # tile requests up to 255 rows past the end
    (dict(d_qk=96, d_v=96), ea.ATTN_ERR_UNSUPPORTED),
    (dict(d_qk=128, d_v=64), ea.ATTN_ERR_UNSUPPORTED),
    (dict(d_qk=192, d_v=192), ea.ATTN_ERR_UNSUPPORTED),
    (dict(scale=math.nan), ea.ATTN_ERR_VALUE),
    (dict(scale=math.inf), ea.ATTN_ERR_VALUE),
    (dict(q=None), ea.ATTN_ERR_NULL),
    (dict(lse=None), ea.ATTN_ERR_NULL),
    (dict(o=None), ea.ATTN_ERR_NULL),
    (dict(q=P + 8), ea.ATTN_ERR_ALIGN),
    (dict(v=P + 4), ea.ATTN_ERR_ALIGN),
    (dict(lse=P + 2), ea.ATTN_ERR_ALIGN),
    (dict(cu=P + 1), ea.ATTN_ERR_ALIGN),
    (dict(N=0, q=None, k=None, v=None, o=None, lse=None), ea.ATTN_OK),
])
def test_validation_codes(kw, code):
    assert call(**kw) == code


@pytest.mark.parametrize("field,value", [
    ("poly_exp_sixteenths", 3), ("poly_exp_sixteenths", 16), ("poly_exp_sixteenths", -2),
    ("schedule", 2), ("rescale_threshold_log2", math.inf), ("rescale_threshold_log2", math.nan),
    ("rescale_threshold_log2", 64.5), ("rescale_threshold_log2", 200.0),
])
def test_option_validation(field, value):
    o = ea.default_opts()
    setattr(o, field, value)
    assert call(opts=o) == ea.ATTN_ERR_VALUE


@pytest.mark.parametrize("tau,code", [(64.0, ea.ATTN_OK), (64.001, ea.ATTN_ERR_VALUE), (-5.0, ea.ATTN_OK)])
def test_rescale_threshold_bound(tau, code):
    """Thresholds up to 64 (log2 units) are accepted; larger ones are rejected
    before anything runs (N = 0 returns after the option checks)."""
    o = ea.default_opts()
    o.rescale_threshold_log2 = tau
    assert call(N=0, q=None, k=None, v=None, o=None, lse=None, opts=o) == code


def test_misaligned_stats_rejected():
    o = ea.default_opts()
    o.stats = P + 4
    assert call(opts=o) == ea.ATTN_ERR_ALIGN


def test_debug_exp2_validation():
    f = ea.lib.attn_debug_exp2
    assert f(P, P, -1, 0, None) == ea.ATTN_ERR_SHAPE
    assert f(P, P, 4, 2, None) == ea.ATTN_ERR_VALUE
    assert f(None, P, 4, 0, None) == ea.ATTN_ERR_NULL
    assert f(P + 2, P, 4, 0, None) == ea.ATTN_ERR_ALIGN
    assert f(None, None, 0, 1, None) == ea.ATTN_OK


def test_geometry_query():
    for d_qk, d_v in ea.SUPPORTED_DIMS:
        g = ea.geometry(d_qk, d_v)
        assert g["rows_per_item"] % g["rows_per_wave"] == 0
        assert g["keys_per_tile"] % 32 == 0
    with pytest.raises(ea.AttnError):
        ea.geometry(96, 96)


def call_bwd(**kw):
    args = dict(q=P, k=P, v=P, o=P, do=P, lse=P, dq=P, dk=P, dv=P, delta=P, cu=None, B=1, H=1, N=1,
                d_qk=128, d_v=128, scale=1.0, causal=0, stream=None)
    args.update(kw)
    return ea.bwd_raw(args["q"], args["k"], args["v"], args["o"], args["do"], args["lse"], args["dq"],
                      args["dk"], args["dv"], args["delta"], args["cu"], args["B"], args["H"], args["N"],
                      args["d_qk"], args["d_v"], args["scale"], args["causal"], args["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(B=0), ea.ATTN_ERR_SHAPE),
    (dict(H=0), ea.ATTN_ERR_SHAPE),
    (dict(N=-1), ea.ATTN_ERR_SHAPE),
    (dict(B=2, N=2 ** 30 + 1), ea.ATTN_ERR_SHAPE),
    (dict(H=64, N=262144), ea.ATTN_ERR_SHAPE),            # 4 GiB of K rows in one sequence
    (dict(H=64, N=262000), ea.ATTN_ERR_SHAPE),            # tile requests up to 255 rows past the end
    (dict(d_qk=192, d_v=192), ea.ATTN_ERR_UNSUPPORTED),
    (dict(d_qk=128, d_v=64), ea.ATTN_ERR_UNSUPPORTED),
    (dict(d_qk=96, d_v=96), ea.ATTN_ERR_UNSUPPORTED),
    (dict(scale=math.nan), ea.ATTN_ERR_VALUE),
    (dict(do=None), ea.ATTN_ERR_NULL),
    (dict(delta=None), ea.ATTN_ERR_NULL),
    (dict(dv=None), ea.ATTN_ERR_NULL),
    (dict(o=P + 8), ea.ATTN_ERR_ALIGN),
    (dict(dk=P + 2), ea.ATTN_ERR_ALIGN),
    (dict(delta=P + 2), ea.ATTN_ERR_ALIGN),
    (dict(cu=P + 1), ea.ATTN_ERR_ALIGN),
    (dict(N=0, q=None, k=None, v=None, o=None, do=None, lse=None, dq=None, dk=None, dv=None, delta=None),
     ea.ATTN_OK),
])
def test_bwd_validation_codes(kw, code):
    assert call_bwd(**kw) == code


@pytest.mark.parametrize("kw,code", [
    (dict(poly=2), ea.ATTN_ERR_UNSUPPORTED),
    (dict(d_qk=192, d_v=128, poly=4), ea.ATTN_ERR_UNSUPPORTED),
    (dict(N=32769), ea.ATTN_ERR_SHAPE),
    (dict(N=0, q=None, k=None, v=None, o=None, lse=None), ea.ATTN_OK),
])
def test_block_mask_validation(kw, code):
    o = ea.default_opts()
    assert o.block_mask is None
    o.block_mask = P
    if "poly" in kw:
        o.poly_exp_sixteenths = kw.pop("poly")
    assert call(opts=o, **kw) == code



def call_fp8(**kw):
    args = dict(q=P, k=P, v=P, o=P, lse=P, cu=None, B=1, H=1, N=1, d_qk=128, d_v=128,
                scale=1.0, qd=1.0, kd=1.0, vd=1.0, causal=0, stream=None)
    args.update(kw)
    return ea.fwd_fp8_raw(args["q"], args["k"], args["v"], args["o"], args["lse"], args["cu"],
                          args["B"], args["H"], args["N"], args["d_qk"], args["d_v"], args["scale"],
                          args["qd"], args["kd"], args["vd"], args["causal"], args["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(B=0), ea.ATTN_ERR_SHAPE),
    (dict(H=0), ea.ATTN_ERR_SHAPE),
    (dict(N=-1), ea.ATTN_ERR_SHAPE),
    (dict(H=64, N=2 ** 18 + 1), ea.ATTN_ERR_SHAPE),
    (dict(H=64, N=262000), ea.ATTN_ERR_SHAPE),            # tile requests up to 255 rows past the end
    (dict(d_qk=64, d_v=128), ea.ATTN_ERR_UNSUPPORTED),
    (dict(d_qk=192, d_v=192), ea.ATTN_ERR_UNSUPPORTED),
    (dict(scale=math.nan), ea.ATTN_ERR_VALUE),
    (dict(qd=0.0), ea.ATTN_ERR_VALUE),
    (dict(kd=-1.0), ea.ATTN_ERR_VALUE),
    (dict(vd=math.inf), ea.ATTN_ERR_VALUE),
    (dict(vd=math.nan), ea.ATTN_ERR_VALUE),
    (dict(k=None), ea.ATTN_ERR_NULL),
    (dict(lse=None), ea.ATTN_ERR_NULL),
    (dict(v=P + 8), ea.ATTN_ERR_ALIGN),
    (dict(o=P + 2), ea.ATTN_ERR_ALIGN),
    (dict(lse=P + 2), ea.ATTN_ERR_ALIGN),
    (dict(cu=P + 1), ea.ATTN_ERR_ALIGN),
    (dict(N=0, q=None, k=None, v=None, o=None, lse=None), ea.ATTN_OK),
])
def test_fp8_validation_codes(kw, code):
    assert call_fp8(**kw) == code


def call_noalloc(**kw):
    args = dict(q=P, k=P, v=P, o=P, do=P, lse=P, dq=P, dk=P, dv=P, cu=None, B=1, H=1, N=1, d_qk=128, d_v=128,
                scale=1.0, causal=0, stream=None)
    args.update(kw)
    return ea.bwd_noalloc_raw(args["q"], args["k"], args["v"], args["o"], args["do"], args["lse"], args["dq"],
                              args["dk"], args["dv"], args["cu"], args["B"], args["H"], args["N"], args["d_qk"],
                              args["d_v"], args["scale"], args["causal"], args["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(B=0), ea.ATTN_ERR_SHAPE),
    (dict(d_qk=96, d_v=96), ea.ATTN_ERR_UNSUPPORTED),
    (dict(scale=math.nan), ea.ATTN_ERR_VALUE),
    (dict(dk=None), ea.ATTN_ERR_NULL),
    (dict(do=P + 8), ea.ATTN_ERR_ALIGN),
    (dict(lse=P + 2), ea.ATTN_ERR_ALIGN),
    (dict(N=0, q=None, k=None, v=None, o=None, do=None, lse=None, dq=None, dk=None, dv=None), ea.ATTN_OK),
    # the scratch array holds ATTN_NOALLOC_MAX_ROWS rows of D (H * B * N)
    (dict(H=16, B=2, N=ea.NOALLOC_MAX_ROWS // 32 + 1), ea.ATTN_ERR_SCRATCH),
    (dict(H=1, B=1, N=ea.NOALLOC_MAX_ROWS + 1, d_qk=64, d_v=64), ea.ATTN_ERR_SCRATCH),
])
def test_noalloc_validation_codes(kw, code):
    """The allocation-free backward entry point checks its arguments like
    attn_bwd, and rejects problems whose D rows exceed its scratch array,
    before any HIP call."""
    assert call_noalloc(**kw) == code


def test_noalloc_limit_matches_header():
    text = open(HEADER).read()
    m = re.search(r"#define ATTN_NOALLOC_MAX_ROWS \((\d+) \* (\d+) \* (\d+)\)", text)
    assert m and int(m.group(1)) * int(m.group(2)) * int(m.group(3)) == ea.NOALLOC_MAX_ROWS
