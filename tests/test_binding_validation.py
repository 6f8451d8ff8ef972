"""The Python binding checks every caller-supplied buffer before it calls the
library: dtype, shape, contiguity and device.  The kernels read and write
these buffers at the sizes the C ABI states, so a buffer that is too small or
strided must be refused in Python (ValueError) rather than written past its
end.

These run on the CPU: the only check that needs a GPU tensor (the inputs'
``is_cuda``) is replaced by one that accepts CPU tensors, and the library
handle is replaced by one that fails the test if any entry point is reached,
so every case here must be refused before the call.
"""
import pytest
import torch

import exact_attention_57_amd as ea

bf16 = torch.bfloat16


class _NoCalls:
    def __getattr__(self, name):
        raise AssertionError(f"the library's {name} was reached with an invalid buffer")


@pytest.fixture
def cpu_binding(monkeypatch):
    def inputs_on_cpu(names_tensors, dtypes, what):
        dev = names_tensors[0][1].device
        for name, t in names_tensors:
            ea._check_tensor(name, t, dtypes, dev)
        return dev
    monkeypatch.setattr(ea, "_check_inputs", inputs_on_cpu)
    monkeypatch.setattr(ea, "lib", _NoCalls())
    monkeypatch.setattr(ea, "_stream_handle", lambda s: None)
    return ea


def _qkv(B=2, N=40, H=3, d=64, dtype=bf16):
    q = torch.zeros(B, N, H, d, dtype=dtype)
    return q, q.clone(), q.clone()


def test_check_tensor_accepts_exact_buffer():
    t = torch.zeros(3, 5, dtype=torch.float32)
    ea._check_tensor("t", t, (torch.float32,), t.device, shape=(3, 5))
    ea._check_tensor("t", t, (torch.float32,), t.device, min_numel=15)


@pytest.mark.parametrize("bad,msg", [
    (torch.zeros(3, 5, dtype=torch.float64), "dtype"),
    (torch.zeros(5, 3, dtype=torch.float32), "shape"),
    (torch.zeros(5, 3, dtype=torch.float32).t(), "contiguous"),
])
def test_check_tensor_rejects(bad, msg):
    with pytest.raises(ValueError, match=msg):
        ea._check_tensor("t", bad, (torch.float32,), torch.device("cpu"), shape=(3, 5))


def test_check_tensor_rejects_short_buffer_and_other_device():
    t = torch.zeros(14, dtype=torch.float32)
    with pytest.raises(ValueError, match="at least 15"):
        ea._check_tensor("t", t, (torch.float32,), t.device, min_numel=15)
    with pytest.raises(ValueError, match="is on"):
        ea._check_tensor("t", t, (torch.float32,), torch.device("meta"))


def test_inputs_must_be_on_the_gpu():
    q, k, v = _qkv()
    with pytest.raises(ValueError, match="CUDA"):
        ea.fwd(q, k, v)
    with pytest.raises(ValueError, match="CUDA"):
        ea.bwd(q, k, v, v, torch.zeros(3, 80), v)


@pytest.mark.parametrize("kw,msg", [
    (dict(o=torch.zeros(2, 40, 3, 32, dtype=bf16)), "o must have shape"),
    (dict(o=torch.zeros(2, 40, 3, 64, dtype=torch.float16)), "o must have dtype"),
    (dict(o=torch.zeros(2, 40, 64, 3, dtype=bf16).transpose(2, 3)), "o must be contiguous"),
    (dict(lse=torch.zeros(3, 79)), "lse must have shape"),
    (dict(lse=torch.zeros(80, 3).t()), "lse must be contiguous"),
    (dict(lse=torch.zeros(3, 80, dtype=torch.float64)), "lse must have dtype"),
    (dict(stats=torch.zeros(3, dtype=torch.int64)), "stats needs at least 4"),
    (dict(stats=torch.zeros(4, dtype=torch.int32)), "stats must have dtype"),
    (dict(stats=torch.zeros(8, dtype=torch.int64)[::2]), "stats must be contiguous"),
    (dict(block_mask=torch.zeros(2, 3, 1, 2, dtype=torch.uint8)), "block_mask must have shape"),
])
def test_fwd_rejects_bad_buffers(cpu_binding, kw, msg):
    q, k, v = _qkv()
    with pytest.raises(ValueError, match=msg):
        ea.fwd(q, k, v, **kw)


def test_fwd_stamps_build_needs_the_record_area(cpu_binding, monkeypatch):
    # the instrumented build writes one record per workgroup after the four counters
    fake = _NoCalls()
    monkeypatch.setitem(ea._check_libs, "stamps", fake)
    # the library states the rows per workgroup; here 256 stands in for it
    monkeypatch.setattr(ea, "geometry", lambda d_qk, d_v: {"rows_per_item": 256, "keys_per_tile": 128})
    q, k, v = _qkv()                       # B=2, N=40, H=3: one query block per (sequence, head)
    need = 4 + ea.STAMP_RECORD_WORDS * 2 * 3
    with pytest.raises(ValueError, match=f"stats needs at least {need}"):
        ea.fwd(q, k, v, max_seqlen=40, stats=torch.zeros(need - 1, dtype=torch.int64), _lib=fake)
    with pytest.raises(AssertionError, match="reached"):   # a whole record area passes the checks
        ea.fwd(q, k, v, max_seqlen=40, stats=torch.zeros(need, dtype=torch.int64), _lib=fake)
    with pytest.raises(AssertionError, match="reached"):   # the default build needs the counters only
        ea.fwd(q, k, v, max_seqlen=40, stats=torch.zeros(4, dtype=torch.int64))


def test_fwd_packed_cu_seqlens_checked(cpu_binding):
    q = torch.zeros(100, 2, 64, dtype=bf16)
    with pytest.raises(ValueError, match="cu_seqlens must have dtype"):
        ea.fwd(q, q, q, cu_seqlens=torch.tensor([0, 50, 100], dtype=torch.int64), max_seqlen=50)
    with pytest.raises(ValueError, match="cu_seqlens must have shape"):
        ea.fwd(q, q, q, cu_seqlens=torch.zeros(2, 2, dtype=torch.int32), max_seqlen=50)


@pytest.mark.parametrize("kw,msg", [
    (dict(dq=torch.zeros(2, 40, 3, 32, dtype=bf16)), "dq must have shape"),
    (dict(dk=torch.zeros(2, 40, 3, 64, dtype=torch.float32)), "dk must have dtype"),
    (dict(dv=torch.zeros(2, 40, 64, 3, dtype=bf16).transpose(2, 3)), "dv must be contiguous"),
    (dict(delta=torch.zeros(3 * 80 - 1)), "delta needs at least"),
    (dict(delta=torch.zeros(2 * 3 * 80)[::2]), "delta must be contiguous"),
    (dict(delta=torch.zeros(3 * 80, dtype=torch.float64)), "delta must have dtype"),
])
def test_bwd_rejects_bad_buffers(cpu_binding, kw, msg):
    q, k, v = _qkv()
    lse = torch.zeros(3, 80)
    with pytest.raises(ValueError, match=msg):
        ea.bwd(q, k, v, v.clone(), lse, v.clone(), **kw)


def test_bwd_rejects_bad_lse(cpu_binding):
    q, k, v = _qkv()
    for lse, msg in ((torch.zeros(3, 79), "lse must have shape"), (torch.zeros(80, 3), "lse must have shape"),
                     (torch.zeros(3, 80, dtype=torch.float16), "lse must have dtype")):
        with pytest.raises(ValueError, match=msg):
            ea.bwd(q, k, v, v.clone(), lse, v.clone())


@pytest.mark.parametrize("kw,msg", [
    (dict(o=torch.zeros(2, 40, 3, 32, dtype=bf16)), "o must have shape"),
    (dict(lse=torch.zeros(3, 80, dtype=torch.float16)), "lse must have dtype"),
    (dict(lse=torch.zeros(3, 81)), "lse must have shape"),
])
def test_fwd_fp8_rejects_bad_buffers(cpu_binding, kw, msg):
    q8, k8, v8 = _qkv(dtype=torch.uint8)
    with pytest.raises(ValueError, match=msg):
        ea.fwd_fp8(q8, k8, v8, **kw)


def test_debug_exp2_rejects_bad_output(cpu_binding):
    x = torch.zeros(10)
    with pytest.raises(ValueError, match="y must have shape"):
        ea.debug_exp2(x, False, y=torch.zeros(9))
