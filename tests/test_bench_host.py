"""Host-side checks of bench.py (CPU): the FLOP convention every reported
rate uses, the block-sparse FLOP count, the compulsory-byte figures, and the
rule that a stored traffic record is used only for the kernel source it was
measured on.  The expected values are the workload definitions' own numbers
(4*B*H*N^2*d non-causal, halved when causal, 2*B*H*N^2*(d_qk + d_v) for
split head dims, summed over packed sequences)."""
import json
import os

import numpy as np
import pytest

import bench
import workloads


def test_flop_convention_on_the_workloads():
    f = bench.algorithmic_flops
    assert f([256], 2, 64, 64, False) == 4 * 2 * 256 ** 2 * 64                     # 3.355e7
    assert f([4096] * 4, 16, 128, 128, False) == 4 * 4 * 16 * 4096 ** 2 * 128      # 5.498e11
    assert f([16384] * 2, 16, 128, 128, True) == 4 * 2 * 16 * 16384 ** 2 * 128 / 2
    assert f([8192] * 2, 32, 192, 128, True) == 2 * 2 * 32 * 8192 ** 2 * (192 + 128) / 2
    lengths = [300, 1, 0, 777]
    assert f(lengths, 3, 128, 128, True) == sum(f([L], 3, 128, 128, True) for L in lengths)
    assert abs(f([4096] * 4, 16, 128, 128, False) - 5.498e11) / 5.498e11 < 1e-3


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("dims", [(128, 128), (192, 128)])
def test_block_sparse_flops_all_ones_equals_dense(causal, dims):
    lengths = [1000, 129, 0, 4096]
    nb = (max(lengths) + 127) // 128
    mask = np.ones((len(lengths), 2, nb, nb), dtype=np.uint8)
    dense = bench.algorithmic_flops(lengths, 2, dims[0], dims[1], causal)
    sparse = bench.block_sparse_flops(lengths, 2, dims[0], dims[1], causal, mask)
    if not causal:
        assert sparse == dense
    else:
        # blocks: the diagonal ones count half, so the count is the dense
        # convention (N^2 / 2) computed per block, exactly
        assert abs(sparse - dense) / dense < 1e-12


def test_block_sparse_flops_counts_kept_blocks():
    L = 1000                                   # 8 blocks, the last of 1000 - 7*128 = 104 rows
    mask = np.zeros((1, 1, 8, 8), dtype=np.uint8)
    mask[0, 0, 2, 5] = 1                        # a full 128 x 128 block
    mask[0, 0, 7, 7] = 1                        # the 104 x 104 corner block
    got = bench.block_sparse_flops([L], 1, 128, 128, False, mask)
    assert got == 2.0 * 256 * (128 * 128 + 104 * 104)
    got_c = bench.block_sparse_flops([L], 1, 128, 128, True, mask)
    assert got_c == 2.0 * 256 * (0 + 104 * 104 / 2)   # block (2, 5) lies above the diagonal


def test_compulsory_bytes():
    # read q, k, v once (bf16), write o (bf16) and lse (fp32) once
    assert bench.compulsory_bytes(16384, 16, 128, 128) == 16384 * 16 * (3 * 256 + 256 + 4)


def test_traffic_record_is_keyed_to_the_kernel_source(tmp_path, monkeypatch):
    wl = "noncausal_b4h16n4096d128"
    variant = "tau=8.0,poly=0,schedule=0"
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    os.makedirs(tmp_path / "profiles")
    for rel in sum(bench.KERNEL_SOURCES.values(), []):
        dst = tmp_path / rel
        os.makedirs(dst.parent, exist_ok=True)
        dst.write_text("kernel source v1\n" + rel)
    rec = {"kernel_source_sha256_16": bench.kernel_source_hash("bf16"), "variant": variant,
           "hbm_bytes_per_launch": 123}
    (tmp_path / "profiles" / f"traffic_{wl}.json").write_text(json.dumps(rec))
    assert bench.load_traffic(wl, variant) == 123
    assert bench.load_traffic(wl, "tau=0.0,poly=0,schedule=0") is None      # another variant
    assert bench.load_traffic(wl, "fp8") is None                            # no FP8 record
    (tmp_path / bench.KERNEL_SOURCES["bf16"][0]).write_text("kernel source v2")
    assert bench.load_traffic(wl, variant) is None                          # source changed


def test_committed_traffic_records_match_the_sources():
    """The committed records are for the kernel sources in the tree (else the
    benchmark reports traffic as null, which is allowed but worth knowing)."""
    assert bench.load_traffic("noncausal_b4h16n4096d128", "tau=8.0,poly=0,schedule=0") is not None
    assert bench.load_traffic("noncausal_b4h16n4096d128", "fp8") is not None


def test_more_than_one_gpu_is_refused():
    import subprocess
    import sys
    r = subprocess.run([sys.executable, os.path.join(bench.ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2 and "single-GPU" in r.stderr


@pytest.mark.parametrize("flag", ["--bwd", "--fp8"])
def test_stats_only_for_the_bf16_forward(flag):
    """--stats reads the bf16 forward kernel's counters: with the backward or
    FP8 pass it is refused before any GPU work."""
    import subprocess
    import sys
    r = subprocess.run([sys.executable, os.path.join(bench.ROOT, "bench.py"), "--stats", flag],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode != 0 and "--stats" in r.stderr


def test_source_hash_ignores_comments(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    for rel in sum(bench.KERNEL_SOURCES.values(), []):
        dst = tmp_path / rel
        os.makedirs(dst.parent, exist_ok=True)
        dst.write_text("int f() {  // one\n  return 1; /* two */\n}\n")
    h0 = bench.kernel_source_hash("bf16")
    (tmp_path / bench.KERNEL_SOURCES["bf16"][0]).write_text("// new words\nint f() {  // other\n\n  return 1;\n}\n")
    assert bench.kernel_source_hash("bf16") == h0
    (tmp_path / bench.KERNEL_SOURCES["bf16"][0]).write_text("int f() {\n  return 2;\n}\n")
    assert bench.kernel_source_hash("bf16") != h0
