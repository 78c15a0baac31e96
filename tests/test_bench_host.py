"""Host-side logic of bench.py (no GPU): the one-GPU guard, the algorithmic
byte count the roofline divides by, and the key that ties the recorded HBM
traffic counters to the fused kernel's code."""

import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
import synth  # noqa: E402


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=60)
    assert r.returncode == 2
    assert "single GPU" in r.stderr
    assert r.stdout == ""


def test_algorithmic_bytes_of_the_13b_step():
    # the d-wide slab of every cached token once per KV head, plus k full key
    # rows and k full value rows per query head, bf16
    w = synth.WORKLOADS["l2_13b_run"]
    by = bench.algorithmic_bytes(w, 3584, 896)
    assert by["slab"] == 16 * 40 * 3584 * 32 * 2
    assert by["rows"] == 16 * 40 * 896 * 2 * 128 * 2
    assert by["total"] == 440_401_920
    assert by["dense"] == 16 * 40 * 3584 * 2 * 128 * 2
    assert by["dense"] / by["total"] == 2.6666666666666665


def test_code_tokens_ignore_comments_and_layout_only():
    a = "int f(int x) {\n  return x + 1;  // one more\n}\n"
    b = "int f(int x) {   return x + 1;\n\n}  // reformatted, new comment\n"
    c = "int f(int x) {\n  return x + 2;\n}\n"
    assert bench.code_tokens(a) == bench.code_tokens(b)
    assert bench.code_tokens(a) != bench.code_tokens(c)


def test_recorded_traffic_only_for_its_kernel_hash():
    h = bench.kernel_source_hash()
    assert len(h) == 16
    t = bench.measured_traffic(h, "l2_13b_run")
    if t is not None:  # recorded on the current kernel code
        assert 400e6 < t < 480e6
    assert bench.measured_traffic("0" * 16, "l2_13b_run") is None
    assert bench.measured_traffic(h, "no_such_workload") is None


def test_design_bytes_per_path():
    # a toy grouped-query shape, bf16: B=1, Hq=4, Hkv=2, D=8, d=2, S=10, k=3
    import dataclasses
    import numpy as np
    w = dataclasses.replace(synth.WORKLOADS["l3_8b_gqa"], B=1, Hq=4, Hkv=2, D=8, d=2)
    idx = np.array([[[0, 1, 2], [1, 2, 3], [5, 6, 7], [5, 6, 7]]])
    slab, ids, scores = 1 * 2 * 10 * 2 * 2, 4 * 3 * 4, 2 * 4 * 10 * 4
    row = (2 * 8 - 2) * 2
    assert bench.design_bytes(w, 10, 3, "split", idx) == slab + ids + scores + 4 * 3 * row
    # union: KV head 0 gathers {0,1,2,3}, KV head 1 gathers {5,6,7}
    assert bench.design_bytes(w, 10, 3, "union", idx) == slab + ids + scores + 7 * row
    # fused: the slab once per query head
    assert bench.design_bytes(w, 10, 3, "fused", idx) == 2 * slab + ids + 4 * 3 * row
    # sliced: 4 rows of k = 3 take one slice each (at least 64 kept tokens
    # per slice), so there is nothing to exchange
    assert bench.sliced_slices(4, 3) == 1
    assert bench.design_bytes(w, 10, 3, "sliced", idx) == 2 * slab + ids + 4 * 3 * row
    # with slices: each row's S scores written once and read by the other
    # slices (S * nsl floats), and nsl - 1 partials written and read
    assert bench.sliced_slices(32, 1024) == 8
    assert bench.sliced_slices(640, 896) == 1 and bench.sliced_slices(576, 896) == 4
    w2 = dataclasses.replace(w, B=1, Hq=32, Hkv=32)
    idx2 = np.tile(np.arange(1024), (1, 32, 1))
    base = bench.design_bytes(w2, 4096, 1024, "fused", idx2)
    assert bench.design_bytes(w2, 4096, 1024, "sliced", idx2) == base + 32 * (4096 * 4 * 8 + 2 * 7 * 10 * 4)
