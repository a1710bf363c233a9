"""Host-side checks of bench.py (no GPU): the one-GPU contract and the
algorithmic byte and FLOP counts its roofline figures divide by."""
import os
import subprocess
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
import workloads as wl  # noqa: E402


def test_more_than_one_gpu_is_refused_with_a_message():
    p = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert p.returncode == 2
    assert "one GPU" in p.stderr
    assert p.stdout == ""


def test_decode_bytes_and_flops():
    # Each of the 64 adapters' A [4096, 16] and B [16, 4096] once, x once, y
    # read and written once, fp16.
    w = wl.llama7b_decode(seed=0)
    assert bench.algorithmic_bytes(w) == 64 * (4096 * 16 + 16 * 4096) * 2 + 64 * 4096 * 2 * 3
    assert bench.algorithmic_bytes(w) == 18350080
    assert bench.algorithmic_flops(w) == 2 * 64 * 16 * (4096 + 4096)


def test_bytes_count_covered_rows_and_nonempty_segments_only():
    # 3 segments (one empty) covering rows 0..4 of 7: uncovered rows and the
    # empty segment move nothing.
    w = wl.make_workload("t", "f16", 32, 48, 8, 4, [2, 0, 3], [1, 2, 3], 1.0, seed=1, num_rows=7)
    e = 2
    want = 2 * (32 * 8 + 8 * 48) * e + 5 * 32 * e + 2 * 5 * 48 * e
    assert bench.algorithmic_bytes(w) == want
    assert bench.algorithmic_flops(w) == 2 * 5 * 8 * (32 + 48)
    assert int(np.asarray(w.seg_lengths).sum()) == 5
