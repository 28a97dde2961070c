"""Host-side logic of bench.py (no GPU): the one-GPU guard, the algorithmic byte count of a
decode step and the shared/unshared cache accounting."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from synth.workloads import W2, W5  # noqa: E402

GiB = 1 << 30


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_decode_step_bytes_w2():
    B, N, K, k, D, W, Hq = 32, 65536, 256, 2048, 128, 128, 16
    ab = bench.algorithmic_bytes(W2)
    # one scoring launch: bf16 keys of every entry and the index query; the fp32 score per
    # entry is an intermediate, reported beside it
    assert ab["score_launch"] == B * (N * K * 2 + K * 2) == 1_073_758_208
    assert ab["score_spill"] == B * N * 4
    # the four layers add their attention reads/writes, two selections and Full's new row on top
    record = D // 2 + D // 32 * 4
    attend = B * (k * record + 2 * W * D * 2 + Hq * D * 2 + Hq * D * 4 + Hq * 4)
    select = B * k * 4
    full = B * (D * 4 + record + K * 2 * 2)
    assert ab["step"] == 2 * ab["score_launch"] + 4 * (attend + select) + 2 * select + full


def test_decode_step_bytes_w5_headline():
    B, N, K = 64, 131072, 256
    ab = bench.algorithmic_bytes(W5)
    assert ab["score_launch"] == B * (N * K * 2 + K * 2)
    # 8 selecting layers of the 16 stream every key once each: 99 % of the step's bytes
    assert 0.99 < 8 * ab["score_launch"] / ab["step"] < 1.0


@pytest.mark.parametrize("wl,shared_fp4,shared_keys,ratio", [
    (W5, 2.5 * GiB, 16 * GiB, 4.0),   # 4 groups of 4 layers: 4 stored copies instead of 16
    (W2, 0.15625 * GiB, 1 * GiB, 4.0),
])
def test_cache_accounting_shared_vs_unshared(wl, shared_fp4, shared_keys, ratio):
    c = bench.cache_accounting(wl)
    s = c["shared_bytes"]
    assert s["fp4_codes"] + s["fp4_scales"] == shared_fp4
    assert s["index_keys"] == shared_keys
    assert c["ratio"] == ratio
    assert c["unshared_total"] == ratio * c["shared_total"]
