"""bench.py's host-side contract (no GPU): it refuses more than one GPU, the
algorithmic bytes that price its roofline follow from the tiers' stored
column sizes, and the committed counter summary is used only while the
kernel sources are the ones it was taken on."""
import os
import subprocess
import sys

import bench
import workloads as WL
from workloads.accounting import gemv_algorithmic_bytes

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""   # no JSON line


def test_headline_algorithmic_bytes_by_hand():
    # 7B attention projections at skip/approx/full 40/30/30 % of 4096 inputs
    kf, ka = WL.tier_counts(4096, WL.CONFIGS[2].splits[0])
    assert (kf, ka) == (1229, 1229)
    # per launch: fp16 full columns (2 bytes per row), int4 code columns (half
    # a byte per row plus an fp16 scale per 128 rows), x (fp16), the two int32
    # index lists and y (fp16)
    o = 1229 * 4096 * 2 + 1229 * (4096 // 2 + 2 * 32) + 4096 * 2 + 4 * 2458 + 4096 * 2
    qkv = 1229 * 12288 * 2 + 1229 * (12288 // 2 + 2 * 96) + 4096 * 2 + 4 * 2458 + 12288 * 2
    assert (o, qkv) == (12_689_832, 38_033_448)
    assert gemv_algorithmic_bytes(4096, 4096, kf, ka, "fp16", "int4") == o
    assert gemv_algorithmic_bytes(12288, 4096, kf, ka, "fp16", "int4") == qkv


def test_traffic_is_null_once_the_kernel_changed(monkeypatch):
    monkeypatch.setattr(bench, "kernel_source_hash", lambda: "0" * 64)
    assert bench.measured_traffic() is None


def test_traffic_comes_from_the_committed_summary():
    text = open(bench.PMC_SUMMARY).read()
    sha = next(line for line in text.splitlines()
               if line.startswith("kernel sources sha256")).rsplit(":", 1)[1].strip()
    t = bench.measured_traffic()
    if sha == bench.kernel_source_hash():
        assert t is not None and t > 0
    else:
        assert t is None
