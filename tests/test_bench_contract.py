"""bench.py's host-side contract (no GPU): it refuses more than one GPU, the
algorithmic bytes that price its roofline follow from the tiers' stored
column sizes, and the committed counter summary is used only while the
kernel sources are the ones it was taken on."""
import os
import subprocess
import sys

import pytest

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


def test_headline_is_the_32_layer_7b_stream():
    spec = bench.specs_for(bench.HEADLINE_CONFIG, False)[0]
    assert bench.HEADLINE_CONFIG == 4 and not spec.host
    assert (spec.hidden, spec.inter, spec.attn, spec.split) == (4096, 11008, True, (50, 25, 25))
    assert spec.tokens * spec.layers_per_token == 128 and spec.sets == 32


def test_config4_layer_bytes_by_hand():
    # 7B layer at skip/approx/full 50/25/25: 1024 + 1024 of 4096 inputs, 2752 +
    # 2752 of down's 11008; per group: fp16 full columns, int4 code columns
    # (half a byte per row plus an fp16 scale per 128 rows), x, the two int32
    # index lists, y (gate/up: a, half its stored rows)
    spec = bench.specs_for(4, False)[0]
    assert bench.group_counts(spec, 0) == (1024, 1024)
    assert bench.group_counts(spec, 3) == (2752, 2752)
    qkv = 1024 * 12288 * 2 + 1024 * (12288 // 2 + 2 * 96) + 4096 * 2 + 4 * 2048 + 12288 * 2
    o = 1024 * 4096 * 2 + 1024 * (4096 // 2 + 2 * 32) + 4096 * 2 + 4 * 2048 + 4096 * 2
    gu = 1024 * 22016 * 2 + 1024 * (22016 // 2 + 2 * 172) + 4096 * 2 + 4 * 2048 + 11008 * 2
    dn = 2752 * 4096 * 2 + 2752 * (4096 // 2 + 2 * 32) + 11008 * 2 + 4 * 5504 + 4096 * 2
    assert [bench.group_bytes(spec, g) for g in range(4)] == [qkv, o, gu, dn]
    assert bench.layer_bytes(spec) == qkv + o + gu + dn == 127_431_168


def test_traffic_is_null_once_the_kernel_changed(monkeypatch):
    monkeypatch.setattr(bench, "kernel_source_hash", lambda *a: "0" * 64)
    for layer, table in ((True, bench.PMC_SUMMARY), (False, bench.GEMV_PMC_SUMMARY)):
        for config in table:
            assert bench.measured_traffic(config, layer) is None


@pytest.mark.parametrize("layer", [True, False])
def test_traffic_comes_from_the_committed_summary(layer):
    table, sources = ((bench.PMC_SUMMARY, bench.KERNEL_SOURCES) if layer else
                      (bench.GEMV_PMC_SUMMARY, bench.GEMV_SOURCES))
    for config, path in table.items():
        if not os.path.exists(path):
            assert bench.measured_traffic(config, layer) is None
            continue
        text = open(path).read()
        sha = next(line for line in text.splitlines()
                   if line.startswith("kernel sources sha256")).rsplit(":", 1)[1].strip()
        t = bench.measured_traffic(config, layer)
        if sha == bench.kernel_source_hash(sources):
            assert t is not None and t > 0
        else:
            assert t is None
