"""Host-side parts of bench.py (no GPU): the one-GPU refusal, the per-expert byte
count the bandwidth figures use, and the traffic record the roofline reads."""
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""


def test_expert_bytes_at_the_headline_shape():
    # gate, up and down: 3 x 2048 x 512 weights at 4 bits, plus a bf16 scale and
    # a bf16 bias per 64 weights
    assert bench.expert_bytes(2048, 512) == 3 * 2048 * 512 // 2 + 3 * 2048 * 512 // 64 * 4
    assert bench.expert_bytes(2048, 512) == 1769472


def test_traffic_record_matches_its_counters():
    """profiles/traffic.json: the figure the roofline reports is the sum of the two
    scaled counter readings, and it is used only for the kernel sources it was
    measured on."""
    rec = json.load(open(os.path.join(ROOT, "profiles", "traffic.json")))
    gu = rec["gate_up_prefill_t4096_zipf"]
    assert gu["bytes_per_launch"] == gu["read_bytes"] + gu["write_bytes"]
    assert gu["bytes_per_launch"] >= gu["algorithmic_bytes"]
    got = bench.traffic_from_profile(bench.GEMM_SOURCES, "gate_up_prefill_t4096_zipf")
    if gu["source_sha"] == bench.sources_hash(bench.GEMM_SOURCES):
        assert got == gu["bytes_per_launch"]
    else:
        assert got is None
    assert bench.traffic_from_profile(bench.GEMM_SOURCES, "no_such_record") is None
