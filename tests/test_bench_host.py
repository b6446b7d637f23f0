"""Host-side checks of bench.py (no GPU): the one-GPU contract, the
algorithmic byte counts it divides by, and the rule that a committed HBM
traffic record is used only for its own workload, tile config and kernel
sources."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402

DEFAULT_TAG = "bm32 nr2 waves4 split_k1 stages2"


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, cwd=ROOT, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_weight_bytes_formulas():
    # INT4: K/2 code bytes + K/32 bf16 scales per row; MXFP4: K/32 E8M0 scales
    assert bench.weight_bytes(1, 16, 256) == 16 * 128 + 16 * 8 * 2
    assert bench.mx_weight_bytes(1, 16, 256) == 16 * 128 + 16 * 8
    # the EP8 decode gate/up share: 48 experts of [4096, 7168]
    assert bench.weight_bytes(48, 4096, 7168) == 792_723_456
    assert bench.weight_bytes(0, 4096, 7168) == 0


def _record():
    text = open(bench.TRAFFIC_PROFILE).read()
    start = text.index("<!-- traffic: ") + len("<!-- traffic: ")
    return json.loads(text[start:text.index(" -->", start)])


def test_traffic_record_applies_only_to_its_workload_config_and_sources(monkeypatch):
    rec = _record()
    want = int(round(rec["fetch_kib"] * 1024 * rec["fetch_factor"] + rec["write_kib"] * 1024 * rec["write_factor"]))
    if rec["sources_sha256"] != bench.kernel_sources_sha256():
        pytest.skip("kernel sources changed since the committed counters were taken")
    assert bench.measured_traffic(rec["workload"], rec["config"]) == want
    assert rec["config"] == DEFAULT_TAG and rec["workload"] == "ep8_decode"
    assert bench.measured_traffic("ep8_prefill", rec["config"]) is None
    assert bench.measured_traffic(rec["workload"], "bm16 nr2 waves4 split_k1 stages2") is None
    monkeypatch.setattr(bench, "kernel_sources_sha256", lambda: "0" * 64)
    assert bench.measured_traffic(rec["workload"], rec["config"]) is None


def test_measured_traffic_is_within_a_plausible_range_of_the_algorithmic_bytes():
    # at least the weights of the touched experts, and no more than twice the
    # algorithmic bytes (re-reads would show here first)
    rec = _record()
    traffic = rec["fetch_kib"] * 1024 * rec["fetch_factor"] + rec["write_kib"] * 1024 * rec["write_factor"]
    assert bench.weight_bytes(48, 4096, 7168) <= traffic <= 2 * 806_922_432
