"""Host-side logic of bench.py (CPU only): the one-GPU refusal, the kernel-hash gate on the
committed rocprofv3 figures, and the internal consistency of those figures (per-launch bytes
from the counter means and the copy calibration, algorithmic bytes from the shape, a two-launch
decode as the sum of its launches, one kernel source hash across every profile file)."""
import glob
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402

H, D = 32, 128
S, P = 12400, 8304  # the two-reference edit layout's sequence and prefix lengths
N = S - P


def _load(name):
    with open(os.path.join(ROOT, "profiles", name)) as f:
        return json.load(f)


def _entries(d):
    return {k: v for k, v in d.items() if isinstance(v, dict)}


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr
    assert r.stdout == ""


def test_profile_entry_follows_the_kernel_hash(tmp_path, monkeypatch):
    path = tmp_path / "p.json"
    path.write_text(json.dumps({"k": {"kernel_source_sha256": "aa", "bytes_per_launch": 7}}))
    monkeypatch.setattr(bench, "kernel_source_sha256", lambda: "aa")
    assert bench.profile_entry(str(path), "k")["bytes_per_launch"] == 7
    assert bench.profile_entry(str(path), "missing") is None
    monkeypatch.setattr(bench, "kernel_source_sha256", lambda: "bb")
    assert bench.profile_entry(str(path), "k") is None
    assert bench.profile_entry(str(tmp_path / "absent.json"), "k") is None
    path.write_text("not json")
    assert bench.profile_entry(str(path), "k") is None


def test_traffic_and_utilisation_are_null_for_another_kernel_source(monkeypatch):
    monkeypatch.setattr(bench, "kernel_source_sha256", lambda: "0" * 64)
    assert bench.measured_traffic("prefill_b1") is None
    assert bench.mfma_utilisation() is None


def test_committed_profiles_share_one_kernel_hash():
    hashes = set()
    for name in ("hbm_traffic.json", "sq_counters.json"):
        for e in _entries(_load(name)).values():
            hashes.add(e["kernel_source_sha256"])
    assert len(hashes) == 1
    (h,) = hashes
    summaries = glob.glob(os.path.join(ROOT, "profiles", "*.md"))
    assert summaries
    for p in summaries:
        with open(p) as f:
            assert h in f.read(), os.path.basename(p)


def test_traffic_bytes_follow_counters_and_calibration():
    t = _entries(_load("hbm_traffic.json"))
    for key, e in t.items():
        kib = e["fetch_size_kib_mean"] * e["read_scale"] + e["write_size_kib_mean"] * e["write_scale"]
        assert abs(e["bytes_per_launch"] - kib * 1024) <= 1e-6 * e["bytes_per_launch"] + 1024, key
    # the cached step's two launches add up to the call
    assert t["decode_cfg_b2"]["bytes_per_launch"] == pytest.approx(
        t["decode_cfg_b2_main"]["bytes_per_launch"] + t["decode_cfg_b2_tail"]["bytes_per_launch"],
        rel=1e-9, abs=2)


def test_algorithmic_bytes_from_the_shape():
    t = _entries(_load("hbm_traffic.json"))
    # prefill, B = 1: Q, K, V read (bf16), O written (fp32), the prefix K and V written (bf16)
    pre = S * H * D * (3 * 2 + 4) + 2 * P * H * D * 2
    # cached CFG step, B = 2: target Q, K, V and the cached K, V read (bf16), O written (fp32)
    dec = 2 * H * D * (3 * N * 2 + 2 * P * 2 + N * 4)
    assert t["prefill_b1"]["algorithmic_bytes"] == pre
    assert t["decode_cfg_b2"]["algorithmic_bytes"] == dec
    for key in ("prefill_b1", "decode_cfg_b2"):
        e = t[key]
        assert e["traffic_over_algorithmic"] == pytest.approx(
            e["bytes_per_launch"] / e["algorithmic_bytes"], abs=5e-4)


def test_utilisation_fractions_are_fractions():
    for key, e in _entries(_load("sq_counters.json")).items():
        for f in ("mfma_busy_of_simd_cycles", "mfma_busy_of_busy_cu_cycles", "cu_busy_of_dispatch"):
            assert 0.0 < e[f] <= 1.0, (key, f)
        # busy-CU cycles are a subset of all cycles, so the MFMA share of them is not smaller
        assert e["mfma_busy_of_busy_cu_cycles"] >= e["mfma_busy_of_simd_cycles"] - 1e-4, key
