"""Host-side pieces of bench.py (no GPU): the one-GPU guard, the sysfs clock
reader, and the rule that counter-derived traffic is used only when it was
taken on the current kernel source for the same workload."""
from __future__ import annotations

import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr
    assert r.stdout == ""


def test_clock_reader_starts_no_process(monkeypatch):
    def refuse(*a, **k):
        raise AssertionError("gpu_clocks started a process")
    monkeypatch.setattr(subprocess, "run", refuse)
    monkeypatch.setattr(subprocess, "Popen", refuse)
    c = bench.gpu_clocks()
    assert c is None or all(set(e) == {"card", "sclk_mhz", "power_cap_w"} for e in c)


def _profile(tmp_path, sha, workload, value):
    d = tmp_path / "profiles"
    d.mkdir(exist_ok=True)
    (d / "traffic_gqa_partial_b16_m256_n4096.md").write_text(
        f"# traffic\n\nworkload: {workload}\nkernel_source_sha256: {sha}\n"
        f"traffic_bytes_per_launch: {value}\n")


def test_traffic_only_from_the_current_source(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    cur = bench.kernel_source_sha()
    _profile(tmp_path, cur, "gqa_b16_m256_n4096", 2.5e7)
    assert bench.read_traffic("gqa_b16_m256_n4096") == 2.5e7
    _profile(tmp_path, "0" * 64, "gqa_b16_m256_n4096", 2.5e7)
    assert bench.read_traffic("gqa_b16_m256_n4096") is None
    _profile(tmp_path, cur, "gqa_b2_m256_n4096", 2.5e7)
    assert bench.read_traffic("gqa_b16_m256_n4096") is None
    assert bench.read_traffic("gqa_b64_m8_n8192") is None   # no summary at all


def test_oracle_thread_count_changes_no_result():
    """The single-core timing of the CPU baseline sets the oracle's thread
    count; every output row is one thread's work in a fixed order, so the
    bits do not depend on it."""
    import numpy as np
    import oracle
    from gqa_attention_split_amd.inputs import make_qkv
    q, k, v = make_qkv(2, 40, 300, seed=5)
    n_all = oracle.threads()
    a = oracle.gqa_f64(q, k, v)
    oracle.set_threads(1)
    try:
        b = oracle.gqa_f64(q, k, v)
        assert oracle.threads() == 1
    finally:
        oracle.set_threads(n_all)
    assert oracle.threads() == n_all
    assert np.array_equal(a, b)


def test_load_clock_only_from_the_current_source(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    d = tmp_path / "profiles"
    d.mkdir()
    f = d / "counters_gqa_partial_b16_m256_n4096.md"
    f.write_text(f"kernel_source_sha256: {bench.kernel_source_sha()}\nload_clock_ghz: 2.05\n")
    assert bench.read_load_clock("gqa_b16_m256_n4096") == 2.05
    f.write_text("kernel_source_sha256: " + "0" * 64 + "\nload_clock_ghz: 2.05\n")
    assert bench.read_load_clock("gqa_b16_m256_n4096") is None
    assert bench.read_load_clock("gqa_b64_m8_n8192") is None
    # the QK-normalised path reads its own pass
    g = d / "counters_gqa_partial_qknorm_b16_m256_n4096.md"
    g.write_text(f"kernel_source_sha256: {bench.kernel_source_sha()}\nload_clock_ghz: 1.89\n")
    assert bench.read_load_clock("gqa_b16_m256_n4096", qk_norm=True) == 1.89
    assert bench.read_load_clock("gqa_b16_m256_n4096") is None
