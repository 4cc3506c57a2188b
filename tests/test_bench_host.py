"""bench.py's host-side logic on the CPU (nothing here touches a GPU): the
one-GPU contract, the expected accepted length, the committed traffic lookup
and its source-hash guard."""
import os
import subprocess
import sys

import bench
import workloads as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr
    assert r.stdout == ""


def test_expected_accepted_length():
    # E[n] = (1 - p^K) / (1 - p): the number of accepted tokens when each
    # candidate matches independently with probability p (the n-th emitted
    # token is the AR view's, so n >= 1 and n <= K)
    cfg = W.CONFIGS[3]                      # p = 0.85, K = 32
    p, K = 0.85, cfg.K
    direct = sum(p ** i for i in range(K))  # P(n > i) summed over i
    assert abs(bench.expected_n(cfg) - direct) < 1e-12
    assert abs(bench.expected_n(cfg) - 6.63) < 5e-3
    assert bench.expected_n(cfg.with_(K=1)) == 1.0


def test_traffic_is_read_only_while_the_sources_match(tmp_path, monkeypatch):
    # the committed headline summary, when it matches the current attention
    # sources, is at least the launch's algorithmic bytes
    t = bench.measured_traffic("qwen3-8b-36layers", 0)
    assert t is None or t > 34_213_888
    # a forced split count is another launch: no committed figure applies
    assert bench.measured_traffic("qwen3-8b-36layers", 26) is None
    # a summary recorded for other sources is ignored
    h = bench.attn_source_hash()
    monkeypatch.setattr(bench, "attn_source_hash", lambda sources=None: h)
    prof = tmp_path / "profiles"
    prof.mkdir()
    (prof / "block_attn_w_traffic.txt").write_text(
        "source_hash: 0000000000000000\ntraffic_bytes_per_launch: 123\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.measured_traffic("w", 0) is None
    (prof / "block_attn_w_traffic.txt").write_text(
        f"source_hash: {h}\ntraffic_bytes_per_launch: 123\n")
    assert bench.measured_traffic("w", 0) == 123
