"""bench.py's host logic on the CPU: the work it counts, the profile files it
reads, the clock reading, and its refusals without one GPU."""
import os
import subprocess
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def brute_pairs(n_q, n_kv, causal, lq, lkv):
    total = 0
    for Lq, Lk in zip(lq, lkv):
        for i in range(Lq):
            for j in range(Lk):
                if not causal or j <= i:
                    total += 1
    return total


@pytest.mark.parametrize("causal", [False, True])
def test_legal_pairs_matches_brute_force(causal):
    rng = np.random.default_rng(5)
    for n_q, n_kv in ((7, 7), (9, 5), (5, 13), (64, 80)):
        lq = rng.integers(0, n_q + 1, size=3)
        lkv = rng.integers(0, n_kv + 1, size=3)
        assert bench.legal_pairs(n_q, n_kv, causal, lq, lkv, 3) == brute_pairs(n_q, n_kv, causal, lq, lkv)
    assert bench.legal_pairs(16, 16, causal) == brute_pairs(16, 16, causal, [16], [16])


def test_decoder_work_counts():
    # causal [32, 8, 256, 64]: n(n+1)/2 pairs per head, 4*d FLOPs per pair;
    # Q, K, V read and O written once
    pairs = bench.legal_pairs(256, 256, True, batch=32) * 8
    assert pairs == 32 * 8 * 256 * 257 // 2
    assert pairs * 4 * 64 == 2155872256
    assert 4 * 32 * 8 * 256 * 64 * 2 == 33554432


def test_read_traffic_checks_the_source_hash(tmp_path, monkeypatch):
    prof = tmp_path / "profiles"
    prof.mkdir()
    good = bench.kernel_source_hash("decoder")
    (prof / "traffic_decoder.txt").write_text(
        "# comment: 1\nkernel_source_hash: %s\nhbm_bytes_per_launch: 1234\n" % good)
    (prof / "traffic_encoder.txt").write_text("kernel_source_hash: 0000000000000000\nhbm_bytes_per_launch: 99\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    # kernel_source_hash reads the sources under ROOT: keep the real ones
    monkeypatch.setattr(bench, "kernel_source_hash", lambda w, _h=good: _h)
    assert bench.read_traffic("decoder") == 1234.0
    assert bench.read_traffic("encoder") is None          # taken on other sources
    assert bench.read_traffic("cross") is None            # no file


def test_committed_traffic_files_parse():
    for w in bench.KERNEL_FILES:
        path = os.path.join(ROOT, "profiles", f"traffic_{w}.txt")
        kv = {}
        for line in open(path):
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                kv[k.strip()] = v.strip()
        assert len(kv["kernel_source_hash"]) == 16
        assert float(kv["hbm_bytes_per_launch"]) > 0
        assert float(kv["ratio_to_algorithmic"]) >= 0.99


def test_read_sclk_takes_the_current_level(tmp_path):
    f = tmp_path / "pp_dpm_sclk"
    f.write_text("S: 127Mhz\n0: 500Mhz\n1: 2137Mhz *\n")
    assert bench.read_sclk(str(f)) == 2137
    f.write_text("0: 500Mhz\n1: 2400Mhz\n")
    assert bench.read_sclk(str(f)) is None
    assert bench.read_sclk(str(tmp_path / "missing")) is None


def test_trials_info():
    t = bench.trials_info([0.3, 0.1, 0.2])
    assert t == {"replays": 3, "min_ms": 0.1, "median_ms": 0.2, "max_ms": 0.3}


def run_bench(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args],
                          capture_output=True, text=True, timeout=300)


def test_more_than_one_gpu_is_refused():
    r = run_bench("--gpus", "2")
    assert r.returncode == 2
    assert "one GPU" in r.stderr


@pytest.mark.skipif(os.environ.get("HIP_VISIBLE_DEVICES") is None and os.path.exists("/dev/kfd"),
                    reason="a GPU may be present")
def test_no_gpu_is_an_error():
    r = run_bench("--steps", "1", "--warmup", "0")
    assert r.returncode == 1
    assert "needs a GPU" in r.stderr


def test_hot_context_is_context_only():
    import types
    cold = types.SimpleNamespace(hot=False)
    assert bench.hot_context(None, cold) == {}
    assert bench.hot_context((0.008, [0.008, 0.009]), types.SimpleNamespace(hot=True)) == {}
    out = bench.hot_context((0.008, [0.008, 0.009, 0.007]), cold, flops=2e9, algo_bytes=32e6)
    assert out["hot_ms_per_step"] == 0.008
    assert abs(out["hot_tflops"] - 250.0) < 1e-9 and abs(out["hot_gbs_algorithmic"] - 4000.0) < 1e-9
    assert out["hot_trials"]["median_ms"] == 0.008 and "value" not in out
