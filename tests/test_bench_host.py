"""bench.py's host-side logic (no GPU): the one-GPU contract, the flop table behind every TFLOP/s
figure, and the rule that a committed HBM-traffic record is used only while the kernel's sources are
the ones it was measured on."""
import hashlib
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


@pytest.mark.parametrize("argv,env", [(["--gpus", "2"], {}), ([], {"WORLD_SIZE": "4"})], ids=["gpus2", "world4"])
def test_more_than_one_gpu_exits_with_a_message(argv, env):
    e = dict(os.environ, **env)
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py")] + argv, capture_output=True,
                       text=True, env=e, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""  # no JSON line


def causal(T):
    return T * (T + 1) // 2


def test_flop_table_counts_causal_entries():
    # one ordinary and one replaced head, B = 1: per causal entry 4d (S, PV) forward, 8d (S, dP, dV,
    # dK) in bwd_kv, 2d (dQ) in bwd_dq; a replaced head 2d (PV) forward and 2d (dV) backward
    T, d = 100, 64
    kf = bench.kernel_flops(1, T, d, [0, 1])
    c = causal(T)
    assert kf["mixed_fwd"] == c * (4 * d + 2 * d)
    assert kf["bwd_kv"] == c * (8 * d + 2 * d)
    assert kf["bwd_dq"] == c * 2 * d
    assert kf["bwd_pre"] == 0


@pytest.mark.parametrize("rep", [[0] * 8, [1] * 8, [0, 0, 0, 1] * 2, [1, 0] * 4])
def test_flop_table_is_additive(rep):
    T, d = 257, 128
    one = bench.kernel_flops(1, T, d, rep)
    three = bench.kernel_flops(3, T, d, rep)
    for k in one:
        assert three[k] == 3 * one[k]  # linear in the batch
    # the layer is the sum of its heads
    per_head = [bench.kernel_flops(1, T, d, [x]) for x in rep]
    for k in one:
        assert one[k] == sum(ph[k] for ph in per_head)
    assert bench.total_flops(1, T, d, rep, True) == one["mixed_fwd"] + one["bwd_kv"] + one["bwd_dq"]
    assert bench.total_flops(1, T, d, rep, False) == one["mixed_fwd"]


def test_traffic_record_follows_its_sources(tmp_path, monkeypatch):
    csrc = tmp_path / "fixed_pattern_mixed_amd" / "csrc"
    csrc.mkdir(parents=True)
    (tmp_path / "profiles").mkdir()
    src = csrc / "k.hip"
    src.write_text("kernel v1\n")
    h = hashlib.sha256(src.read_bytes()).hexdigest()
    rec = {"w": {"kern": {"bytes": 1234, "sources": ["k.hip"], "source_sha256": h}}}
    (tmp_path / "profiles" / "hbm_traffic.json").write_text(json.dumps(rec))
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.measured_traffic("w", "kern") == 1234
    assert bench.measured_traffic("w", "other") is None
    assert bench.measured_traffic("x", "kern") is None
    src.write_text("kernel v2\n")  # the kernel changed since the counters were taken
    assert bench.measured_traffic("w", "kern") is None


def test_step_spread():
    """Median (middle value, or the mean of the middle two), minimum and maximum of the per-step
    durations; nothing for no steps."""
    import bench
    assert bench.step_spread([1.0, 3.0, 2.0, 5.0]) == {"median": 2.5, "min": 1.0, "max": 5.0, "n": 4}
    assert bench.step_spread([2.0, 9.0, 4.0]) == {"median": 4.0, "min": 2.0, "max": 9.0, "n": 3}
    assert bench.step_spread([]) is None


def test_backward_unit():
    """The backward as one unit: the summed durations of its kernels (whichever dQ kernel ran) and
    the algorithmic flops of the key-block work plus one dQ product; nothing for forward-only runs."""
    import bench
    rep = [0, 0, 0, 1] * 4
    kf = bench.kernel_flops(2, 8192, 128, rep)
    ks = {"bwd_pre": {"avg_ms": 0.02}, "bwd_kv": {"avg_ms": 1.0}, "bwd_dq_ds": {"avg_ms": 0.38},
          "mixed_fwd": {"avg_ms": 0.5}}
    u = bench.backward_unit(ks, kf)
    assert u["kernels"] == ["bwd_pre", "bwd_kv", "bwd_dq_ds"] and abs(u["ms"] - 1.4) < 1e-9
    assert abs(u["tflops"] - (kf["bwd_kv"] + kf["bwd_dq"]) / 1.4e-3 / 1e12) < 0.1
    assert bench.backward_unit({"mixed_fwd": {"avg_ms": 0.5}}, kf) is None
