"""Host-side logic of bench.py (no GPU): the one-GPU guard, the kernel-source
digest that gates counter-derived traffic, and the algorithmic byte count of
a step."""
import importlib.util
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench():
    spec = importlib.util.spec_from_file_location("bench_mod", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_traffic_is_reported_only_for_the_profiled_sources(tmp_path, monkeypatch):
    b = _bench()
    d = b.source_digest()
    assert d == b.source_digest() and len(d) == 16
    f = tmp_path / "traffic.json"
    f.write_text(json.dumps({"source_digest": d, "cast_hbm_bytes_per_launch": 123}))
    monkeypatch.setattr(b, "TRAFFIC_FILE", str(f))
    assert b.measured_traffic() == 123
    f.write_text(json.dumps({"source_digest": "0" * 16, "cast_hbm_bytes_per_launch": 123}))
    assert b.measured_traffic() is None
    f.write_text("not json")
    assert b.measured_traffic() is None


def test_step_bytes_of_the_headline_workload():
    from precision_quantization_row_amd import workloads
    M, K = 8192, 28672
    # X read twice (amax pass, cast pass), both amax vectors written and read
    # once, both copies of codes and scales written once
    want = 2 * M * K * 2 + 2 * 4 * (M + K) + M * K // 2 + M * K // 16 + K * M // 2 + K * M // 16
    assert workloads.algorithmic_bytes(M, K, 2) == want


def test_cases_are_named_and_selectable():
    """Every group of other rows is a named case; --case accepts exactly those
    names (and rejects others before touching a GPU)."""
    b = _bench()
    assert set(b.CASES) == {"amax", "2d", "4over6", "qdq", "fp32_edge", "grouped", "small", "hw"}
    assert set(b.DEFAULT_CASES) == set(b.CASES) - {"hw"}
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--case", "nope"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2 and "invalid choice" in r.stderr


def test_cpu_model_names_the_host():
    b = _bench()
    m = b.cpu_model()
    assert isinstance(m, str) and m and m != "unknown"
