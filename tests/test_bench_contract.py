"""Host-side checks of bench.py (CPU only): it refuses more than one GPU with
a message and exit status 2, and the HBM traffic it reports comes from a
counter record taken on the current kernel sources, else it is null."""
import importlib.util
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench_module():
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_more_than_one_gpu_is_refused():
    out = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                         text=True, timeout=60)
    assert out.returncode == 2
    assert "one GPU" in out.stderr
    assert out.stdout == ""


def test_world_size_above_one_is_refused():
    env = dict(os.environ, WORLD_SIZE="2")
    out = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py")], capture_output=True, text=True,
                         timeout=60, env=env)
    assert out.returncode == 2 and "one GPU" in out.stderr


def test_traffic_records_name_their_sources():
    with open(os.path.join(ROOT, "profiles", "hbm_traffic.json")) as f:
        table = json.load(f)
    assert table
    for key, rec in table.items():
        assert rec["sources"] and rec["source_digest"], key
        # (each of the three is rounded to whole bytes on its own)
        assert abs(rec["bytes_per_launch"] - rec["read_bytes"] - rec["write_bytes"]) <= 1, key
        for n in rec["sources"]:
            assert os.path.exists(os.path.join(ROOT, "fp8_scaled_gemm_amax_amd", "csrc", n)), (key, n)


def test_traffic_is_null_once_the_kernel_source_changes(monkeypatch):
    bench = _bench_module()
    import fp8_scaled_gemm_amax_amd.profiling as prof
    with open(os.path.join(ROOT, "profiles", "hbm_traffic.json")) as f:
        table = json.load(f)
    key, rec = next(iter(table.items()))
    monkeypatch.setattr(prof, "source_digest", lambda names: rec["source_digest"])
    assert bench.measured_traffic(key) == rec["bytes_per_launch"]
    monkeypatch.setattr(prof, "source_digest", lambda names: "0" * 16)
    assert bench.measured_traffic(key) is None
    assert bench.measured_traffic("no_such_kernel:c0") is None
