"""bench.py's command line on the CPU: more than one GPU is refused with a
message (the library measures one GPU), before any GPU work."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2", "--steps", "1"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_traffic_hash_names_existing_sources():
    """The measured-traffic figure is tied to source files that exist."""
    import importlib.util
    spec = importlib.util.spec_from_file_location("bench_mod", os.path.join(ROOT, "bench.py"))
    m = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(m)
    h = m.kernel_sources_hash()
    assert len(h) == 64
    assert m.TRAFFIC_MEASURED["read_bytes"] > 0 and m.TRAFFIC_MEASURED["write_bytes"] > 0
