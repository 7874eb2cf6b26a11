"""Host-side checks of bench.py's contract (no GPU): more than one GPU is refused with a
message and exit status 2, and the HBM-traffic record is read only when its source
fingerprint matches."""
import importlib.util
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench():
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2, r.stdout + r.stderr
    msg = json.loads(r.stdout.strip().splitlines()[-1])
    assert "one GPU" in msg["error"]


def test_source_fingerprint_is_stable():
    b = _bench()
    a1, a2 = b.kernel_source_sha(), b.kernel_source_sha()
    assert a1 == a2 and len(a1) == 64


def test_traffic_record_needs_a_matching_fingerprint():
    b = _bench()
    recorded = None
    for line in open(b.COUNTERS):
        if line.startswith("kernel_source_sha256:"):
            recorded = line.split(":", 1)[1].strip()
    assert recorded, "the counter summary records the fingerprint it was taken on"
    t = b.counters_for(recorded)
    assert isinstance(t, float) and t > 5e8          # the dLLM launch moves about 544 MB
    assert b.counters_for("0" * 64) is None
