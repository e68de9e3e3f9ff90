"""Host-side checks of the benchmark script (no GPU): the one-GPU contract and
the traffic records it reads."""
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, cwd=ROOT, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_traffic_records_are_well_formed():
    """profiles/traffic.json: every record names the kernel, its counters and
    the sources whose hash decides whether bench.py may report it."""
    t = json.load(open(os.path.join(ROOT, "profiles", "traffic.json")))
    assert t["fetch_scale"] > 0 and t["write_scale"] > 0
    for name in ("stack_t8_2bit", "prefill"):
        rec = t[name]
        assert rec["fetch_kib"] > 0 and rec["write_kib"] >= 0
        assert len(rec["sources_sha256"]) == 64
        for src in rec["sources"]:
            assert os.path.exists(os.path.join(ROOT, src)), src
        assert os.path.exists(os.path.join(ROOT, rec["profile"]))
