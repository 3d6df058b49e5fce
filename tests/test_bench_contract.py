"""Host-side parts of bench.py's contract (no GPU needed): more than one GPU is
refused with a message, and the HBM traffic of the dominant kernel is taken
from the committed counter summary only while the kernel sources are the ones
the counters were measured on."""
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=60)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_counter_traffic_follows_the_kernel_sources(tmp_path, monkeypatch):
    sys.path.insert(0, ROOT)
    import bench
    d = json.load(open(os.path.join(ROOT, "profiles", "counters.json")))
    e = d["ffn_gate_up"]
    # the summary's own sources give its traffic
    monkeypatch.setattr(bench, "kernel_source_hash", lambda: e["source_hash"])
    assert bench.counter_traffic("ffn_gate_up", 0) == e["hbm_bytes_per_launch"]
    # traffic = FETCH_SIZE x factor + WRITE_SIZE x factor, in KiB per launch
    assert e["hbm_bytes_per_launch"] == round((e["fetch_kib"] * e["fetch_factor"] + e["write_kib"] * e["write_factor"])
                                              * 1024)
    # any other source hash gives no traffic
    monkeypatch.setattr(bench, "kernel_source_hash", lambda: "0" * 16)
    assert bench.counter_traffic("ffn_gate_up", 0) is None
    assert bench.counter_traffic("no_such_kernel", 0) is None
