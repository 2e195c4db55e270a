"""Host-side rules of bench.py that need no GPU: the counter-derived traffic figure is reported only
for the shape and kernel source it was measured on, and a multi-GPU request is refused."""

import os
import subprocess
import sys

import bench
from token_sparse_attention_amd.configs import CONFIGS

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_traffic_only_for_the_profiled_shape():
    kv = dict(ln.split(":", 1) for ln in open(bench.TRAFFIC_FILE) if ":" in ln and not ln.startswith("#"))
    kv = {k.strip(): v.strip() for k, v in kv.items()}
    prof = CONFIGS[4]
    assert (kv["workload_L"], kv["workload_Hq"], kv["workload_d"]) == (str(prof.L), str(prof.Hq), str(prof.d))
    t = bench.measured_traffic(prof)
    if kv["attention_source_sha256_16"] == bench.source_hash(bench.ATTN_SOURCE):
        assert t == int(kv["hbm_bytes_per_launch"])
    else:
        assert t is None
    # the 256K chain has another shape: its launch was never counted
    assert bench.measured_traffic(CONFIGS[5]) is None
    assert bench.measured_traffic(CONFIGS[2]) is None


def test_traffic_null_when_source_changed(monkeypatch):
    monkeypatch.setattr(bench, "source_hash", lambda path: "0000000000000000")
    assert bench.measured_traffic(CONFIGS[4]) is None


def test_multi_gpu_request_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=300, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""
