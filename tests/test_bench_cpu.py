"""Host-side contract of bench.py (no GPU).

* A run asked for more than one GPU exits with status 2 and says why,
  before touching a device.
* The HBM traffic figure of the dominant kernel is read from its committed
  summary only while the kernel sources still hash to the digest stamped in
  that summary; any other digest gives null.
"""
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr and "--gpus 2" in r.stderr
    assert r.stdout.strip() == ""


def test_traffic_follows_the_source_digest(monkeypatch):
    cases = [(k, c) for k in ("projection", "sparse_grad_weight") for c in ("headline", "headline_fp8")]
    for k, c in cases:
        path = bench.traffic_file(k, c)
        assert os.path.exists(path), path
        stamped = [l.split(":", 1)[1].strip() for l in open(path) if l.startswith("source_sha256:")]
        assert len(stamped) == 1 and len(stamped[0]) == 64
    fresh = {kc: bench.read_traffic(*kc) for kc in cases}
    if all(v is not None for v in fresh.values()):
        for kc, v in fresh.items():
            assert v > 1e9, (kc, v)         # several GB per launch at the headline shape
    monkeypatch.setattr(bench, "source_digest", lambda: "0" * 64)
    assert all(bench.read_traffic(*kc) is None for kc in cases)
