"""Host-side checks of the benchmark script: the one-GPU contract and the
committed HBM traffic and SQ counter records it reports from."""
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, "bench.py", "--gpus", "2"], cwd=ROOT, capture_output=True, text=True,
                       timeout=120)
    assert r.returncode == 2
    msg = json.loads(r.stdout.strip().splitlines()[-1])
    assert "one GPU" in msg["error"]


def test_traffic_record_is_consistent():
    with open(os.path.join(ROOT, "profiles", "traffic_headline.json")) as f:
        tr = json.load(f)
    assert abs(tr["bytes_per_launch"] - tr["fetch_bytes"] - tr["write_bytes"]) < 1.0
    # X is read once and the outputs written once at least
    assert tr["bytes_per_launch"] >= tr["algorithmic_bytes"]
    assert abs(tr["traffic_over_algorithmic"] - tr["bytes_per_launch"] / tr["algorithmic_bytes"]) < 1e-9
    assert len(tr["source_hash"]) == 16


def test_counters_record_is_consistent():
    """The committed SQ counter record: its derived fractions follow from its
    own counter means, and every fraction lies in [0, 1]."""
    with open(os.path.join(ROOT, "profiles", "counters_headline.json")) as f:
        cr = json.load(f)
    assert len(cr["source_hash"]) == 16
    for kn, cs in cr["kernels"].items():
        d = cr["derived"][kn]
        busy = (cs["SQ_VALU_MFMA_BUSY_CYCLES"] / cr["n_simd"]) / (cs["SQ_BUSY_CYCLES"] / cr["n_se"])
        assert abs(d["mfma_busy_frac"] - busy) < 1e-12
        assert abs(d["wave_issue_frac"] - cs["SQ_ACTIVE_INST_ANY"] / cs["SQ_WAVE_CYCLES"]) < 1e-12
        for key in ("mfma_busy_frac", "wave_issue_frac", "wave_wait_frac"):
            assert 0.0 <= d[key] <= 1.0
