"""Host-side checks of bench.py: it refuses more than one GPU before touching
one, whatever the workload, and the stored HBM-traffic record it reads has
the fields it uses."""

import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.parametrize("extra", [[], ["--config", "4"], ["--config", "6"], ["--config", "3"]])
def test_more_than_one_gpu_is_refused(extra):
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"] + extra,
                       capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2, r.stderr
    msg = json.loads(r.stdout.strip().splitlines()[-1])
    assert msg["n_gpus"] == 2 and "one GPU" in msg["error"]


def test_traffic_record_fields():
    with open(os.path.join(ROOT, "profiles", "traffic_isd_step_serving.json")) as f:
        tr = json.load(f)
    for key in ("kernel_digest", "config", "bytes_per_launch", "algorithmic_bytes_per_launch",
                "fetch_kib_per_dispatch", "write_kib_per_dispatch", "fetch_scale", "write_scale",
                "commands"):
        assert key in tr, key
    assert len(tr["kernel_digest"]) == 16
    # the record's bytes follow from its counters and calibration scales
    b = tr["fetch_kib_per_dispatch"] * 1024 * tr["fetch_scale"] + \
        tr["write_kib_per_dispatch"] * 1024 * tr["write_scale"]
    assert abs(b - tr["bytes_per_launch"]) <= 1024
    assert tr["bytes_per_launch"] >= tr["algorithmic_bytes_per_launch"]


def test_counter_records_match_the_kernel_sources():
    """bench.py reports counter-derived traffic only while the sources a record
    was taken from are unchanged; both committed records must be current."""
    import importlib.util
    spec = importlib.util.spec_from_file_location("bench_mod", os.path.join(ROOT, "bench.py"))
    b = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(b)
    with open(b.TRAFFIC_FILE) as f:
        assert json.load(f)["kernel_digest"] == b.kernel_digest()
    with open(b.HEAD_TRAFFIC_FILE) as f:
        assert json.load(f)["kernel_digest"] == b.kernel_digest(b.HEAD_SOURCES)
