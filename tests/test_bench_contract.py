"""Host-side checks of the benchmark script: the committed traffic records match the
kernel sources they were measured on, and a request for several GPUs is refused."""

import glob
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def _records():
    out = []
    for path in sorted(glob.glob(os.path.join(ROOT, "profiles", "hbm_traffic_*.md"))):
        with open(path) as fh:
            for line in fh:
                if line.startswith("traffic-record:"):
                    out.append((os.path.basename(path), json.loads(line.split(":", 1)[1])))
    return out


def test_traffic_records_exist():
    assert _records(), "no committed traffic record under profiles/"


@pytest.mark.parametrize("name,rec", _records())
def test_traffic_record_matches_current_sources(name, rec):
    # bench.py reports roofline.traffic only while the kernel's sources hash to the
    # recorded value; a kernel change must come with freshly taken counters
    assert rec["src_sha256"] == bench.sources_sha256(rec["kernel"]), name
    assert name == f"hbm_traffic_{rec['kernel']}_{rec['workload']}.md"
    assert rec["bytes_per_launch"] == rec["read_bytes"] + rec["write_bytes"]
    assert bench.measured_traffic(rec["kernel"], rec["workload"]) == rec["bytes_per_launch"]


def test_several_gpus_are_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""
