"""Host-side checks of bench.py that need no GPU: the one-GPU contract, and
the stored rocprofv3 traffic figures it reports as ``roofline.traffic``."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


@pytest.mark.parametrize("n", [2, 8])
def test_more_than_one_gpu_is_refused_with_a_message(n):
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", str(n)],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_source_hash_is_stable_and_short():
    h = bench.source_hash()
    assert h == bench.source_hash()
    assert len(h) == 16 and all(c in "0123456789abcdef" for c in h)


def test_stored_traffic_entries_are_well_formed():
    with open(bench.TRAFFIC_FILE) as f:
        t = json.load(f)
    entries = {k: v for k, v in t.items() if not k.startswith("_")}
    assert "nn_bf16_8192" in entries
    for name, e in entries.items():
        assert len(e["source_hash"]) == 16
        assert e["kernel"].startswith("void tdg::")
        # copy-scaled fetch and write, in bytes per launch
        want = (e["fetch_kib_per_dispatch"] * e["fetch_scale"] + e["write_kib_per_dispatch"] * e["write_scale"]) * 1024
        assert e["hbm_bytes_per_launch"] == pytest.approx(want, rel=1e-3)
        assert e["hbm_bytes_per_launch"] >= 0.9 * e["algorithmic_bytes_per_launch"] > 0
    assert bench.stored_traffic("no such workload") is None


def test_stored_traffic_is_withheld_for_other_sources(tmp_path, monkeypatch):
    with open(bench.TRAFFIC_FILE) as f:
        t = json.load(f)
    e = dict(t["nn_bf16_8192"])
    e["source_hash"] = "0" * 16 if e["source_hash"] != "0" * 16 else "1" * 16
    p = tmp_path / "traffic.json"
    p.write_text(json.dumps({"nn_bf16_8192": e}))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(p))
    assert bench.stored_traffic("nn_bf16_8192") is None
    e["source_hash"] = bench.source_hash()
    p.write_text(json.dumps({"nn_bf16_8192": e}))
    assert bench.stored_traffic("nn_bf16_8192") == e["hbm_bytes_per_launch"]
