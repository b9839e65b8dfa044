"""Host-side logic of bench.py: the committed counter records and the single-GPU guard (no GPU needed)."""
import json
import os
import re
import shutil
import subprocess
import sys

import pytest

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_counter_records_match_the_committed_sources():
    # while the committed profiles were taken from the current kernel sources both figures are reported
    t = bench.counted_traffic("exact", 256, 128)
    m = bench.counted_mfma_busy("exact", 256, 128)
    if t is None or m is None:
        pytest.skip("the committed counter profiles predate the current kernel sources")
    assert 774e6 < t < 1e11     # at least the algorithmic bytes, at most a bound
    assert 0 < m <= 100
    # another configuration has no record
    assert bench.counted_traffic("exact", 128, 128) is None
    assert bench.counted_traffic("dense", 256, 128) is None


def test_counter_records_go_stale_when_a_source_changes(tmp_path, monkeypatch):
    """A record is reported while the listed sources hash to its digest, and not after an edit."""
    import hashlib
    name = "attn_fwd_headline_exact_256x128_hbm_counters.md"
    text = open(os.path.join(ROOT, "profiles", name)).read()
    rec = json.loads(re.search(r"```json\n(.*?)\n```", text, re.S).group(1))
    os.makedirs(tmp_path / "profiles")
    h = hashlib.sha256()
    for f in rec["sources"]:
        os.makedirs(tmp_path / os.path.dirname(f), exist_ok=True)
        shutil.copy(os.path.join(ROOT, f), tmp_path / f)
        h.update(open(tmp_path / f, "rb").read())
    rec["sources_sha256"] = h.hexdigest()   # a record taken from exactly these sources
    with open(tmp_path / "profiles" / name, "w") as fh:
        fh.write("```json\n" + json.dumps(rec) + "\n```\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.counted_traffic("exact", 256, 128) == rec["traffic_bytes"]
    with open(tmp_path / rec["sources"][0], "a") as fh:
        fh.write("\n// edited\n")
    assert bench.counted_traffic("exact", 256, 128) is None


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2 and "one GPU only" in r.stderr and r.stdout == ""
