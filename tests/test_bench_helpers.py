"""Host logic of bench.py that reads the committed profiler summaries.

The HBM traffic and the MFMA busy fraction are taken from rocprofv3 runs
committed as JSON; each records a hash of its kernel's sources, and a
summary whose kernel has changed since must be ignored (reported as null).
"""

import json
import os

import bench


def _write(tmp, name, body):
    with open(os.path.join(tmp, name), "w") as f:
        json.dump(body, f)


def _setup(tmp_path, monkeypatch):
    src = tmp_path / "k.hip"
    src.write_text("kernel source\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path))
    return bench.source_hash(["k.hip"])


def test_traffic_and_mfma_read_their_own_summaries(tmp_path, monkeypatch):
    h = _setup(tmp_path, monkeypatch)
    _write(tmp_path, "a_counters.json", {"workload": "w1", "kernel_hash": h,
                                         "kernel_sources": ["k.hip"],
                                         "hbm_bytes_per_launch": 123.0})
    _write(tmp_path, "a_mfma_util.json", {"workload": "w1", "kernel_hash": h,
                                          "kernel_sources": ["k.hip"], "mfma_util_pct": 37.5})
    _write(tmp_path, "b_mfma_util.json", {"workload": "w2", "kernel_hash": h,
                                          "kernel_sources": ["k.hip"], "mfma_util_pct": 20.0})
    assert bench.traffic_from_counters("w1") == 123.0
    assert bench.mfma_busy_from_counters("w1") == 0.375
    assert bench.mfma_busy_from_counters("w2") == 0.2
    # a workload with only an MFMA summary has no traffic figure
    assert bench.traffic_from_counters("w2") is None
    assert bench.traffic_from_counters("w3") is None
    assert bench.mfma_busy_from_counters("w3") is None


def test_stale_summaries_are_ignored(tmp_path, monkeypatch):
    h = _setup(tmp_path, monkeypatch)
    _write(tmp_path, "a_counters.json", {"workload": "w1", "kernel_hash": h,
                                         "kernel_sources": ["k.hip"],
                                         "hbm_bytes_per_launch": 123.0})
    _write(tmp_path, "a_mfma_util.json", {"workload": "w1", "kernel_hash": h,
                                          "kernel_sources": ["k.hip"], "mfma_util_pct": 37.5})
    (tmp_path / "k.hip").write_text("kernel source, changed\n")
    assert bench.traffic_from_counters("w1") is None
    assert bench.mfma_busy_from_counters("w1") is None


def test_comment_edits_keep_summaries_current(tmp_path, monkeypatch):
    """A summary stays current through comment and layout edits of its
    kernel's sources, and goes stale on a change of the code itself."""
    src = tmp_path / "k.hip"
    src.write_text("int f(int x) { return x + 1; }  // one\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path))
    h = bench.source_hash(["k.hip"])
    _write(tmp_path, "a_counters.json", {"workload": "w1", "kernel_hash": h,
                                         "kernel_sources": ["k.hip"],
                                         "hbm_bytes_per_launch": 7.0})
    src.write_text("/* a note */\nint f(int x) {\n    return x + 1;   // one, reworded\n}\n")
    assert bench.traffic_from_counters("w1") == 7.0
    src.write_text("int f(int x) { return x + 2; }  // one\n")
    assert bench.traffic_from_counters("w1") is None
    # comment markers inside string literals are code
    assert bench.code_text('s = "a // b"; // c') == 's = "a // b";'


def test_committed_summaries_match_the_kernel_sources():
    """Every counter summary under profiles/ was taken on the kernels as they
    are: its recorded hash matches the current sources, so bench.py reports
    its figures.  (A change to a kernel's code without new counter runs
    fails here.)"""
    import glob
    files = sorted(glob.glob(os.path.join(bench.PROFILES, "*_counters.json")) +
                   glob.glob(os.path.join(bench.PROFILES, "*_mfma_util.json")))
    assert files, "no committed counter summaries"
    stale = []
    for path in files:
        with open(path) as f:
            c = json.load(f)
        if c["kernel_hash"] != bench.source_hash(c["kernel_sources"]):
            stale.append(os.path.basename(path))
    assert not stale, f"summaries older than their kernels: {stale}"
    workloads = {json.load(open(p))["workload"] for p in files}
    for w in ("sweep_b256_s0.5", "sweep_b256_s0.5+tiled_w", "gemma_e2b"):
        assert w in workloads
        assert bench.traffic_from_counters(w) is not None
