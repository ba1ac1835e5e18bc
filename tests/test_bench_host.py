"""CPU tests of bench.py's host-side helpers (no GPU needed)."""

import json
import os

import bench
import workloads


def test_input_copies_keep_inputs_cold():
    # enough copies that more than 600 MB lie between two uses of one copy
    for name in ("tiny", "decode", "long", "prefill", "adversarial"):
        w = workloads.make(name)
        c = bench.input_copies(w)
        footprint = 4.0 * w.num_rows * w.row_stride
        assert 2 <= c <= bench.MAX_COPIES
        assert c == bench.MAX_COPIES or c * footprint >= bench.COLD_BYTES


def test_traffic_only_for_the_sources_it_was_measured_on(monkeypatch, tmp_path):
    entries = [{"workload": "prefill", "kernel_hash": "aaaa", "bytes_per_launch": 123.0},
               {"workload": "long", "kernel_hash": "aaaa", "bytes_per_launch": 45.0}]
    path = tmp_path / "traffic.json"
    path.write_text(json.dumps(entries))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(path))
    monkeypatch.setattr(bench, "kernel_source_hash", lambda: "aaaa")
    assert bench.measured_traffic("prefill") == 123.0
    assert bench.measured_traffic("long") == 45.0
    assert bench.measured_traffic("decode") is None
    monkeypatch.setattr(bench, "kernel_source_hash", lambda: "bbbb")  # sources changed since
    assert bench.measured_traffic("prefill") is None
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "missing.json"))
    assert bench.measured_traffic("prefill") is None


def test_committed_traffic_file_is_well_formed():
    entries = json.load(open(os.path.join(bench.ROOT, "profiles", "traffic.json")))
    for e in entries:
        assert e["bytes_per_launch"] == e["read_bytes_per_launch"] + e["write_bytes_per_launch"]
        assert abs(e["fetch_scale"] * e["copy_fetch_kib_per_gib"] - 1048576.0) < 1.0
        assert e["workload"] in bench.DESCRIPTIONS
