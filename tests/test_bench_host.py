"""Host logic of bench.py (CPU only): the code hash that ties the committed HBM-traffic counters to the
kernels they were taken on."""
import json
import os

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_code_hash_ignores_comments_and_blank_lines():
    a = "int f(int x) {  // doubles x\n\n  return 2 * x;   \n}\n/* trailing\n   note */\n"
    b = "int f(int x) {\n  return 2 * x;\n}\n"
    assert bench.code_sha([a]) == bench.code_sha([b])


def test_code_hash_sees_every_code_change():
    base = "int f(int x) {\n  return 2 * x;\n}\n"
    for changed in ("int f(int x) {\n  return 3 * x;\n}\n",      # a constant
                    "int f(int y) {\n  return 2 * y;\n}\n",      # a name
                    "int f(int x) {\n  return 2 * x; }\n"):      # a line joined
        assert bench.code_sha([changed]) != bench.code_sha([base])
    # the files' order and boundaries count too
    assert bench.code_sha(["int a;\n", "int b;\n"]) != bench.code_sha(["int b;\n", "int a;\n"])


def test_traffic_record_is_void_once_the_code_differs(tmp_path, monkeypatch):
    kind = "decode"
    rec = {kind: {"source_sha": bench.source_sha(kind), "hbm_bytes_per_launch": 123}}
    path = tmp_path / "traffic.json"
    path.write_text(json.dumps(rec))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(path))
    assert bench.measured_traffic(kind) == 123
    rec[kind]["source_sha"] = "0" * 16
    path.write_text(json.dumps(rec))
    assert bench.measured_traffic(kind) is None


def test_every_traffic_record_names_a_known_kernel_source_set():
    with open(os.path.join(ROOT, "profiles", "traffic_counters.json")) as f:
        data = json.load(f)
    for kind, rec in data.items():
        if kind == "calibration":
            continue
        assert kind in bench.KERNEL_SOURCES, kind
        assert len(rec["source_sha"]) == 16 and rec["hbm_bytes_per_launch"] > 0
