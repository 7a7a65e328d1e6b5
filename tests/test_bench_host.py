"""Host logic of bench.py that needs no GPU: the counter-to-traffic
conversion behind roofline.traffic and the algorithmic byte counts."""
import csv
import json
import os

import pytest

import bench

FIELDS = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"]


def _write(path, counter, rows):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=FIELDS)
        w.writeheader()
        for i, (name, kib) in enumerate(rows):
            w.writerow({"Dispatch_Id": i, "Kernel_Name": name, "Counter_Name": counter,
                        "Counter_Value": kib})


def test_write_traffic_scales_by_the_copy(tmp_path, monkeypatch):
    # three 1 MiB copies (3 MiB read and written): the fetch counter reads half,
    # the write counter reads all of it, so the scales are 2 and 1
    copy = [("__amd_rocclr_copyBuffer", 512.0)] * 3
    draft = "void dspark::(anonymous namespace)::k_bias_bf16<0, 2, true, false>(dspark::BiasPassArgs)"
    _write(tmp_path / "f.csv", "FETCH_SIZE", copy + [(draft, 1000.0), (draft, 1200.0)])
    _write(tmp_path / "w.csv", "WRITE_SIZE", [("__amd_rocclr_copyBuffer", 1024.0)] * 3 +
           [(draft, 10.0), (draft, 30.0)])
    out = tmp_path / "traffic.json"
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(out))
    bench.write_traffic(str(tmp_path / "f.csv"), str(tmp_path / "w.csv"), 1, ("f", "w"))
    t = json.load(open(out))
    assert t["fetch_scale"] == pytest.approx(2.0) and t["write_scale"] == pytest.approx(1.0)
    k = t["kernels"]["draft_bias"]
    assert k["read_bytes"] == int(1100.0 * 1024 * 2.0)
    assert k["write_bytes"] == int(20.0 * 1024)
    assert k["source"].endswith("csrc/bias_pass.hip") and len(k["sources_sha256"]) == 64
    assert "cstar_bias" not in t["kernels"]  # no counter rows, no entry
    # the bench reads it back while the source is unchanged
    assert bench.measured_traffic("draft_bias") == k["bytes_per_launch"]


def test_traffic_goes_stale_when_an_included_header_changes(tmp_path, monkeypatch):
    # a kernel source that includes a local header: the digest covers both
    src = tmp_path / "pkg" / "csrc"
    src.mkdir(parents=True)
    (src / "k.hip").write_text('#include "h.h"\n#include <hip/hip_runtime.h>\nint k;\n')
    (src / "h.h").write_text("int h = 1;\n")
    monkeypatch.setattr(bench, "HERE", str(tmp_path))
    d0 = bench.source_digest("pkg/csrc/k.hip")
    assert d0 == bench.source_digest("pkg/csrc/k.hip")
    out = tmp_path / "traffic.json"
    out.write_text(json.dumps({"kernels": {"draft_bias": {
        "source": "pkg/csrc/k.hip", "sources_sha256": d0, "bytes_per_launch": 123}}}))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(out))
    assert bench.measured_traffic("draft_bias") == 123
    (src / "h.h").write_text("int h = 2;\n")  # only the header changes
    assert bench.source_digest("pkg/csrc/k.hip") != d0
    assert bench.measured_traffic("draft_bias") is None


def test_write_traffic_calibrates_on_the_first_three_copies(tmp_path, monkeypatch):
    # later device copies (cold-cache flushes of another size) and a file whose
    # rows are not in dispatch order leave the scales at those of the first three
    draft = "void dspark::(anonymous namespace)::k_bias_bf16<0, 2, true, false>(dspark::BiasPassArgs)"
    rows = [("__amd_rocclr_copyBuffer", 512.0)] * 3 + [(draft, 1000.0), ("__amd_rocclr_copyBuffer", 9999.0)]
    for path, counter, rr in ((tmp_path / "f.csv", "FETCH_SIZE", rows),
                              (tmp_path / "w.csv", "WRITE_SIZE",
                               [(n, 2 * v) for n, v in rows])):
        with open(path, "w", newline="") as f:
            w = csv.DictWriter(f, fieldnames=FIELDS)
            w.writeheader()
            for i in reversed(range(len(rr))):  # written last dispatch first
                w.writerow({"Dispatch_Id": i, "Kernel_Name": rr[i][0], "Counter_Name": counter,
                            "Counter_Value": rr[i][1]})
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "traffic.json"))
    bench.write_traffic(str(tmp_path / "f.csv"), str(tmp_path / "w.csv"), 1, ("f", "w"))
    t = json.load(open(tmp_path / "traffic.json"))
    assert t["fetch_scale"] == pytest.approx(2.0) and t["write_scale"] == pytest.approx(1.0)


def test_algorithmic_bytes_of_the_high_concurrency_round():
    from draft_sampling_verification_w1_amd import synth
    cfg = synth.CONFIGS["high_concurrency"]
    R, g, V = cfg.R, cfg.gamma, cfg.V
    # one draft position: U_k, the rows' W1 operands, W2 once per draft call
    assert bench.algorithmic_bytes("draft_bias", cfg) == R * V * 2 + R * 256 * 2 + 256 * V * 2 / g
    # the c* pass: U and T of every position, W2, the W1 operands
    assert bench.algorithmic_bytes("cstar_bias", cfg) == 2 * R * g * V * 2 + 256 * V * 2 + R * g * 256 * 2
    assert bench.algorithmic_bytes("target_lse", cfg) == R * g * V * 2
