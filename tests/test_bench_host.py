"""Host logic of bench.py (no GPU): the algorithmic-byte count behind every
GB/s figure, the timing summaries, and the rule that keeps PMC traffic tied to
the kernel source and workload it was measured on."""
import json
import os

import pytest

import bench


def test_alg_bytes_tiny_bf16_by_hand():
    # lengths 37, 64, 1000, 4097 -> 1 + 1 + 16 + 65 = 83 tiles; 8 query / 1 KV head
    ab = bench.alg_bytes([37, 64, 1000, 4097], 8, 1, 128, "bf16")
    live = 37 + 64 + 1000 + 4097
    assert ab["kv"] == live * 1 * (2 * 128 * 2)            # K and V rows, bf16
    assert ab["q"] == 4 * 8 * 128 * 2
    assert ab["out"] == 4 * 8 * 128 * 2
    assert ab["meta"] == 4 * 83 + 4 * 4                     # page-table words + lengths
    assert ab["layer"] == 2678108                           # 2.68 MB
    assert ab["split"] == ab["layer"] - ab["out"]


def test_alg_bytes_fp8_counts_scales_and_query_tokens():
    ab = bench.alg_bytes([64, 65], 64, 8, 128, "fp8", q_len=2)
    assert ab["kv"] == (64 + 65) * 8 * (2 * 128 * 1 + 8)    # e4m3 K and V plus their fp32 scales
    assert ab["q"] == 2 * 2 * 64 * (128 + 4)                # e4m3 Q plus its scale, per query token
    assert ab["out"] == 2 * 2 * 64 * 128 * 2                # bf16 out, per query token
    assert ab["meta"] == 4 * (1 + 2) + 4 * 2


def test_alg_bytes_empty_request_moves_no_kv():
    ab = bench.alg_bytes([0, 64], 8, 1, 128, "bf16")
    assert ab["kv"] == 64 * 512
    assert ab["meta"] == 4 * 1 + 4 * 2


def test_summarize_statistics():
    s = bench.summarize([5.0, 1.0, 3.0, 2.0, 4.0, 6.0, 7.0, 8.0, 9.0, 10.0])
    assert s["min"] == 1.0 and s["median"] == 5.5 and s["mean"] == 5.5
    assert s["p90"] == 9.0                                  # 9th of 10 sorted values


def test_traffic_reported_only_for_its_source_workload_and_P(tmp_path, monkeypatch):
    ok = bench.source_sha(bench.SPLIT_SRC)
    f = tmp_path / "traffic.json"
    doc = {"kernel": "split_kernel", "workloads": {
        "long": {"source_sha256": ok, "workload": "long", "P": 512, "bytes_per_launch": 123},
        "tp8_share": {"source_sha256": "0" * 64, "workload": "tp8_share", "P": 256, "bytes_per_launch": 7}}}
    f.write_text(json.dumps(doc))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(f))
    assert bench.traffic_from_profile("long", 512) == 123
    assert bench.traffic_from_profile("long", 256) is None       # taken with another number of bins
    assert bench.traffic_from_profile("tp8_share", 256) is None  # taken on another kernel source
    assert bench.traffic_from_profile("skewed", 256) is None     # never taken
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "missing.json"))
    assert bench.traffic_from_profile("long", 512) is None


def test_write_traffic_keeps_one_entry_per_workload(tmp_path, monkeypatch):
    """Two PMC runs (FETCH_SIZE, WRITE_SIZE) become one entry; an entry of
    another workload already in the file is kept."""
    def run_dir(name, counter, calib_kib, split_kib):
        d = tmp_path / name
        d.mkdir()
        rows = ["Dispatch_Id,Kernel_Name,Counter_Name,Counter_Value",
                f'1,"__amd_rocclr_copyBuffer",{counter},{calib_kib}',
                f'2,"void lbsa::split_kernel<false, 1>(lbsa::AttnArgs)",{counter},{split_kib}',
                f'3,"void lbsa::split_kernel<false, 1>(lbsa::AttnArgs)",{counter},{split_kib}']
        (d / "x_counter_collection.csv").write_text("\n".join(rows) + "\n")
        return str(d)
    f = tmp_path / "traffic.json"
    f.write_text(json.dumps({"kernel": "split_kernel", "workloads": {"tp8_share": {"bytes_per_launch": 1}}}))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(f))
    calib = bench.CALIB_BYTES / 1024.0
    bench.write_traffic(run_dir("fetch", "FETCH_SIZE", 2 * calib, 1000.0),
                        run_dir("write", "WRITE_SIZE", calib, 10.0), "long", 512)
    doc = json.loads(f.read_text())
    assert set(doc["workloads"]) == {"tp8_share", "long"}
    e = doc["workloads"]["long"]
    assert e["fetch"]["factor"] == 0.5 and e["write"]["factor"] == 1.0
    assert e["bytes_per_launch"] == round(1000.0 * 1024 * 0.5 + 10.0 * 1024)
    assert e["P"] == 512
    assert bench.traffic_from_profile("long", 512) == e["bytes_per_launch"]


def test_more_than_one_gpu_is_refused():
    import subprocess
    import sys
    r = subprocess.run([sys.executable, os.path.join(bench.ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode != 0
    assert "one GPU" in r.stderr
