"""Host-side bookkeeping of bench.py: the refusal of several GPUs, the HBM-counter
ingestion (per-dispatch counters scaled by a plain copy of known size) and the rule that
the committed traffic figure is used only while the GEMM sources are unchanged."""
import csv
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    msg = json.loads(r.stdout.strip().splitlines()[-1])
    assert msg["n_gpus"] == 2 and "one GPU" in msg["error"]


def _counter_csv(path, counter, rows):
    """rows: (dispatch id, kernel name, KiB), written in the given order."""
    with open(path, "w", newline="") as f:
        wr = csv.DictWriter(f, fieldnames=["Dispatch_Id", "Kernel_Name", "Counter_Name",
                                           "Counter_Value"])
        wr.writeheader()
        for did, name, kib in rows:
            wr.writerow({"Dispatch_Id": did, "Kernel_Name": name, "Counter_Name": counter,
                         "Counter_Value": kib})


def test_ingest_scales_by_the_copy_and_keeps_dispatch_order(tmp_path):
    # dispatch order of --pmc-pass: the four kernels, a fill, then the 1 GiB copy.  The copy
    # is read as half its bytes by the fetch counter and exactly by the write counter, so
    # the fetched figures must come out doubled and the written ones unchanged.
    names = ["gemm_col", "gemm_row", "psum", "gemm_out", "fill", "__amd_rocclr_copyBuffer"]
    fetch_kib = [1000.0, 2000.0, 3000.0, 4000.0, 5.0, float(1 << 19)]
    write_kib = [10.0, 20.0, 30.0, 40.0, 5.0, float(1 << 20)]
    ids = range(1, len(names) + 1)
    f, w = tmp_path / "f.csv", tmp_path / "w.csv"
    # the fetch file lists its dispatches last to first: the ingestion orders them by id
    _counter_csv(f, "FETCH_SIZE", list(zip(ids, names, fetch_kib))[::-1])
    _counter_csv(w, "WRITE_SIZE", list(zip(ids, names, write_kib)))
    out = tmp_path / "traffic.json"
    assert bench.ingest_pmc(str(f), str(w), str(out)) == 0
    rec = json.load(open(out))
    assert rec["calibration"]["fetch_scale"] == pytest.approx(2.0)
    assert rec["calibration"]["write_scale"] == pytest.approx(1.0)
    for i, key in enumerate(bench.PMC_PASS_KERNELS):
        ent = rec["kernels"][f"{key}@llama3_70b_swiglu_bf16"]
        assert ent["kernel_symbol"] == names[i]
        assert ent["fetch_bytes"] == pytest.approx(fetch_kib[i] * 1024 * 2)
        assert ent["write_bytes"] == pytest.approx(write_kib[i] * 1024)
        assert ent["bytes_per_launch"] == pytest.approx(ent["fetch_bytes"] + ent["write_bytes"])
        assert ent["source_digest"] == bench.kernel_source_digest()


def test_traffic_is_used_only_for_the_sources_it_was_measured_on(tmp_path):
    path = tmp_path / "traffic.json"
    key = "column_gemm_swiglu@llama3_70b_swiglu_bf16"
    rec = {"kernels": {key: {"bytes_per_launch": 123.0,
                             "source_digest": bench.kernel_source_digest()}}}
    path.write_text(json.dumps(rec))
    assert bench.load_traffic("column_gemm_swiglu", "llama3_70b_swiglu_bf16", str(path)) == 123.0
    rec["kernels"][key]["source_digest"] = "0" * 16
    path.write_text(json.dumps(rec))
    assert bench.load_traffic("column_gemm_swiglu", "llama3_70b_swiglu_bf16", str(path)) is None
    assert bench.load_traffic("row_gemm", "llama3_70b_swiglu_bf16", str(path)) is None
    assert bench.load_traffic("column_gemm_swiglu", "x", str(tmp_path / "missing.json")) is None


def test_parity_failures_name_every_failed_check():
    """bench.py exits non-zero (after printing its line) when any comparison with the oracle,
    or the ring/whole-sequence and reduce-scatter/full-sum checks, misses its bar."""
    good = {"max_err": {"pass": True}, "configs": {"a": {"pass": True}, "b": {}},
            "context_parallel_ring": {"max_err_vs_whole": 1e-4},
            "sequence_parallel": {"rows_equal_full_sum": True}}
    assert bench.parity_failures(good) == []
    assert bench.parity_failures({"cpu_baseline": None}) == []
    bad = json.loads(json.dumps(good))
    bad["max_err"]["pass"] = False
    bad["configs"]["a"]["pass"] = False
    bad["context_parallel_ring"]["max_err_vs_whole"] = float("nan")
    bad["sequence_parallel"]["rows_equal_full_sum"] = False
    assert bench.parity_failures(bad) == ["max_err", "configs.a", "context_parallel_ring",
                                          "sequence_parallel"]


def test_percentiles_nearest_rank():
    st = bench.percentiles([float(v) for v in range(100, 0, -1)])
    assert (st["median"], st["p10"], st["p90"], st["calls"]) == (51.0, 11.0, 90.0, 100)


def test_column_gemm_traffic_bounds_of_the_70b_shard():
    # X 16384 x 8192, W1 and W3 blocks 8192 x 3584, H 16384 x 3584, all bf16
    compulsory, model = bench.column_gemm_traffic_bounds(16384, 8192, 3584)
    assert compulsory == 2 * (16384 * 8192 + 2 * 8192 * 3584 + 16384 * 3584) == 503_316_480
    # 64 x 28 = 1,792 tiles: 7 sweeps x 8 XCDs x 12 panels of 256 x 8192 bf16, plus H
    assert model == 7 * 8 * 12 * (256 * 8192 * 2) + 2 * 16384 * 3584 == 2_936_012_800
