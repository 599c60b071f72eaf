"""Host-side contract of bench.py, without a GPU: it runs on exactly one GPU,
it reports the counter summaries only for the kernel sources those counters
were taken on, and its summaries of profiler output group the timed
dispatches by sweep point."""

import importlib.util
import json
import os
import shutil
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "block_sparse_flashattention_tiled_amd", "csrc")


def _bench():
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2", "--steps", "1"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 2
    assert "exactly one GPU" in r.stderr


def test_counters_only_for_the_profiled_kernel_sources(tmp_path, monkeypatch):
    b = _bench()
    rec = {"kernel_sha256": "a" * 64, "points": [{"point": "0", "hbm_read_bytes": 1.0, "hbm_write_bytes": 2.0}]}
    (tmp_path / b.COUNTERS_FILE).write_text(json.dumps(rec))
    monkeypatch.setattr(b, "PROFILES", str(tmp_path))
    monkeypatch.setattr(b, "kernel_source_hash", lambda: "a" * 64)
    assert b.measured_counters() == rec
    monkeypatch.setattr(b, "kernel_source_hash", lambda: "0" * 64)
    assert b.measured_counters() is None
    monkeypatch.setattr(b, "PROFILES", str(tmp_path / "missing"))
    assert b.measured_counters() is None


PROD = "void bsfa::bsfa_fwd_pair_kernel<128, 128, 128, true, false, false, true, false>(bsfa::FwdParams)"
CALIB = "void bsfa::bsfa_fwd_pair_kernel<128, 128, 128, true, true, true, true, false>(bsfa::FwdParams)"
DIAG = "void bsfa::bsfa_fwd_pair_kernel<128, 128, 128, true, true, false, true, false>(bsfa::FwdParams)"
PIPE = "void bsfa::bsfa_fwd_pipe_kernel<true, false, true, false>(bsfa::FwdParams)"
PIPE_DIAG = "void bsfa::bsfa_fwd_pipe_kernel<true, true, true, false>(bsfa::FwdParams)"


def test_production_instances_of_both_forward_kernels():
    b = _bench()
    assert b._forward_production(PROD) and b._forward_production(PIPE)
    assert not b._forward_production(CALIB) and not b._forward_production(DIAG)
    assert not b._forward_production(PIPE_DIAG)
    assert not b._forward_production("__amd_rocclr_copyBuffer")


def _write_csv(path, header, rows):
    import csv

    path.parent.mkdir(parents=True, exist_ok=True)
    with open(path, "w", newline="") as f:
        wr = csv.writer(f)
        wr.writerow(header)
        wr.writerows(rows)


def test_trace_summary_takes_the_timed_dispatches_by_point(tmp_path):
    b = _bench()
    rows, t, did = [], 1000, 0
    # the calibration pass, one warmup step, then two timed steps of four points
    durs = [[9.9, 7.0, 6.0, 5.0], [8.0, 5.0, 4.0, 3.0], [8.2, 5.2, 4.2, 3.2]]
    rows.append([did, CALIB, t, t + 4_000_000])
    t += 5_000_000
    for step in durs:
        for ms in step:
            did += 1
            rows.append([did, PROD, t, t + int(ms * 1e6)])
            t += int(ms * 1e6) + 1000
    _write_csv(tmp_path / "run" / "x_kernel_trace.csv", ["Dispatch_Id", "Kernel_Name", "Start_Timestamp",
                                                         "End_Timestamp"], rows)
    s = b.summarize_trace(str(tmp_path), 2, ["0", "0.6", "0.8", "0.9"])
    assert [p["dispatches"] for p in s["points"]] == [2, 2, 2, 2]
    assert abs(s["points"][0]["ms_mean"] - 8.1) < 1e-5 and abs(s["points"][3]["ms_mean"] - 3.1) < 1e-5
    assert abs(s["forward_ms_per_step"] - (8.1 + 5.1 + 4.1 + 3.1)) < 1e-5


def test_counter_summary_scales_by_the_copy_probe(tmp_path):
    b = _bench()
    header = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"]
    rows = [[1, "__amd_rocclr_copyBuffer", "FETCH_SIZE", 524288.0], [1, "__amd_rocclr_copyBuffer",
                                                                      "TCC_READ_SECTORS_sum", 2 ** 25]]
    did = 1
    for step in range(2):
        for p in range(4):
            did += 1
            rows.append([did, PROD, "FETCH_SIZE", 1000.0 * (p + 1) + step])
            rows.append([did, PROD, "TCC_READ_SECTORS_sum", 100.0 * (p + 1)])
            rows.append([did + 100, DIAG, "FETCH_SIZE", 1.0])  # diagnostics launches are not counted
    _write_csv(tmp_path / "f" / "run_counter_collection.csv", header, rows)
    header2 = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"]
    rows2 = []
    did = 1
    for step in range(2):
        for p in range(4):
            did += 1
            rows2 += [[did, PROD, "SQ_VALU_MFMA_BUSY_CYCLES", 400.0], [did, PROD, "SQ_BUSY_CU_CYCLES", 200.0]]
    _write_csv(tmp_path / "s" / "run_counter_collection.csv", header2, rows2)
    s = b.summarize_counters([str(tmp_path / "f"), str(tmp_path / "s")], 1, ["0", "0.6", "0.8", "0.9"])
    assert abs(s["scale"]["FETCH_SIZE"] - 2.0) < 1e-12 and abs(s["scale"]["TCC_READ_SECTORS_sum"] - 1.0) < 1e-12
    p0 = s["points"][0]
    assert p0["counters"]["FETCH_SIZE"] == 1001.0  # the last (timed) step only
    assert p0["hbm_read_bytes"] == 1001.0 * 1024 * 2.0
    assert p0["l2_read_bytes"] == 100.0 * 32
    assert p0["mfma_busy"] == 0.5
    rows_ = b.roofline_points([{"target": 0.0, "executed_tflops": 1000.0, "frac_of_peak": 0.4, "ms_mean": 2.0,
                                "stream_read_bytes": 1600.0}], s)
    assert rows_[0]["mfma_busy"] == 0.5 and rows_[0]["l2_read_over_stream"] == 2.0


def test_kernel_hash_follows_every_kernel_source(tmp_path, monkeypatch):
    b = _bench()
    csrc = tmp_path / "block_sparse_flashattention_tiled_amd" / "csrc"
    shutil.copytree(CSRC, csrc)
    monkeypatch.setattr(b, "ROOT", str(tmp_path))
    base = b.kernel_source_hash()
    assert base == _bench().kernel_source_hash()  # same sources, same hash
    for name in b.KERNEL_SOURCES:
        f = csrc / name
        original = f.read_bytes()
        f.write_bytes(original + b"\n")
        assert b.kernel_source_hash() != base, name
        f.write_bytes(original)
    assert b.kernel_source_hash() == base
