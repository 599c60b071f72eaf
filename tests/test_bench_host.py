"""Host-side contract of bench.py, without a GPU: it runs on exactly one GPU,
and it reports the counter-measured HBM traffic only for the kernel sources
those counters were taken on."""

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


def test_traffic_only_for_the_profiled_kernel_sources(monkeypatch):
    b = _bench()
    rec = json.load(open(os.path.join(ROOT, "profiles", "bsfa_fwd_llama32k_traffic.json")))
    monkeypatch.setattr(b, "kernel_source_hash", lambda: rec["kernel_sha256"])
    assert b.measured_traffic("llama32k") == rec["hbm_bytes_per_launch"]
    monkeypatch.setattr(b, "kernel_source_hash", lambda: "0" * 64)
    assert b.measured_traffic("llama32k") is None
    assert b.measured_traffic("no-such-workload") is None


def test_kernel_hash_follows_every_kernel_source(tmp_path, monkeypatch):
    b = _bench()
    csrc = tmp_path / "block_sparse_flashattention_tiled_amd" / "csrc"
    shutil.copytree(CSRC, csrc)
    monkeypatch.setattr(b, "ROOT", str(tmp_path))
    base = b.kernel_source_hash()
    assert base == _bench().kernel_source_hash()  # same sources, same hash
    for name in ("bsfa_fwd_kernels.h", "bsfa_internal.h", "bsfa_fwd_128x128.hip"):
        f = csrc / name
        original = f.read_bytes()
        f.write_bytes(original + b"\n")
        assert b.kernel_source_hash() != base, name
        f.write_bytes(original)
    assert b.kernel_source_hash() == base
