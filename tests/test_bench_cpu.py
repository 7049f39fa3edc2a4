"""CPU checks of bench.py's host logic: the one-GPU guard, the source digest
that keys the committed counter summary, and the bounded CPU-oracle baseline."""
import os
import subprocess
import sys
import types

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from combine_dispatch_layout_amd import workloads as W  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_source_digest_ignores_comments_and_whitespace(tmp_path, monkeypatch):
    src = tmp_path / "k.hip"
    monkeypatch.setattr(bench, "KERNEL_SOURCE", str(src))
    src.write_text("int a = 1; // one\n/* block\n comment */ int b;\n")
    d0 = bench.source_digest()
    src.write_text("int   a = 1;   // other words\n\n int b; /* x */\n")
    assert bench.source_digest() == d0
    src.write_text("int a = 2; // one\n/* block\n comment */ int b;\n")
    assert bench.source_digest() != d0


def test_committed_traffic_only_for_the_current_source(tmp_path, monkeypatch):
    src = tmp_path / "k.hip"
    src.write_text("__global__ void k() {}\n")
    summary = tmp_path / "t.txt"
    monkeypatch.setattr(bench, "KERNEL_SOURCE", str(src))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(summary))
    summary.write_text("# comment: ignored\nkernel: k\nhbm_bytes_per_launch: 12345\n"
                       "source_sha256: %s\n" % bench.source_digest())
    assert bench.committed_traffic() == 12345.0
    summary.write_text("hbm_bytes_per_launch: 12345\nsource_sha256: 0000000000000000\n")
    assert bench.committed_traffic() is None
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "missing.txt"))
    assert bench.committed_traffic() is None


def test_cpu_baseline_is_bounded_and_reports_the_sample():
    w = W.WORKLOADS["tiny"]
    x, ids, wts = W.make_inputs(w)
    s = types.SimpleNamespace(x_host=x, ids_host=ids, w_host=wts, T=w.T, k=w.k, L=w.L,
                              bytes_step=lambda: 1e6)
    r = bench.cpu_baseline(W, s, budget_s=0.05, max_reps=3)
    assert r["kind"] == "oracle" and r["cores"] == 1 and r["unit"] == "GB/s"
    assert r["value"] > 0 and r["tokens_per_s"] > 0
    n = int(r["sample"].split()[0])
    assert 1 <= n <= 3
    assert len(r["ms_layout_dispatch_combine"]) == 3
