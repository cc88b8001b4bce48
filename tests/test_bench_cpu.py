"""Host-side logic of bench.py (no GPU): the one-GPU guard, the kernel-trace
summary writer and the source-hash check that decides whether a committed
traffic figure still describes the current kernels."""
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
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


@pytest.mark.parametrize("workload", sorted(bench.TRACE_RUN))
def test_trace_summary_records_its_command(tmp_path, monkeypatch, workload):
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    (tmp_path / "profiles").mkdir()
    d = tmp_path / "prof"
    d.mkdir()
    stats = d / "x_kernel_stats.csv"
    with open(stats, "w", newline="") as fh:
        w = csv.writer(fh)
        w.writerow(["Name", "Calls", "TotalDurationNs", "AverageNs", "Percentage", "MinNs", "MaxNs", "StdDev"])
        w.writerow(["void trimkv::(anonymous namespace)::k_attn_bf16<128, 0>(trimkv::AttnArgs)", 3, 3000, 1000.0,
                    60.0, 900, 1100, 10.0])
        w.writerow(["trimkv::k_score<4>(int const*)", 2, 2000, 1000.0, 40.0, 950, 1050, 5.0])
    bench.trace_summary(workload, str(stats))
    text = (tmp_path / "profiles" / ("kernel_stats_%s.md" % workload)).read_text()
    args, _ = bench.TRACE_RUN[workload]
    assert ("-d %s -o x -- python -u bench.py %s" % (d, args)) in text
    assert "| k_attn_bf16<128, 0> | 3 | 1.0 | 0.9 | 1.1 | 60.0 |" in text
    assert "| k_score<4> | 2 | 1.0 |" in text


def test_traffic_only_for_unchanged_sources(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    (tmp_path / "profiles").mkdir()
    hashes = {s: bench.source_hash(f) for s, (_, f) in bench.STAGE_KERNEL.items()}
    kname = bench.STAGE_KERNEL["decode"][0]
    blob = {"read_factor": 2.0, "write_factor": 1.0, "source_hash": hashes,
            "kernels": {kname: {"fetch_kib": 10.0, "write_kib": 1.0, "traffic_bytes": 12345}}}
    page = "# x\n\n```json\n%s\n```\n" % json.dumps(blob)
    (tmp_path / "profiles" / "pmc_llama8b_32k.md").write_text(page)
    assert bench.traffic_for("llama8b_32k", "decode") == 12345
    blob["source_hash"] = dict(hashes, decode="0" * 16)
    (tmp_path / "profiles" / "pmc_llama8b_32k.md").write_text("# x\n\n```json\n%s\n```\n" % json.dumps(blob))
    assert bench.traffic_for("llama8b_32k", "decode") is None
    assert bench.traffic_for("batched16_16k", "decode") is None
