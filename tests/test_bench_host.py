"""Host-side checks of bench.py (no GPU): the single-GPU guard, and the lookup of stored HBM
traffic records, which must only be used while the kernel sources they were measured on are
unchanged."""
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_source_digest_depends_on_the_function():
    g = bench.source_digest("gemm_fwd_256x256")
    q = bench.source_digest("quant_dual_1x128_kernel")
    assert len(g) == len(q) == 16 and g != q
    assert bench.source_digest("gemm_wgrad_192x256") == g


def _write_summary(path, recs):
    with open(path, "w") as fh:
        fh.write("header line\n")
        for r in recs:
            fh.write("traffic-record: " + json.dumps(r) + "\n")


def test_stored_traffic_uses_only_matching_records(tmp_path, monkeypatch):
    path = tmp_path / "traffic.txt"
    monkeypatch.setattr(bench, "TRAFFIC_SUMMARY", str(path))
    fwd = "gemm_fwd_256x256"
    good = {"function": fwd, "fetch_kib_per_launch": 100.0, "write_kib_per_launch": 50.0,
            "fetch_factor": 2.0, "write_factor": 1.0, "source_digest": bench.source_digest(fwd)}
    stale = dict(good, function="gemm_dgrad_256x256", source_digest="0" * 16)
    _write_summary(path, [good, stale])
    assert bench.stored_traffic(fwd) == 1024.0 * (100.0 * 2.0 + 50.0 * 1.0)
    assert bench.stored_traffic("gemm_dgrad_256x256") is None  # sources changed since measured
    assert bench.stored_traffic("quant_dual_1x128_kernel") is None  # no record
    monkeypatch.setattr(bench, "TRAFFIC_SUMMARY", str(tmp_path / "missing.txt"))
    assert bench.stored_traffic(fwd) is None


def test_committed_summary_parses():
    recs = []
    with open(os.path.join(ROOT, "profiles", "hbm_traffic_qwen3_1p7b_linear_stack_M8192.txt")) as fh:
        for line in fh:
            if line.startswith("traffic-record:"):
                recs.append(json.loads(line.split(":", 1)[1]))
    fns = {r["function"] for r in recs}
    assert {"gemm_fwd_256x256", "gemm_dgrad_256x256", "quant_dual_1x128_kernel",
            "quant_w_128x128_group_kernel"} <= fns
    for r in recs:
        assert r["fetch_kib_per_launch"] > 0 and r["write_kib_per_launch"] > 0
