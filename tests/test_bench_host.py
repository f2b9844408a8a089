"""Host logic of bench.py (no GPU): the one-GPU refusal, the HBM-traffic
records that hold only while the kernel's sources are unchanged, and the
per-shape kernel-trace summary."""
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def _records():
    with open(os.path.join(ROOT, "profiles", "traffic.json")) as f:
        data = json.load(f)
    out = []
    for key, ent in data.items():
        workload, kernel, *proj = key.split("/")
        out.append((workload, kernel, proj[0].split(",") if proj else [None], ent))
    return out


def test_traffic_records_follow_the_kernel_source(monkeypatch):
    recs = _records()
    assert recs
    for workload, kernel, projections, ent in recs:
        current = ent["source_sha"] == bench.source_sha(kernel)
        for pr in projections:        # a record may cover several projections of one launch shape
            got = bench.stored_traffic(kernel, workload, pr)
            assert got == (ent["hbm_bytes_per_launch"] if current else None), (workload, kernel, pr)
    # any edit of the kernel's sources voids every record
    monkeypatch.setattr(bench, "source_sha", lambda kernel: "0" * 16)
    for workload, kernel, projections, _ in recs:
        for pr in projections:
            assert bench.stored_traffic(kernel, workload, pr) is None


def test_unknown_traffic_key_is_none():
    assert bench.stored_traffic("gemm_expand", "no_such_workload", "gate") is None


def test_trace_summary_groups_by_kernel_and_grid(tmp_path, capsys):
    rows = [("k_a", 1024, 1, 256, 0, 10000), ("k_a", 1024, 1, 256, 20000, 40000), ("k_a", 512, 4, 256, 0, 5000)]
    with open(tmp_path / "run_kernel_trace.csv", "w") as f:
        f.write("Kernel_Name,Grid_Size_X,Grid_Size_Y,Workgroup_Size_X,Start_Timestamp,End_Timestamp\n")
        for r in rows:
            f.write("%s,%d,%d,%d,%d,%d\n" % r)
    bench.trace_summary(str(tmp_path))
    body = [ln for ln in capsys.readouterr().out.splitlines() if ln.startswith("| ") and "calls" not in ln]
    # timestamps in ns, durations in us; largest total first; 2-D grids as x by y
    assert body == ["| 2 | 15.000 | 10.000 | 20.000 | 30.0 | 1024 | 256 | `k_a` |",
                    "| 1 | 5.000 | 5.000 | 5.000 | 5.0 | 512x4 | 256 | `k_a` |"]
