"""Host-only paths of bench.py: the one-GPU guard and the profile/latency
summaries it writes from profiler and calibration output (no GPU needed)."""
import csv
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], cwd=ROOT,
                          capture_output=True, text=True, timeout=300)


def test_bench_refuses_more_than_one_gpu():
    p = _bench("--gpus", "2")
    assert p.returncode != 0
    assert "one GPU" in (p.stdout + p.stderr)


def test_report_from_kernel_stats(tmp_path):
    stats = tmp_path / "stats"
    stats.mkdir()
    with open(stats / "x_kernel_stats.csv", "w", newline="") as fh:
        w = csv.DictWriter(fh, ["Name", "Calls", "TotalDurationNs", "AverageNs", "Percentage", "MinNs", "MaxNs"])
        w.writeheader()
        w.writerow({"Name": "msa_prefill_kernel<128>", "Calls": 20, "TotalDurationNs": 3.5e6, "AverageNs": 175000,
                    "Percentage": 97.5, "MinNs": 170000, "MaxNs": 181000})
        w.writerow({"Name": "msa_upload_kernel", "Calls": 20, "TotalDurationNs": 8e4, "AverageNs": 4000,
                    "Percentage": 2.5, "MinNs": 3500, "MaxNs": 4600})
    out = tmp_path / "report.md"
    p = _bench("--report", str(out), "--key", "prefill", "--kernel", "msa_prefill_kernel", "--units", "w",
               "--stats", str(stats), "--command", "rocprofv3 --kernel-trace --stats -- python bench.py",
               "--notes", "a note")
    assert p.returncode == 0, p.stderr
    text = out.read_text()
    assert "| `msa_prefill_kernel<128>` | 20 | 175.00 | 170.00 | 181.00 | 97.5% |" in text
    assert text.index("msa_prefill_kernel<128>") < text.index("msa_upload_kernel")   # sorted by total time
    assert "    rocprofv3 --kernel-trace --stats -- python bench.py" in text and "- a note" in text


def test_latency_report(tmp_path):
    res = {"model": "T = ...", "workload": "w", "k": [10.0, 0.5, 0.01, 1e-4, 2e-4], "rms_rel": 0.03, "n": 144,
           "dT_check_blocks_moved": 16,
           "checks": [{"l1": 128, "q1": 8, "l2": 128, "q2": 8, "T_us": 100.0, "T_moved_us": 110.0,
                       "measured_dT_us": 10.0, "eq5_dT_us": 9.5, "model_T_us": 101.0}],
           "chunk_rule": [{"l1": 256, "q1": 0, "l2": 0, "budget_us": 250.0, "chunk_blocks": 64, "T_us": 240.0}]}
    src = tmp_path / "lat.json"
    src.write_text(json.dumps(res))
    dst = tmp_path / "lat.md"
    p = _bench("--latency-report", str(src), "--report", str(dst))
    assert p.returncode == 0, p.stderr
    text = dst.read_text()
    assert "| 10.000 | 0.5000 | 0.01000 | 1.000e-04 | 2.000e-04 | 0.030 | 144 |" in text
    assert "| 128 | 8 | 128 | 8 | 100.0 | 101.0 | 10.0 | 9.5 |" in text
    assert "| 256 | 0 | 0 | 250 | 64 | 240.0 |" in text
