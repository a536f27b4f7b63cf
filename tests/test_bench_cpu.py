"""Host-side logic of bench.py, on the CPU: the one-GPU refusal, the roofline arithmetic, which committed
counter summary a line may quote, and the copy calibration of the counter summaries."""
import csv
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.abspath(os.path.join(os.path.dirname(__file__), ".."))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and not r.stdout.strip()


def test_pass_bytes_per_token_head():
    # raw q, k, g (128 each) and v, z (128 each) in bf16, the beta logit, bf16 y out
    assert bench.pass_bytes_per_token_head(128, 128) == 2 * (3 * 128 + 2 * 128) + 2 + 2 * 128 == 1538


def test_prompt_roofline_prices_the_dominant_kernel():
    per_kernel = {"chunk_intra": 0.0712, "chunk_scan": 0.0507, "gated_rmsnorm": 0.014}
    r = bench.prompt_roofline(per_kernel, 4096, 16, 128, 128, 1, "fp16")
    assert r["kernel"] == "chunk_intra" and r["bound"] == "hbm" and r["peak"] == bench.HBM_PEAK_GBS
    achieved = 1538 * 4096 * 16 / (0.0712e-3) / 1e9
    assert r["achieved"] == pytest.approx(achieved) and r["frac"] == pytest.approx(achieved / 8000.0)
    assert r["token_heads"] == 4096 * 16 and r["ms_per_launch"] == 0.0712


def test_committed_traffic_only_for_its_own_workload():
    """A summary is quoted for its workload's shape and precision at the current kernel sources only."""
    for name, path in bench.TRAFFIC_FILES.items():
        if not os.path.exists(path):
            continue
        t = json.load(open(path))
        shape = tuple(t["shape"])
        kernel = next(iter(t["kernels"]))
        want = t["kernels"][kernel]["hbm_bytes_per_launch"]
        current = t["source_sha256"] == bench.source_digest()
        assert bench.committed_traffic(kernel, t["precision"], name, shape) == (want if current else None)
        other = shape[:1] + (shape[1] + 1,) + shape[2:]
        assert bench.committed_traffic(kernel, t["precision"], name, other) is None
        assert bench.committed_traffic(kernel, "no-such-policy", name, shape) is None
    assert bench.committed_traffic("chunk_intra", "fp16", "no-such-workload") is None


def _counter_csv(path, counter, rows):
    with open(path, "w", newline="") as fh:
        wr = csv.DictWriter(fh, fieldnames=["Kernel_Name", "Grid_Size", "Counter_Name", "Counter_Value"])
        wr.writeheader()
        for name, grid, value in rows:
            wr.writerow({"Kernel_Name": name, "Grid_Size": grid, "Counter_Name": counter, "Counter_Value": value})


def test_pmc_summary_calibrates_on_the_large_copy(tmp_path, monkeypatch):
    """FETCH_SIZE is scaled by what it reads for the 1 GiB copy; a small copy with the same grid size (a
    workload's own tensor copy) must not enter the calibration."""
    copy, intra = "__amd_rocclr_copyBuffer", "void kda::chunk_intra_kernel<128, 128, 2, unsigned short, true>"
    gib_kib = (1 << 30) / 1024
    f, w = tmp_path / "f.csv", tmp_path / "w.csv"
    _counter_csv(f, "FETCH_SIZE", [(copy, 131072, gib_kib / 2)] * 3 + [(copy, 131072, 8000.0), (intra, 1024, 100.0)])
    _counter_csv(w, "WRITE_SIZE", [(copy, 131072, gib_kib)] * 3 + [(copy, 131072, 16000.0), (intra, 1024, 50.0)])
    monkeypatch.setattr(bench, "source_digest", lambda: "digest")
    out = bench.pmc_summary(str(f), str(w), "cmd", "fp16", "prefill", (1, 4096, 16, 128, 128))
    assert out["copy_calibration"]["fetch_scale"] == pytest.approx(2.0)
    assert out["copy_calibration"]["write_scale"] == pytest.approx(1.0)
    k = out["kernels"]["chunk_intra"]
    assert k["read_bytes"] == pytest.approx(100.0 * 2 * 1024) and k["write_bytes"] == pytest.approx(50.0 * 1024)
    assert out["workload"] == "prefill" and out["shape"] == [1, 4096, 16, 128, 128]
