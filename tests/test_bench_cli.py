"""bench.py's host-side contract, on the CPU: one GPU only, and the counter
summary that turns two rocprofv3 --pmc CSVs into calibrated bytes per
launch (the `traffic` figure of the roofline object)."""
import csv
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def run_bench(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args],
                          capture_output=True, text=True, cwd=ROOT, timeout=300)


def test_more_than_one_gpu_exits_with_a_message():
    r = run_bench("--gpus", "2")
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


FIELDS = ["Correlation_Id", "Dispatch_Id", "Agent_Id", "Queue_Id", "Process_Id", "Thread_Id",
          "Grid_Size", "Kernel_Id", "Kernel_Name", "Workgroup_Size", "LDS_Block_Size",
          "Scratch_Size", "VGPR_Count", "Accum_VGPR_Count", "SGPR_Count", "Counter_Name",
          "Counter_Value", "Start_Timestamp", "End_Timestamp"]


def write_csv(path, counter, rows):
    with open(path, "w", newline="") as fh:
        w = csv.DictWriter(fh, fieldnames=FIELDS)
        w.writeheader()
        for i, (name, value) in enumerate(rows):
            d = {k: 0 for k in FIELDS}
            d.update(Dispatch_Id=i, Kernel_Name=name, Counter_Name=counter, Counter_Value=value)
            w.writerow(d)


def test_pmc_summary_calibrates_and_averages(tmp_path):
    """Hand-made counter values: the calibration copy reads half its bytes on
    FETCH_SIZE and all of them on WRITE_SIZE, so fetch is scaled by 2 and
    write by 1; a kernel's KiB are averaged over its dispatches."""
    copy = "void at::native::vectorized_elementwise_kernel<4, at::native::MulFunctor<float>>(int)"
    gemm = "void qmoe::(anonymous namespace)::expert_gemm_kernel<true, false, 1, false, 4, false, 128>(qmoe::GroupedGemm, int)"
    kib = (1 << 30) / 1024  # the 1 GiB calibration copy
    f = tmp_path / "fetch.csv"
    w = tmp_path / "write.csv"
    write_csv(f, "FETCH_SIZE", [(copy, kib / 2), (copy, 10.0), (gemm, 100.0), (gemm, 300.0)])
    write_csv(w, "WRITE_SIZE", [(copy, kib), (gemm, 50.0), (gemm, 50.0)])
    r = run_bench("--pmc-summary", str(f), str(w))
    assert r.returncode == 0, r.stderr
    lines = r.stdout.splitlines()
    assert "scale fetch 2.0, write 1.0" in lines[0]
    row = [ln for ln in lines if ln.startswith("qmoe::expert_gemm_kernel<true")]
    assert len(row) == 1
    parts = row[0].split()
    # n, FETCH KiB (mean of 100, 300), WRITE KiB, (200 * 2 + 50 * 1) KiB in bytes
    assert parts[-4] == "2" and float(parts[-3]) == 200.0 and float(parts[-2]) == 50.0
    assert float(parts[-1]) == (200.0 * 2 + 50.0) * 1024
