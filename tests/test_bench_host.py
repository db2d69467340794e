"""Host logic of bench.py, on the CPU: the one-GPU guard, and the summary of
rocprofv3 kernel-trace and counter CSV files (--small-from) on synthetic files
whose answers are worked out here by hand."""
import csv
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402

NS = "w8a8::(anonymous namespace)::"
K32 = (f"void {NS}gemm_tiled<{NS}Cfg<128, 128, 2, 2, 128, 2, 1024, 2, false, 32, true, false>, "
       f"{NS}ElemI8, 0, 0, true, true>(void const*, float const*, long)")
K16 = (f"void {NS}gemm_tiled<{NS}Cfg<192, 256, 2, 4, 128, 2, 1024, 1, false, 16, true, false>, "
       f"{NS}ElemI8, 0, 0, true, true>(void const*, float const*, long)")


def _csv(path, rows):
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=list(rows[0]))
        w.writeheader()
        w.writerows(rows)


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300, cwd=ROOT)
    assert r.returncode == 2
    assert "exactly one GPU" in r.stderr


def test_small_from_rates_and_per_cu_shares(tmp_path, capsys):
    trace, pmc = str(tmp_path / "trace"), str(tmp_path / "pmc")
    rows, t = [], 0
    for name, dur_ns in ((K32, 10_000), (K16, 20_000)):
        # 12 launches: the first two slow (warm-up, outside the last 10)
        for i in range(12):
            d = dur_ns * (3 if i < 2 else 1)
            rows.append({"Kernel_Name": name, "Start_Timestamp": t, "End_Timestamp": t + d})
            t += d + 1000
    _csv(os.path.join(trace, "x_kernel_trace.csv"), rows)
    crow = []
    for name, n_mfma, busy in ((K32, 262144, 32 * 262144), (K16, 1000, 16 * 1000)):
        for disp in range(3):
            for cname, v in (("SQ_INSTS_MFMA", n_mfma), ("SQ_VALU_MFMA_BUSY_CYCLES", busy),
                             ("GRBM_GUI_ACTIVE", 8 * 1000), ("TA_TA_BUSY_sum", 256 * 500),
                             ("TD_TC_STALL_sum", 256 * 250)):
                crow.append({"Kernel_Name": name, "Dispatch_Id": f"{name[-40:]}{disp}",
                             "Counter_Name": cname, "Counter_Value": v})
    _csv(os.path.join(pmc, "y_counter_collection.csv"), crow)
    bench.small_from(trace, pmc)
    out = json.loads(capsys.readouterr().out)
    assert len(out) == 2
    r32 = next(v for k, v in out.items() if "128, 128" in k)
    r16 = next(v for k, v in out.items() if "192, 256" in k)
    assert r32["launches"] == 10 and r32["median_us"] == 10.0
    assert r16["median_us"] == 20.0
    # 32x32x32 int8: 65536 ops per MFMA; 16x16x64: 32768
    assert r32["issued_TOPS"] == round(262144 * 65536 / 10e-6 / 1e12, 1)
    assert r16["issued_TOPS"] == round(1000 * 32768 / 20e-6 / 1e12, 1)
    assert r32["mfma_busy_frac_at_2.4GHz"] == round(32 * 262144 / (1024 * 10e-6 * 2.4e9), 4)
    # per CU: sum over 256 CUs / (256 x GRBM_GUI_ACTIVE per XCC)
    for r in (r32, r16):
        assert r["TA_TA_BUSY_per_cu_frac"] == 0.5
        assert r["TD_TC_STALL_per_cu_frac"] == 0.25
