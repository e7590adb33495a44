"""Host logic of bench.py's counter summaries, on synthetic rocprofv3 CSVs: the MFMA busy
fraction, clock and FLOPs per launch, and the HBM bytes per launch scaled by the copy
calibration (the figures the committed profiles hold)."""

import csv
import importlib.util
import json
import os

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FIELDS = ["Correlation_Id", "Dispatch_Id", "Agent_Id", "Queue_Id", "Process_Id", "Thread_Id", "Grid_Size",
          "Kernel_Id", "Kernel_Name", "Workgroup_Size", "LDS_Block_Size", "Scratch_Size", "VGPR_Count",
          "Accum_VGPR_Count", "SGPR_Count", "Counter_Name", "Counter_Value", "Start_Timestamp", "End_Timestamp"]


def _bench():
    spec = importlib.util.spec_from_file_location("bench_mod", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def _write(path, rows):
    with open(path, "w", newline="") as fh:
        w = csv.DictWriter(fh, fieldnames=FIELDS)
        w.writeheader()
        for r in rows:
            w.writerow({k: r.get(k, 0) for k in FIELDS})


def test_summarize_mfma(tmp_path):
    b = _bench()
    pmc = tmp_path / "pmc"
    pmc.mkdir()
    with open(pmc / "wl__gemm_fwd_MFMA_agent_info.csv", "w", newline="") as fh:
        w = csv.DictWriter(fh, fieldnames=["Name", "Num_Xcc", "Simd_Count"])
        w.writeheader()
        w.writerow({"Name": "gfx950", "Num_Xcc": 8, "Simd_Count": 1024})
    rows = []
    # a warm-up dispatch of another kernel, then PROFILE_REPS GEMM dispatches of 100 us each:
    # one XCD active for 200,000 cycles (2.0 GHz), the 1024 SIMDs' MFMA pipes busy 0.5 of them
    rows.append(dict(Dispatch_Id=1, Kernel_Name="other", Counter_Name="GRBM_GUI_ACTIVE", Counter_Value=1,
                     Start_Timestamp=0, End_Timestamp=1))
    for d in range(2, 2 + b.PROFILE_REPS):
        base = dict(Dispatch_Id=d, Kernel_Name="void sge::gemm_kernel<0>(sge::GemmParams)",
                    Start_Timestamp=1000 * d * 1000, End_Timestamp=1000 * d * 1000 + 100_000)
        rows += [dict(base, Counter_Name="GRBM_GUI_ACTIVE", Counter_Value=8 * 200_000),
                 dict(base, Counter_Name="SQ_VALU_MFMA_BUSY_CYCLES", Counter_Value=0.5 * 200_000 * 1024),
                 dict(base, Counter_Name="SQ_INSTS_VALU_MFMA_MOPS_BF16", Counter_Value=2 ** 28),
                 dict(base, Counter_Name="SQ_INSTS_VALU_MFMA_MOPS_F8", Counter_Value=0)]
    _write(pmc / "wl__gemm_fwd_MFMA_counter_collection.csv", rows)
    out = tmp_path / "out"
    out.mkdir()
    b.summarize_mfma(str(pmc), str(out))
    r = json.load(open(out / "mfma_util.json"))["wl:gemm_fwd"]
    assert abs(r["mfma_busy"] - 0.5) < 1e-12
    assert abs(r["clock_ghz"] - 2.0) < 1e-12
    assert abs(r["mfma_tflop_per_dispatch"] - 2 ** 28 * 512 / 1e12) < 1e-12
    assert abs(r["frac_of_peak"] - 0.5 * 2.0 / 2.4) < 1e-12


def test_summarize_traffic(tmp_path):
    b = _bench()
    d = tmp_path / "pmc"
    d.mkdir()
    # calibration: the 1 GiB blit reads as 2^19 KiB fetched, the elementwise copy as 2^18 KiB (factor
    # 4, the one used) and both as 2^20 KiB written (factor 1)
    for c, blit_kib, elem_kib in (("FETCH_SIZE", 2 ** 19, 2 ** 18), ("WRITE_SIZE", 2 ** 20, 2 ** 20)):
        _write(d / f"copy_{c}_counter_collection.csv",
               [dict(Dispatch_Id=1, Kernel_Name="__amd_rocclr_copyBuffer", Counter_Name=c, Counter_Value=blit_kib),
                dict(Dispatch_Id=2, Kernel_Name="void at::native::vectorized_elementwise_kernel<4>", Counter_Name=c,
                     Counter_Value=elem_kib)])
    # a launch of two kernels repeated PROFILE_REPS times after a warm-up step
    for c, per_kernel in (("FETCH_SIZE", (100.0, 50.0)), ("WRITE_SIZE", (10.0, 20.0))):
        rows = [dict(Dispatch_Id=1, Kernel_Name="warm", Counter_Name=c, Counter_Value=999.0)]
        for i in range(b.PROFILE_REPS):
            for j, name in enumerate(("k_a", "k_b")):
                rows.append(dict(Dispatch_Id=2 + 2 * i + j, Kernel_Name=name, Counter_Name=c,
                                 Counter_Value=per_kernel[j]))
        _write(d / f"wl__quant_x_{c}_counter_collection.csv", rows)
    out = tmp_path / "out"
    out.mkdir()
    b.summarize_traffic(str(d), str(out))
    t = json.load(open(out / "traffic.json"))
    assert t["calibration"]["fetch_factor"] == 4.0 and t["calibration"]["write_factor"] == 1.0
    assert t["calibration"]["blit_fetch_factor"] == 2.0
    assert t["bytes_per_launch"]["wl:quant_x"] == int((150.0 * 4.0 + 30.0 * 1.0) * 1024)
