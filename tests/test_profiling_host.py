"""Host-side checks of the profile summaries (profiling.py, no GPU): kernel names map to the
functions bench.py books launches under, and the counter and trace summaries compute their
figures from synthetic rocprofv3 CSVs of known content."""
import csv
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

from blockwise_fp8_gemm_x128_amd import profiling  # noqa: E402


def test_function_names():
    f = profiling.function_of
    assert f("puro::(anonymous namespace)::gemm_fwd_256x256(unsigned char const*, ...)") == \
        "gemm_fwd_256x256"
    assert f("void puro::(anonymous namespace)::quant_dual_1x128_kernel<false, true>(...)") == \
        "quant_dual_1x128_kernel"
    assert f("void puro::(anonymous namespace)::quant_dual_1x128_kernel<false, false>(...)") == \
        "quant_dual_1x128_kernel(columns only)"
    assert f("void puro::(anonymous namespace)::quant_dual_1x128_kernel<true, true>(...)") == \
        "quant_dual_1x128_kernel[pow2]"
    assert f("void puro::(anonymous namespace)::sumsq_kernel<true>(float const*, ...)") == \
        "sumsq_kernel<true>"
    assert f("void at::native::vectorized_elementwise_kernel<4, ...>(...)") == ""


def _counter_csv(path, rows):
    cols = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value", "Start_Timestamp",
            "End_Timestamp"]
    with open(path, "w", newline="") as fh:
        w = csv.DictWriter(fh, fieldnames=cols)
        w.writeheader()
        for r in rows:
            w.writerow(r)


def test_sq_summary_ratios(tmp_path):
    k = "puro::(anonymous namespace)::gemm_fwd_256x256(x)"
    p1 = tmp_path / "p1.csv"
    p2 = tmp_path / "p2.csv"
    # two dispatches; ratios are of sums over both
    _counter_csv(p1, [
        {"Dispatch_Id": 1, "Kernel_Name": k, "Counter_Name": "SQ_INSTS_MFMA", "Counter_Value": 100},
        {"Dispatch_Id": 1, "Kernel_Name": k, "Counter_Name": "SQ_BUSY_CU_CYCLES", "Counter_Value": 50},
        {"Dispatch_Id": 1, "Kernel_Name": k, "Counter_Name": "SQ_VALU_MFMA_BUSY_CYCLES", "Counter_Value": 100},
        {"Dispatch_Id": 1, "Kernel_Name": k, "Counter_Name": "SQ_WAVE_CYCLES", "Counter_Value": 1000},
        {"Dispatch_Id": 1, "Kernel_Name": k, "Counter_Name": "SQ_WAIT_INST_ANY", "Counter_Value": 250},
        {"Dispatch_Id": 2, "Kernel_Name": k, "Counter_Name": "SQ_INSTS_MFMA", "Counter_Value": 300},
        {"Dispatch_Id": 2, "Kernel_Name": k, "Counter_Name": "SQ_BUSY_CU_CYCLES", "Counter_Value": 150},
        {"Dispatch_Id": 2, "Kernel_Name": k, "Counter_Name": "SQ_VALU_MFMA_BUSY_CYCLES", "Counter_Value": 300},
        {"Dispatch_Id": 2, "Kernel_Name": k, "Counter_Name": "SQ_WAVE_CYCLES", "Counter_Value": 1000},
        {"Dispatch_Id": 2, "Kernel_Name": k, "Counter_Name": "SQ_WAIT_INST_ANY", "Counter_Value": 250},
    ])
    _counter_csv(p2, [
        {"Dispatch_Id": 1, "Kernel_Name": k, "Counter_Name": "SQ_INSTS_VALU", "Counter_Value": 600},
        {"Dispatch_Id": 2, "Kernel_Name": k, "Counter_Name": "SQ_INSTS_VALU", "Counter_Value": 1800},
    ])
    text = profiling.sq_summary([str(p1), str(p2)], "t")
    line = [l for l in text.splitlines() if l.strip().startswith("gemm_fwd_256x256")][0].split()
    assert line[1] == "2"                      # dispatches per pass
    assert float(line[2]) == 6.0               # VALU/MFMA = 2400 / 400
    assert abs(float(line[6]) - 0.5) < 1e-9    # MFMA busy = 400 / (4 * 200)
    assert abs(float(line[8]) - 0.25) < 1e-9   # wait = 500 / 2000


def test_ceiling_summary_rates(tmp_path):
    trace = tmp_path / "trace.csv"
    cols = ["Dispatch_Id", "Kernel_Name", "Start_Timestamp", "End_Timestamp", "Grid_Size_X"]
    name = "void (anonymous namespace)::mfma_probe_kernel<0>(unsigned char const*, ...)"
    with open(trace, "w", newline="") as fh:
        w = csv.DictWriter(fh, fieldnames=cols)
        w.writeheader()
        # warm-up launch, then the timed one: 2048 waves (grid 131072 threads) for 10 ms
        w.writerow({"Dispatch_Id": 1, "Kernel_Name": name, "Start_Timestamp": 0,
                    "End_Timestamp": 1_000_000, "Grid_Size_X": 131072})
        w.writerow({"Dispatch_Id": 2, "Kernel_Name": name, "Start_Timestamp": 2_000_000,
                    "End_Timestamp": 12_000_000, "Grid_Size_X": 131072})
    log = tmp_path / "log.txt"
    log.write_text(json.dumps({"iters": 1000, "mfma_ceiling": {
        "zero | 2 waves/SIMD | MFMA chain": {"pflops": 1.0, "clock_ghz": 1.2,
                                             "ticks_mhz": 50.0}}}) + "\n")
    text = profiling.ceiling_summary(str(trace), str(log), "t")
    row = [l for l in text.splitlines() if l.strip().startswith("zero")][0].split()
    want_pf = 2048 * 1000 * 8 * 2.0 * 16 * 16 * 128 / 10e-3 / 1e15
    assert abs(float(row[-5]) - 10.0) < 1e-9             # rocprof ms
    assert abs(float(row[-4]) - round(want_pf, 2)) < 1e-9  # PF over the rocprof duration
    assert abs(float(row[-1]) - 2.4) < 1e-9              # clock = 1.2 GHz * 100 / 50 MHz
