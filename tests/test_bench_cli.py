"""bench.py's command-line contract on the CPU (no GPU is touched)."""

import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused_with_a_message():
    proc = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                          text=True, timeout=120)
    assert proc.returncode == 2
    assert "one GPU" in proc.stderr and proc.stdout == ""


def test_counter_csv_parsing_and_derived_fields(tmp_path):
    # rocprofv3 CSV rows -> per-kernel means; derived MFMA-busy share, clock and HBM rate
    sys.path.insert(0, ROOT)
    import bench
    cc = tmp_path / "run_counter_collection.csv"
    rows = ["Dispatch_Id,Kernel_Name,Counter_Name,Counter_Value"]
    for d in range(3):
        rows.append(f'{d},"h3attn::(anonymous namespace)::attn_fwd_kernel(int)",SQ_VALU_MFMA_BUSY_CYCLES,{4.0e10 + d}')
        rows.append(f'{d},"h3attn::(anonymous namespace)::attn_fwd_kernel(int)",GRBM_GUI_ACTIVE,4.8e8')
        rows.append(f'{d},"void h3attn::(anonymous namespace)::attn_fwd_fp8_kernel<false, {"true" if d else "false"}>(int)",'
                    'FETCH_SIZE,1000')
        # the Skip-Softmax instance is not the dense kernel the FP8 line reports
        rows.append(f'{d},"void h3attn::(anonymous namespace)::attn_fwd_fp8_kernel<true, false>(int)",FETCH_SIZE,9')
        rows.append(f'{d},"h3attn::(anonymous namespace)::kv_prologue_kernel(int)",FETCH_SIZE,7')
    cc.write_text("\n".join(rows) + "\n")
    c = bench.parse_counter_csv(str(cc))
    assert set(c) == {"bf16", "fp8"}
    assert c["bf16"]["GRBM_GUI_ACTIVE"] == 4.8e8 and c["fp8"]["FETCH_SIZE"] == 1000
    kt = tmp_path / "run_kernel_trace.csv"
    kt.write_text('Kernel_Name,Start_Timestamp,End_Timestamp\n"attn_fwd_kernel(int)",1000,30001000\n')
    durations = bench.parse_kernel_trace_csv(str(kt))
    assert abs(durations["bf16"] - 0.03) < 1e-12
    c["bf16"].update({"FETCH_SIZE": 5e6, "WRITE_SIZE": 1.6e5})
    f = bench.counter_fields(c, durations, "bf16", 30.0, 256)
    assert abs(f["mfma_busy"] - (4.0e10 + 1) / (4.8e8 / 8 * 1024)) < 1e-4
    assert abs(f["clock_ghz"] - 2.0) < 1e-3
    assert f["traffic"] == int(round((5e6 * 2.0 + 1.6e5) * 1024))
    assert abs(f["hbm_gbps"] - f["traffic"] / 0.03 / 1e9) < 0.1
    # nothing measured -> every field null
    assert bench.counter_fields({}, {}, "fp8", 18.0, 256) == {"mfma_busy": None, "clock_ghz": None,
                                                            "traffic": None, "hbm_gbps": None}
