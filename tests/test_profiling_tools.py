"""The rocprofv3 summary tools of profiling.py on small synthetic counter files (no GPU)."""
import csv
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PROF = [sys.executable, "-m", "token_sparse_attention_proxy_amd.profiling"]

ATT = ("void tsa::(anonymous namespace)::attn_fwd_bf16<128, false, false, true>(unsigned short "
       "const*, int)")
DENSE = ("void tsa::(anonymous namespace)::attn_fwd_bf16<128, false, false, false>(unsigned "
         "short const*, int)")
SCORE = "void tsa::(anonymous namespace)::score_merge(HIP_vector_type<float, 2u> const*, long)"
COPY = "__amd_rocclr_copyBuffer"
PROBE = "void tsa::(anonymous namespace)::mfma_probe<true>(float*, int)"


def _run(*args):
    r = subprocess.run(PROF + list(args), cwd=ROOT, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    return r.stdout


def _write(path, header, rows):
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(header)
        w.writerows(rows)


def test_trace_summary_keeps_headline_dispatches(tmp_path):
    hdr = ["Kind", "Kernel_Name", "Start_Timestamp", "End_Timestamp", "Grid_Size_X", "Grid_Size_Y"]
    gx = (131072 + 255) // 256 * 512
    rows = [["KERNEL_DISPATCH", ATT, 0, 100_000_000, gx, 32],
            ["KERNEL_DISPATCH", ATT, 200_000_000, 302_000_000, gx, 32],
            ["KERNEL_DISPATCH", DENSE, 310_000_000, 409_000_000, gx, 32],    # breakdown
            ["KERNEL_DISPATCH", PROBE, 410_000_000, 440_000_000, 256, 1],
            ["KERNEL_DISPATCH", DENSE, 450_000_000, 520_000_000, gx, 32],    # toggle-free operands
            ["KERNEL_DISPATCH", DENSE, 530_000_000, 600_000_000, gx, 32],
            ["KERNEL_DISPATCH", DENSE, 700_000_000, 810_000_000, gx, 32],    # dense baseline
            ["KERNEL_DISPATCH", SCORE, 820_000_000, 820_010_000, 64, 1],      # after: left out
            ["KERNEL_DISPATCH", "void at::native::fill(int)", 10, 20, 1, 1]]  # torch: left out
    _write(str(tmp_path / "trace" / "t_kernel_trace.csv"), hdr, rows)
    bench = {"value": 101.0, "budget": [123997],
             "roofline": {"avg_launch_ms": 101.0, "kernel": "attn_fwd_bf16<128, false, false, true>",
                          "achieved": 1247.1, "frac": 0.4988,
                          "mfma_ceiling": {"random_operands": 1700.0, "constant_operands": 2480.0,
                                           "attention_frac_of_random": 0.7336},
                          "operand_dependence": {"launches": 2}}}
    (tmp_path / "b.json").write_text("log line\n" + json.dumps(bench) + "\n")
    out = tmp_path / "t.md"
    _run("trace-summary", "--trace", str(tmp_path / "trace"), "--bench", str(tmp_path / "b.json"),
         "--command", "CMD", "--out", str(out))
    text = out.read_text()
    assert "| `attn_fwd_bf16<128, false, false, true>` | 2 | 101.0000 | 100.0000 | 102.0000 |" in text
    assert "| `attn_fwd_bf16<128, false, false, false> (breakdown, compressed tensors)` | 1 | 99.0000 |" in text
    assert "| `attn_fwd_bf16<128, false, false, false> (operands that barely toggle)` | 2 | 70.0000 |" in text
    assert "| `attn_fwd_bf16<128, false, false, false> (dense baseline)` | 1 | 110.0000 |" in text
    assert "score_merge" not in text and "fill" not in text
    assert "1700.0 TFLOP/s with random operands" in text


def test_sq_summary_busy_and_clock(tmp_path):
    hdr = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value", "Start_Timestamp",
           "End_Timestamp"]
    # one 100 ms launch: 1.6e8 cycles per XCD (1.6 GHz), MFMA busy half of 1024 SIMDs' cycles
    cyc = 1.6e8
    vals = {"SQ_WAVES": 1000, "SQ_BUSY_CYCLES": 1, "SQ_WAVE_CYCLES": 1, "SQ_INSTS_VALU": 4e9,
            "SQ_INSTS_MFMA": 1e9, "SQ_INSTS_LDS": 1e9, "SQ_VALU_MFMA_BUSY_CYCLES": 0.5 * cyc * 1024,
            "SQ_ACTIVE_INST_VALU": 1, "GRBM_GUI_ACTIVE": cyc * 8}
    rows = [[1, ATT, c, v, 0, 100_000_000] for c, v in vals.items()]
    _write(str(tmp_path / "sq" / "s_counter_collection.csv"), hdr, rows)
    out = tmp_path / "sq.md"
    _run("sq-summary", "--sq", str(tmp_path / "sq"), "--command", "CMD", "--out", str(out))
    text = out.read_text()
    assert "| 0.500 | 3.00 |" in text
    assert "clock of 1.60 GHz" in text


def test_summarize_all_scales_by_the_copy(tmp_path):
    hdr = ["Kernel_Name", "Counter_Name", "Counter_Value"]
    # the 1 GiB blit reads FETCH_SIZE = 0.5 GiB (in KiB), so fetch bytes scale by 2
    fetch = [[COPY, "FETCH_SIZE", (1 << 29) / 1024], [SCORE, "FETCH_SIZE", 1000.0]]
    write = [[COPY, "WRITE_SIZE", (1 << 30) / 1024], [SCORE, "WRITE_SIZE", 10.0]]
    _write(str(tmp_path / "f" / "c_counter_collection.csv"), hdr, fetch)
    _write(str(tmp_path / "w" / "c_counter_collection.csv"), hdr, write)
    out = tmp_path / "traffic.json"
    _run("summarize-all", "--fetch", str(tmp_path / "f"), "--write", str(tmp_path / "w"),
         "--out", str(out))
    e = json.loads(out.read_text())["score_merge"]["llama8b_bf16_L128k"]
    assert abs(e["fetch_bytes_per_launch"] - 2 * 1000 * 1024) < 1e-6
    assert abs(e["write_bytes_per_launch"] - 10 * 1024) < 1e-6
    assert e["source"] == "score.hip" and len(e["source_sha"]) == 16
