"""Host-side logic of the benchmark and of the rocprofv3 summaries (CPU only):
the byte accounting, the one-GPU refusal, the stale-profile rule, and the
three summaries on small hand-made profiler outputs whose results are
computed here by hand."""
import csv
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import bench  # noqa: E402  (imports no torch at module level)
from speculative_verify_gemm_amd import profiling as P  # noqa: E402

LIN = "void k_linear<(anonymous namespace)::MfmaW4<1, 64, false, false>, {}>(LinArgs)"
COPY = "__amd_rocclr_copyBuffer"


def _csv(path, header, rows):
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(header)
        w.writerows(rows)


def _bench_out(path, **fields):
    with open(path, "w") as f:
        f.write("[bench] a progress line\n")
        f.write(json.dumps(fields) + "\n")


def test_linear_bytes_by_hand():
    # M=1, N=16, K=128, g=64: 1024 code bytes, 2 fp16 scales and 2 zeros per row
    # (64 + 64 bytes), 128 activation codes, one fp32 activation scale, 16 fp32 outputs
    assert bench.linear_bytes(1, 16, 128, "w4_z16", 64) == 1024 + 64 + 64 + 128 + 4 + 64
    # 4-bit zeros: the two zeros of a row share one byte
    assert bench.linear_bytes(1, 16, 128, "w4_z4", 64) == 1024 + 64 + 16 + 128 + 4 + 64
    # W8: one byte per code and one fp16 scale per row
    assert bench.linear_bytes(2, 16, 128, "w8", 0) == 2048 + 32 + 256 + 8 + 128
    assert bench.weight_bytes(16, 128, "w4_z16", 64) == 1024 + 64 + 64


def test_bench_refuses_several_gpus():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and not r.stdout


def test_profiled_traffic_only_for_the_current_kernels(tmp_path, monkeypatch):
    from speculative_verify_gemm_amd.build import source_digest
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.profiled_traffic("stack_x", 1) == (None, None)
    os.makedirs(tmp_path / "profiles")
    path = tmp_path / "profiles" / "linear_stack_x_m1_traffic.md"
    path.write_text("digest: 0123456789abcdef\ntraffic_bytes_per_launch: 1.5e+07\n")
    assert bench.profiled_traffic("stack_x", 1) == (None, "stale")
    path.write_text(f"digest: {source_digest()}\ntraffic_bytes_per_launch: 1.5e+07\n")
    assert bench.profiled_traffic("stack_x", 1) == (1.5e7, os.path.join("profiles", "linear_stack_x_m1_traffic.md"))


def test_trace_summary_pools_the_linear_shapes(tmp_path):
    hdr = ["Kernel_Name", "Start_Timestamp", "End_Timestamp", "Grid_Size_X", "Workgroup_Size_X"]
    rows = [[LIN.format("8, 4, 4"), 1000, 5000, 256 * 512, 512],      # 4 us, 256 workgroups
            [LIN.format("8, 4, 4"), 9000, 15000, 256 * 512, 512],     # 6 us
            [LIN.format("16, 6, 2"), 20000, 30000, 256 * 1024, 1024],  # 10 us
            ["fill_kernel(float*)", 0, 2000000, 64, 64]]               # 2 ms, not ours
    _csv(str(tmp_path / "t" / "trace_kernel_trace.csv"), hdr, rows)
    text = P.trace_summary(str(tmp_path / "t"), "cmd")
    assert "| `k_linear<MfmaW4<1, 64, false, false>, 8, 4, 4>` | 256 x 512 | 2 | 5.00 | 5.00 | 4.00 |" in text
    assert "| `k_linear<MfmaW4<1, 64, false, false>, 16, 6, 2>` | 256 x 1024 | 1 | 10.00 |" in text
    assert "`k_linear<MfmaW4<1, 64, false, false>>`: 3 dispatches, mean 6.667 us, median 6.000 us" in text
    assert "Other kernels (torch weight generation and fills at set-up): 1 dispatches, 2.0 ms in total." in text
    # with the traced run's bench output: its kernel digest and headline figures
    bj = tmp_path / "bench.json"
    bj.write_text("[bench] noise\n" + json.dumps({
        "kernel_digest": "00ff00ff00ff00ff", "ms_per_step": 1.8, "config": {"M": 16},
        "roofline": {"mean_launch_us": 9.5, "kernel": "k_linear<MfmaW4<1, 64, false, false>, ...>"}}) + "\n")
    text = P.trace_summary(str(tmp_path / "t"), "cmd", bench_json=str(bj))
    assert "digest: 00ff00ff00ff00ff" in text
    assert "1.8 ms per pass (M = 16), mean linear launch 9.5 us" in text


def test_traffic_summary_scales_by_the_copy(tmp_path):
    hdr = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"]
    calib_kib = 256 * 1024
    # FETCH_SIZE reads half of the copy (scale 2), WRITE_SIZE all of it (scale 1)
    fetch = [[i, COPY, "FETCH_SIZE", calib_kib / 2] for i in range(3)]
    fetch += [[5, COPY, "FETCH_SIZE", calib_kib * 2]]  # a 1 GiB copy of the same run: not the calibration
    fetch += [[10, LIN.format("8, 4, 4"), "FETCH_SIZE", 1000.0], [11, LIN.format("8, 4, 4"), "FETCH_SIZE", 3000.0]]
    write = [[i, COPY, "WRITE_SIZE", calib_kib] for i in range(3)]
    write += [[5, COPY, "WRITE_SIZE", calib_kib * 4]]
    write += [[10, LIN.format("8, 4, 4"), "WRITE_SIZE", 10.0], [11, LIN.format("8, 4, 4"), "WRITE_SIZE", 30.0]]
    _csv(str(tmp_path / "f" / "pmc_counter_collection.csv"), hdr, fetch)
    _csv(str(tmp_path / "w" / "pmc_counter_collection.csv"), hdr, write)
    for n in ("fj", "wj"):
        _bench_out(str(tmp_path / n), kernel_digest="abc")
    text = P.traffic_summary(str(tmp_path / "f"), str(tmp_path / "w"), 256, "stack_x", 16, "cmd",
                             str(tmp_path / "fj"), str(tmp_path / "wj"))
    assert "FETCH_SIZE scale 2.0000 (3 copies), WRITE_SIZE scale 1.0000 (3 copies)" in text
    assert f"fetch_bytes_per_launch: {2000 * 2 * 1024:.6g}" in text
    assert f"write_bytes_per_launch: {20 * 1024:.6g}" in text
    assert f"traffic_bytes_per_launch: {(4000 + 20) * 1024:.6g}" in text
    _bench_out(str(tmp_path / "wj"), kernel_digest="other")
    with pytest.raises(SystemExit):
        P.traffic_summary(str(tmp_path / "f"), str(tmp_path / "w"), 256, "stack_x", 16, "cmd",
                          str(tmp_path / "fj"), str(tmp_path / "wj"))


def test_mfma_summary_arithmetic(tmp_path):
    hdr = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"]
    rows = []
    for did, util, mops in ((1, 3.0, 4000.0), (2, 5.0, 6000.0)):
        rows += [[did, LIN.format("8, 4, 4"), "MfmaUtil", util],
                 [did, LIN.format("8, 4, 4"), "SQ_INSTS_VALU_MFMA_MOPS_I8", mops],
                 [did, LIN.format("8, 4, 4"), "SQ_INSTS_VALU_MFMA_I8", mops / 64]]
    rows += [[3, "void k_act_rht_quant<1024, 1, 32>(float const*)", "MfmaUtil", 0.0]]
    _csv(str(tmp_path / "c" / "pmc_counter_collection.csv"), hdr, rows)
    # 5000 MOPS x 512 = 2.56e6 executed ops per launch in 2 us: 1.28 TOP/s
    _bench_out(str(tmp_path / "plain.json"), kernel_digest="abc", config={"workload": "stack_x", "M": 16},
               roofline={"mean_launch_us": 2.0, "mean_algorithmic_int8_ops_per_launch": 1.28e6})
    text = P.mfma_summary([(str(tmp_path / "c"), str(tmp_path / "plain.json"))], "cmd")
    row = [ln for ln in text.splitlines() if ln.startswith("| stack_x |")]
    assert len(row) == 1
    cells = [c.strip() for c in row[0].strip("|").split("|")]
    assert cells[:4] == ["stack_x", "16", "`k_linear<MfmaW4<1, 64, false, false>>`", "2"]
    assert cells[4] == "4.00"                         # mean busy %
    assert cells[5] == "78"                           # 5000 / 64 MFMA instructions
    assert cells[6] == "0.003" and cells[7] == "0.001"
    assert cells[8] == "2.00"                         # executed / algorithmic
    assert cells[10] == "1.3" and cells[11] == "0.03"  # 1.28 TOP/s, 0.0256 % of 5000
    assert "digest: abc" in text


def test_calib_summary_per_instruction(tmp_path):
    (tmp_path / "plain.txt").write_text("waves per SIMD 4: 2.5 ms, 100 MFMA, 4289.8 TOP/s int8, 18.77 cycles\n")
    hdr = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"]
    k = "void k_mfma_peak<16>(int*, int)"
    rows = [[1, k, "SQ_INSTS_VALU_MFMA_I8", 10.0], [1, k, "SQ_VALU_MFMA_BUSY_CYCLES", 160.0],
            [1, k, "SQ_INSTS_VALU_MFMA_MOPS_I8", 640.0],                       # warm-up dispatch
            [2, k, "SQ_INSTS_VALU_MFMA_I8", 1000.0], [2, k, "SQ_VALU_MFMA_BUSY_CYCLES", 16000.0],
            [2, k, "SQ_INSTS_VALU_MFMA_MOPS_I8", 64000.0]]                     # timed: 64 x 512 ops each
    _csv(str(tmp_path / "c" / "pmc_counter_collection.csv"), hdr, rows)
    _csv(str(tmp_path / "u" / "pmc_counter_collection.csv"), hdr, [[1, k, "MfmaUtil", 5.0], [2, k, "MfmaUtil", 91.9]])
    text = P.calib_summary(str(tmp_path / "plain.txt"), str(tmp_path / "c"), str(tmp_path / "u"), "cmd")
    assert "- waves per SIMD 4: 2.5 ms" in text
    assert "| `k_mfma_peak<16>` | 1000 | 16.00 | 32768 | 91.9 |" in text


def test_hbm_summary_splits_the_trace_by_size(tmp_path):
    (tmp_path / "out.txt").write_text(
        "read o (4096 x 4096)   9437184 bytes:      3.38 us per launch,  2792.4 GB/s\n"
        "read 1 GiB          1073741824 bytes:    188.78 us per launch,  5687.9 GB/s\n")
    hdr = ["Kernel_Name", "Start_Timestamp", "End_Timestamp"]
    k = "k_read(unsigned int const*, unsigned long, unsigned int*)"
    durs = [9000, 9000, 9000, 3000, 4000, 5000] + [1000] * 3 + [200000] * 5   # 3 untimed + 3 timed, then 3 + 5
    rows, t = [], 0
    for d in durs:
        rows.append([k, t, t + d])
        t += d + 100
    rows.append(["other_kernel()", 0, 10])
    _csv(str(tmp_path / "tr" / "trace_kernel_trace.csv"), hdr, rows)
    text = P.hbm_summary(str(tmp_path / "out.txt"), str(tmp_path / "tr"), "cmd", reps=3)
    assert "| o (4096 x 4096) | 9437184 | 3.38 | 2792.4 | 4.00 | 2359.3 |" in text
    assert "| 1 GiB | 1073741824 | 188.78 | 5687.9 | 200.00 | 5368.7 |" in text


def test_read_kernel_times_match_the_stack_sizes(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    os.makedirs(tmp_path / "profiles")
    table = ("| size | bytes | us | GB/s | span | GB/s |\n|---|---|---|---|---|---|\n"
             "| o (4096 x 4096) | 9437184 | 3.38 | 2792.4 | 3.64 | 2592.6 |\n"
             "| qkv (12288 x 4096) | 28311552 | 6.20 | 4564.6 | 6.32 | 4479.7 |\n"
             "| gate/up (24576 x 4096) | 56623104 | 10.61 | 5337.6 | 10.76 | 5262.4 |\n")
    (tmp_path / "profiles" / "hbm_read_calibration.md").write_text(table)
    assert bench.read_kernel_times("stack_w4g64") == {"qkv": 6.2, "o": 3.38, "gateup": 10.61, "down": 6.2}
    assert bench.read_kernel_times("stack_w8") is None              # other byte counts
    (tmp_path / "profiles" / "hbm_read_calibration.md").write_text(table.replace("9437184", "9437185"))
    assert bench.read_kernel_times("stack_w4g64") is None           # a size that is not the launch's
