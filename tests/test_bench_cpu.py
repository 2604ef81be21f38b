"""CPU tests of bench.py's host logic: the rocprofv3 summarisers (kernel to
entry-point mapping, copy calibration of the byte counters, read bytes by
request size, L2 hit rate, SQ counter ratios, the recorded profile file and
its staleness check), the amd-smi clock parser, the timing statistics, and
the refusal of more than one GPU."""

import csv
import json
import ctypes
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

FIELDS = ["Correlation_Id", "Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"]


def _write_counters(path, counter, per_kernel):
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w", newline="") as fh:
        w = csv.DictWriter(fh, fieldnames=FIELDS)
        w.writeheader()
        d = 0
        for name, values in per_kernel.items():
            for v in values:
                d += 1
                w.writerow({"Correlation_Id": d, "Dispatch_Id": d, "Kernel_Name": name, "Counter_Name": counter,
                            "Counter_Value": v})


def test_kernel_to_entry_point():
    assert bench._call_of("void fa::fwd_kernel<false, 128, true, false, 4>(fa::FwdArgs)") == "fa_fwd"
    assert bench._call_of("void fa::bwd_dkdv_kernel<128, true, false>(fa::BwdArgs)") == "fa_bwd"
    assert bench._call_of("void fa::bwd_dq_kernel<64, false>(fa::BwdArgs)") == "fa_bwd"
    assert bench._call_of("void fa::bwd_kernel<128, true, false, true>(fa::BwdArgs)") == "fa_bwd_atomic"
    assert bench._call_of("_ZN2fa21bwd_preprocess_kernelILi128ELb0ELb0EEEvPKDF16bPKvPfS5_x") == "fa_bwd"
    assert bench._call_of("_ZN2fa21bwd_preprocess_kernelILi128ELb0ELb1EEEvPKDF16bPKvPfS5_x") == "fa_bwd_atomic"
    assert bench._call_of("__amd_rocclr_copyBuffer") is None
    # the d=64 dK/dV pass, the FP8 P V forward and the transposed V quantizer
    assert bench._call_of("void fa::bwd_dkdv4_kernel<64, true, false, false>(fa::BwdArgs)") == "fa_bwd"
    assert bench._call_of("void fa::bwd_dkdv4_kernel<64, true, false, true>(fa::BwdArgs)") == "fa_bwd_varlen"
    assert bench._call_of("void fa::fwd_fp8_kernel<128, true, false, false>(fa::FwdArgs)") == "fa_fwd_fp8"
    assert bench._call_of("void fa::fwd_fp8_kernel<128, true, false, true>(fa::FwdArgs)") == "fa_fwd_fp8_pv"
    assert bench._call_of("void fa::fwd_fp8_kernel<128, true, false, false, false>(fa::FwdArgs)") == "fa_fwd_fp8"
    assert bench._call_of("void fa::fwd_fp8_kernel<128, true, false, true, false>(fa::FwdArgs)") == "fa_fwd_fp8_pv"
    assert bench._call_of("void fa::fwd_fp8_kernel<128, true, false, false, true>(fa::FwdArgs)") == \
        "fa_fwd_fp8_quantize_q"
    assert bench._call_of("void fa::fwd_fp8_kernel<64, false, true, true, true>(fa::FwdArgs)") == \
        "fa_fwd_fp8_quantize_q"
    assert bench._call_of("void fa::quantize_vt_fp8_kernel<128>(bool _Accum const*, unsigned char*, float*, int, "
                          "int)") == "fa_quantize_vt_fp8"
    assert bench._call_of("void fa::quantize_fp8_kernel<128>(bool _Accum const*, unsigned char*, float*, "
                          "signed char const*, int, int)") == "fa_quantize_fp8"
    assert bench._call_of("void fa::fwd_kernel<false, 128, true, false, 4, true>(fa::FwdArgs)") == "fa_fwd_varlen"
    assert bench._call_of("void fa::fwd_kernel<false, 128, true, false, 4, false>(fa::FwdArgs)") == "fa_fwd"
    assert bench._call_of("void fa::fwd_kernel<false, 128, true, false, 4, false, false>(fa::FwdArgs)") == "fa_fwd"
    assert bench._call_of("void fa::fwd_kernel<false, 64, true, true, 4, true, false>(fa::FwdArgs)") == "fa_fwd_varlen"
    assert bench._call_of("void fa::fwd_kernel<false, 128, true, false, 4, false, true>(fa::FwdArgs)") \
        == "fa_fwd_persistent"
    assert bench._call_of("void fa::bwd_dkdv_kernel<128, true, false, true>(fa::BwdArgs)") == "fa_bwd_varlen"
    assert bench._call_of("void fa::bwd_dq_kernel<128, true, true>(fa::BwdArgs)") == "fa_bwd_varlen"
    assert bench._call_of("void fa::bwd_dq_kernel<128, true, false, 4>(fa::BwdArgs)") == "fa_bwd"
    # the names rocprofv3 prints for the current instances (every template
    # argument written out)
    assert bench._call_of("void fa::bwd_dq_kernel<128, true, true, 4>(fa::BwdArgs)") == "fa_bwd_varlen"
    assert bench._call_of("void fa::bwd_dq_kernel<128, false, false, 8>(fa::BwdArgs)") == "fa_bwd"
    assert bench._call_of("void fa::bwd_dq_kernel<128, true, false, 8>(fa::BwdArgs)") == "fa_bwd"
    assert bench._call_of("void fa::bwd_dkdv_kernel<128, true, false, false>(fa::BwdArgs)") == "fa_bwd"
    assert bench._call_of("void fa::bwd_dkdv_kernel<64, false, true, true>(fa::BwdArgs)") == "fa_bwd_varlen"
    assert bench._call_of("void fa::fwd_kernel<false, 128, true, false, 8, false, false>(fa::FwdArgs)") == "fa_fwd"
    assert bench._call_of("void fa::quantize_fp8_kernel<128>(__bf16 const*, unsigned char*, float*, "
                          "signed char const*, int, int)") == "fa_quantize_fp8"
    assert bench._call_of("void fa::fwd_fp8_kernel<true, false>(fa::FwdArgs)") == "fa_fwd_fp8"


FWD = "void fa::fwd_kernel<false, 128, true, false, 8, false, false>(fa::FwdArgs)"
DKDV = "void fa::bwd_dkdv_kernel<128, true, false, false, false>(fa::BwdArgs)"
DQ = "void fa::bwd_dq_kernel<128, true, false, 8, false>(fa::BwdArgs)"
COPY = "__amd_rocclr_copyBuffer"


def test_summarize_profiles_calibrates_and_records(tmp_path, capsys):
    prof = tmp_path / "prof"
    os.makedirs(prof / "trace")
    with open(prof / "trace" / "bench_kernel_stats.csv", "w", newline="") as fh:
        w = csv.writer(fh)
        w.writerow(["Name", "Calls", "TotalDurationNs", "AverageNs", "Percentage", "MinNs", "MaxNs", "StdDev"])
        w.writerow([FWD, 2, 400000, 200000, 30, 190000, 210000, 1])
        w.writerow([DKDV, 2, 600000, 300000, 45, 290000, 310000, 1])
        w.writerow([DQ, 2, 300000, 150000, 25, 140000, 160000, 1])
    # a 4 MiB copy: FETCH_SIZE reports half the bytes, WRITE_SIZE all of them
    _write_counters(str(prof / "fetch" / "bench_counter_collection.csv"), "FETCH_SIZE",
                    {COPY: [2048, 2048], FWD: [100, 300], DKDV: [1000], DQ: [500]})
    _write_counters(str(prof / "write" / "bench_counter_collection.csv"), "WRITE_SIZE",
                    {COPY: [4096], FWD: [10, 10], DKDV: [50], DQ: [25]})
    # request counts by size: the dK/dV pass reads 10 x 128 B + 4 x 64 B + 2 x 32 B
    rd = {COPY: {"TCC_EA0_RDREQ_sum": 8, "TCC_EA0_RDREQ_32B_sum": 0, "TCC_EA0_RDREQ_64B_sum": 0,
                 "TCC_EA0_RDREQ_128B_sum": 8},
          DKDV: {"TCC_EA0_RDREQ_sum": 16, "TCC_EA0_RDREQ_32B_sum": 2, "TCC_EA0_RDREQ_64B_sum": 4,
                 "TCC_EA0_RDREQ_128B_sum": 10},
          DQ: {"TCC_EA0_RDREQ_sum": 1, "TCC_EA0_RDREQ_32B_sum": 0, "TCC_EA0_RDREQ_64B_sum": 1,
               "TCC_EA0_RDREQ_128B_sum": 0}}
    _write_multi(str(prof / "rdreq" / "bench_counter_collection.csv"), rd)
    tcc = {DKDV: {"TCC_HIT_sum": 30, "TCC_MISS_sum": 10, "TCC_EA0_RDREQ_DRAM_sum": 9},
           DQ: {"TCC_HIT_sum": 5, "TCC_MISS_sum": 5, "TCC_EA0_RDREQ_DRAM_sum": 4}}
    _write_multi(str(prof / "tcc" / "bench_counter_collection.csv"), tcc)
    out = tmp_path / "profile.json"
    bench.summarize_profiles(str(prof), 4, out_path=str(out))
    text = capsys.readouterr().out
    assert "scale x2.0000" in text and "scale x1.0000" in text
    assert "| 75.0% |" in text  # dK/dV L2 hit rate 30 / 40
    rec = json.loads(out.read_text())
    assert rec["kernel_sources_sha256"] == bench.csrc_sha256()
    assert rec["workload"] == bench.STEP_WORKLOAD
    assert rec["fa_fwd"]["kernel_avg_us"] == 200.0
    assert rec["fa_fwd"]["fetch_bytes"] == 200 * 1024 * 2 and rec["fa_fwd"]["write_bytes"] == 10 * 1024
    # fa_bwd = both of its kernels, summed per launch
    assert rec["fa_bwd"]["kernel_avg_us"] == 450.0
    assert rec["fa_bwd"]["fetch_bytes"] == 1500 * 1024 * 2
    assert rec["fa_bwd"]["write_bytes"] == 75 * 1024
    assert rec["fa_bwd"]["read_bytes_by_request_size"] == 10 * 128 + 4 * 64 + 2 * 32 + 64
    assert rec["fa_bwd"]["l2_hits"] == 35 and rec["fa_bwd"]["l2_misses"] == 15
    assert rec["fa_bwd"]["dram_read_requests"] == 13
    # the recorded profile is used only while the kernel sources are unchanged
    assert bench.profile_record("fa_bwd", str(out))["kernel_avg_us"] == 450.0
    stale = dict(rec, kernel_sources_sha256="0" * 64)
    out.write_text(json.dumps(stale))
    assert bench.profile_record("fa_bwd", str(out)) is None


def _write_multi(path, per_kernel):
    """One dispatch per kernel with several counters."""
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w", newline="") as fh:
        w = csv.DictWriter(fh, fieldnames=FIELDS)
        w.writeheader()
        for d, (name, counters) in enumerate(per_kernel.items(), 1):
            for c, v in counters.items():
                w.writerow({"Correlation_Id": d, "Dispatch_Id": d, "Kernel_Name": name, "Counter_Name": c,
                            "Counter_Value": v})


def test_summarize_pmc_reports_coexec_and_valu_busy(tmp_path, capsys):
    path = tmp_path / "sq" / "bench_counter_collection.csv"
    os.makedirs(path.parent)
    fields = FIELDS + ["Start_Timestamp", "End_Timestamp"]
    # 8 XCDs x 2000 cycles in 1000 ns: 2.0 GHz; MFMA busy on half of 1024 SIMDs x 2000 cycles
    vals = {"GRBM_GUI_ACTIVE": 16000, "SQ_WAVES": 100, "SQ_INSTS_VALU": 800, "SQ_INSTS_MFMA": 200,
            "SQ_INSTS_LDS": 300, "SQ_VALU_MFMA_BUSY_CYCLES": 1024000, "SQ_LDS_BANK_CONFLICT": 0,
            "SQ_VALU_MFMA_COEXEC_CYCLES": 256000, "SQ_ACTIVE_INST_VALU": 128000}
    with open(path, "w", newline="") as fh:
        w = csv.DictWriter(fh, fieldnames=fields)
        w.writeheader()
        for c, v in vals.items():
            w.writerow({"Correlation_Id": 1, "Dispatch_Id": 1, "Kernel_Name": DKDV, "Counter_Name": c,
                        "Counter_Value": v, "Start_Timestamp": 0, "End_Timestamp": 1000})
    bench.summarize_pmc(str(path.parent))
    row = [line for line in capsys.readouterr().out.splitlines() if DKDV in line][0]
    cells = [c.strip() for c in row.split("|")[1:-1]]
    # clock, MFMA busy, VALU busy (128000 / 256 CUs / 2000 cycles), co-exec share of MFMA busy
    assert cells[4:8] == ["2.00", "50.0", "25.0", "25.0"]
    assert cells[10] == "4.00"  # VALU per MFMA


def test_summarize_pmc_reports_lds_busy_and_waits(tmp_path, capsys):
    path = tmp_path / "sq2" / "bench_counter_collection.csv"
    os.makedirs(path.parent)
    fields = FIELDS + ["Start_Timestamp", "End_Timestamp"]
    # 2000 cycles per XCD; LDS busy on a quarter of 256 CUs x 2000 cycles; 100 waves of 400 quad-cycles
    vals = {"GRBM_GUI_ACTIVE": 16000, "SQ_WAVES": 100, "SQ_WAVE_CYCLES": 40000, "SQ_WAIT_ANY": 10000,
            "SQ_WAIT_INST_ANY": 12000, "SQ_WAIT_INST_LDS": 2000, "SQ_LDS_IDX_ACTIVE": 128000,
            "SQ_LDS_DATA_FIFO_FULL": 2560, "SQ_BUSY_CYCLES": 2000}
    with open(path, "w", newline="") as fh:
        w = csv.DictWriter(fh, fieldnames=fields)
        w.writeheader()
        for c, v in vals.items():
            w.writerow({"Correlation_Id": 1, "Dispatch_Id": 1, "Kernel_Name": DKDV, "Counter_Name": c,
                        "Counter_Value": v, "Start_Timestamp": 0, "End_Timestamp": 1000})
    bench.summarize_pmc(str(path.parent))
    out = capsys.readouterr().out
    assert "LDS busy %" in out
    row = [line for line in out.splitlines() if DKDV in line][0]
    cells = [c.strip() for c in row.split("|")[1:-1]]
    # clock, LDS busy, wave cycles per wave, waiting, waiting to issue, waiting to issue LDS, FIFO full per CU
    assert cells[4:11] == ["2.00", "25.0", "1600", "25.0", "30.0", "5.0", "10"]


# `amd-smi metric -g 0 --clock --json` output as printed on an idle MI355X
# (trimmed to two XCDs and one other clock domain).
AMD_SMI_CLOCK = """{
    "gpu_data": [
        {
            "gpu": 0,
            "clock": {
                "gfx_0": {"clk": {"value": 2399, "unit": "MHz"}, "min_clk": {"value": 500, "unit": "MHz"},
                          "max_clk": {"value": 2400, "unit": "MHz"}, "clk_locked": "DISABLED",
                          "deep_sleep": "ENABLED"},
                "gfx_1": {"clk": {"value": 1801, "unit": "MHz"}, "min_clk": {"value": 500, "unit": "MHz"},
                          "max_clk": {"value": 2400, "unit": "MHz"}, "clk_locked": "DISABLED",
                          "deep_sleep": "ENABLED"},
                "mem_0": {"clk": {"value": 2000, "unit": "MHz"}}
            }
        }
    ]
}"""


def test_clock_parsing_and_window():
    assert bench.read_amd_smi_clock(AMD_SMI_CLOCK) == [2399.0, 1801.0]
    assert bench.read_amd_smi_clock("WARNING: low-power state\n" + AMD_SMI_CLOCK) == [2399.0, 1801.0]
    assert bench.read_amd_smi_clock("") is None
    assert bench.read_amd_smi_clock("Unable to get devices, driver not initialized") is None
    assert bench.read_amd_smi_clock('{"gpu_data": [{"gpu": 0, "clock": {"gfx_0": {"clk": "N/A"}}}]}') is None
    samples = [(0.5, 2400.0, 2390.0, 2410.0), (1.5, 1900.0, 1800.0, 2000.0), (2.5, 1950.0, 1850.0, 1990.0),
               (3.5, 1000.0, 990.0, 1010.0)]
    w = bench.clock_window(samples, 1.0, 3.0)
    assert w == {"median": 1925.0, "min_xcd": 1800.0, "max_xcd": 2000.0, "samples": 2}
    assert bench.clock_window(samples, 10.0, 11.0) is None
    # dense bf16 peak at the published 2.4 GHz, and scaled to a measured clock
    assert abs(bench.peak_at_clock(2400.0) - 2516.58) < 0.01
    assert abs(bench.peak_at_clock(1900.0) / bench.peak_at_clock(2400.0) - 1900 / 2400) < 1e-12


def test_time_stats():
    ms = [1.0] * 9 + [2.0]
    s = bench.time_stats(ms, 2e9, 4e6, {"median": 1200.0})
    assert s["calls"] == 10 and s["ms_median"] == 1.0 and s["ms_min"] == 1.0 and s["ms_mean"] == 1.1
    assert s["ms_p90"] == 1.1
    assert s["tflops"] == 2.0 and s["gbps_algorithmic"] == 4.0
    assert s["clock_mhz"] == 1200.0
    assert abs(s["pct_of_bf16_peak_at_clock"] - round(100 * 2.0 / bench.peak_at_clock(1200.0), 2)) < 1e-9
    assert "clock_mhz" not in bench.time_stats(ms, 2e9, 4e6, None)


def test_host_description():
    h = bench.host_description()
    assert h["logical_cpus"] >= 1 and h["blas_threads"] >= 1
    assert isinstance(h["cpu_model"], str) and isinstance(h["blas"], str)


def test_cpu_slices_cover_every_workload():
    from exact_tiled_attention_28_amd.workloads import WORKLOADS
    assert set(bench.CPU_SLICES) == set(WORKLOADS)
    assert bench.STEP_WORKLOAD in WORKLOADS and WORKLOADS[bench.STEP_WORKLOAD].passes == "bwd"


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_machine_limit_probes_export_and_reject_bad_arguments():
    # the helper behind `bench.py --machine-limits`: it loads without a GPU,
    # exports its three launchers and refuses bad arguments before any launch
    from tests.hw import machine_limits
    if not os.path.exists(machine_limits.LIB):
        machine_limits.build()
    lib = machine_limits._lib()
    assert lib.ml_mfma(None, 256, 10, None, None) == -1
    assert lib.ml_exp(None, 256, 10, 1, 1, None, None) == -1
    assert lib.ml_lds(None, 256, 10, 0, None, None) == -1
    buf = ctypes.c_void_p(16)  # never dereferenced: every call below fails its argument check
    assert lib.ml_mfma(buf, 0, 10, buf, None) == -1
    assert lib.ml_exp(buf, 256, 10, 1, 5, buf, None) == -1
    assert lib.ml_lds(buf, 256, 10, 2, buf, None) == -1
