"""CPU tests of bench.py's host logic: the rocprofv3 summariser (kernel to
entry-point mapping, copy calibration of the byte counters, the recorded
traffic file) and the refusal of more than one GPU."""

import csv
import json
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


def test_summarize_profiles_calibrates_and_records(tmp_path, capsys):
    prof = tmp_path / "prof"
    os.makedirs(prof / "trace")
    with open(prof / "trace" / "bench_kernel_stats.csv", "w", newline="") as fh:
        w = csv.writer(fh)
        w.writerow(["Name", "Calls", "TotalDurationNs", "AverageNs", "Percentage", "MinNs", "MaxNs", "StdDev"])
        w.writerow(["void fa::fwd_kernel<false, 128, true, false, 4>(fa::FwdArgs)", 2, 400000, 200000, 40, 190000,
                    210000, 1])
        w.writerow(["void fa::bwd_dkdv_kernel<128, true, false>(fa::BwdArgs)", 2, 600000, 300000, 60, 290000, 310000,
                    1])
    copy = "__amd_rocclr_copyBuffer"
    # a 4 MiB copy: FETCH_SIZE reports half the bytes, WRITE_SIZE all of them
    _write_counters(str(prof / "fetch" / "bench_counter_collection.csv"), "FETCH_SIZE",
                    {copy: [2048, 2048], "void fa::fwd_kernel<false, 128, true, false, 4>(fa::FwdArgs)": [100, 300],
                     "void fa::bwd_dkdv_kernel<128, true, false>(fa::BwdArgs)": [1000]})
    _write_counters(str(prof / "write" / "bench_counter_collection.csv"), "WRITE_SIZE",
                    {copy: [4096], "void fa::fwd_kernel<false, 128, true, false, 4>(fa::FwdArgs)": [10, 10],
                     "void fa::bwd_dkdv_kernel<128, true, false>(fa::BwdArgs)": [50]})
    out = tmp_path / "traffic.json"
    bench.summarize_profiles(str(prof), 4, out_path=str(out))
    text = capsys.readouterr().out
    assert "scale x2.0000" in text and "scale x1.0000" in text
    rec = json.loads(out.read_text())
    assert rec["kernel_sources_sha256"] == bench.csrc_sha256()
    assert rec["fa_fwd"] == {"fetch_bytes": 200 * 1024 * 2, "write_bytes": 10 * 1024}
    assert rec["fa_bwd"] == {"fetch_bytes": 1000 * 1024 * 2, "write_bytes": 50 * 1024}


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
