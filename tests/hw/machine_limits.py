"""Machine limits of one MI355X (gfx950) measured by the in-bounds
microbenchmarks of machine_limits.hip (a measurement helper next to the
tests, not part of the library): the bf16 matrix core's rate at one and two
wavefronts per SIMD, exp and FMA work beside it, the two LDS read patterns of
the kernels, and the shader clock under each load. `python3 bench.py
--machine-limits` prints the table."""

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "machine_limits.hip")
LIB = os.path.join(HERE, "libmachlimits.so")

N_CU = 256
PEAK_BF16_TFLOPS = 2516.58  # published dense bf16 peak (2.4 GHz)
MFMA_FLOPS = 2 * 32 * 32 * 16  # one v_mfma_f32_32x32x16_bf16
WAVES_PER_BLOCK = 4


def build() -> str:
    import subprocess
    from exact_tiled_attention_28_amd.build import hipcc
    cmd = [hipcc(), "--offload-arch=gfx950", "-O2", "-std=c++17", "-fPIC", "-shared",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", SRC, "-o", LIB]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("building the machine-limit probes failed:\n" + res.stdout + res.stderr)
    return LIB


def _lib():
    if not os.path.exists(LIB):
        raise RuntimeError(f"{LIB} is not built (run the repository's build entry point)")
    lib = ctypes.CDLL(LIB)
    p, i = ctypes.c_void_p, ctypes.c_int
    lib.ml_mfma.argtypes = [p, i, i, p, p]
    lib.ml_exp.argtypes = [p, i, i, i, i, p, p]
    lib.ml_lds.argtypes = [p, i, i, i, p, p]
    for f in (lib.ml_mfma, lib.ml_exp, lib.ml_lds):
        f.restype = i
    return lib


def _timed(launch, clk, reps=3):
    """Best of `reps` launches: (ms by events, shader clock in GHz from
    block 0's s_memtime / s_memrealtime over the same launch)."""
    import torch
    best = None
    for _ in range(reps + 1):  # the first launch warms up
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        if launch() != 0:
            raise RuntimeError("probe launch failed")
        e1.record()
        e1.synchronize()
        ms = e0.elapsed_time(e1)
        t = clk.cpu().tolist()
        ghz = (t[2] - t[0]) / (t[3] - t[1]) * 0.1 if t[3] > t[1] else float("nan")
        if best is None or ms < best[0]:
            best = (ms, ghz)
    return best


def run(iters_mfma=20000, iters_exp=20000, iters_lds=4096):
    import torch
    lib = _lib()
    torch.cuda.init()
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    out = torch.empty(2 * N_CU * 256, dtype=torch.float32, device="cuda")
    clk = torch.zeros(4, dtype=torch.int64, device="cuda")
    rows = []

    def clk_peak(ghz):
        return PEAK_BF16_TFLOPS * ghz / 2.4

    for wps in (1, 2):
        blocks = N_CU * wps
        ms, ghz = _timed(lambda: lib.ml_mfma(out.data_ptr(), blocks, iters_mfma, clk.data_ptr(), stream), clk)
        tf = blocks * WAVES_PER_BLOCK * iters_mfma * 4 * MFMA_FLOPS / (ms * 1e-3) / 1e12
        rows.append({"probe": f"MFMA 32x32x16 bf16, 4 independent chains, {wps} wave(s)/SIMD", "ms": ms,
                     "clock_ghz": ghz, "value": tf, "unit": "TFLOP/s", "pct_of_peak": 100 * tf / PEAK_BF16_TFLOPS,
                     "pct_at_clock": 100 * tf / clk_peak(ghz)})
    blocks = 2 * N_CU
    ms, ghz = _timed(lambda: lib.ml_exp(out.data_ptr(), blocks, iters_exp, 0, 4, clk.data_ptr(), stream), clk)
    lane_exps = blocks * WAVES_PER_BLOCK * 64 * iters_exp * 16
    rows.append({"probe": "v_exp_f32 alone (16 per iteration with their FMA and add, 12 FMAs), 2 waves/SIMD",
                 "ms": ms, "clock_ghz": ghz, "value": lane_exps / (ms * 1e-3) / (ghz * 1e9) / N_CU,
                 "unit": "exp lane-ops / clock / CU", "pct_of_peak": None, "pct_at_clock": None})
    for e in (0, 1, 2, 3, 4):
        ms, ghz = _timed(lambda: lib.ml_exp(out.data_ptr(), blocks, iters_exp, 1, e, clk.data_ptr(), stream), clk)
        tf = blocks * WAVES_PER_BLOCK * iters_exp * 4 * MFMA_FLOPS / (ms * 1e-3) / 1e12
        rows.append({"probe": f"MFMA + {e} exp(s) and {3 + 2 * e} other VALU per MFMA, 2 waves/SIMD", "ms": ms,
                     "clock_ghz": ghz, "value": tf, "unit": "TFLOP/s", "pct_of_peak": 100 * tf / PEAK_BF16_TFLOPS,
                     "pct_at_clock": 100 * tf / clk_peak(ghz)})
    outu = out.view(torch.int32)
    for mode, name in ((0, "ds_read_b128, 32-row blocks (K-operand pattern)"),
                       (1, "ds_read_b64_tr_b16, 4-row groups (transpose pattern)")):
        ms, ghz = _timed(lambda: lib.ml_lds(outu.data_ptr(), blocks, iters_lds, mode, clk.data_ptr(), stream), clk)
        nbytes = blocks * WAVES_PER_BLOCK * iters_lds * 16384
        rows.append({"probe": f"LDS {name}, 2 workgroups/CU", "ms": ms, "clock_ghz": ghz,
                     "value": nbytes / (ms * 1e-3) / (ghz * 1e9) / N_CU, "unit": "bytes / clock / CU",
                     "pct_of_peak": None, "pct_at_clock": None})
    return rows


def markdown(rows):
    lines = ["| probe | ms | shader clock GHz | value | unit | % of 2516.6 TFLOP/s | % of the peak at that clock |",
             "|---|---|---|---|---|---|---|"]
    for r in rows:
        pk = "" if r["pct_of_peak"] is None else f"{r['pct_of_peak']:.1f}"
        pc = "" if r["pct_at_clock"] is None else f"{r['pct_at_clock']:.1f}"
        lines.append(f"| {r['probe']} | {r['ms']:.3f} | {r['clock_ghz']:.2f} | {r['value']:.1f} | {r['unit']} | "
                     f"{pk} | {pc} |")
    return "\n".join(lines)
