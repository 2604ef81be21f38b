#!/usr/bin/env python3
"""Benchmark of the attention hot path on one MI355X.

One step = one pass of the whole hot path over one batch of synthetic input:
fa_fwd (bf16 O, fp32 L) followed by fa_bwd (dQ pass forming D, then the dK/dV
pass; fp32 dQ, bf16 dK/dV, bf16 P and dS) on the causal bf16 backward
workload B=4, H=16, N=4096, d=128 (seed 5), whose O and L come from that
forward. Inputs are resident in HBM before the timed region; L2 and MALL are
not flushed between calls. Prints ONE JSON line.

value = causal-adjusted TFLOPS of the step: forward 4*B*H*N^2*d/2 plus
backward 2.5x that, divided by the wall-clock time of the timed steps
(synchronised on both sides). Forward and backward times come from HIP
events recorded between the calls on the launch stream.

Also in the line:
* `configs`: every named workload (forward configs, the backward config)
  timed on its own with at least --config-calls calls: median / min / p90,
  TFLOPS and % of the dense bf16 MFMA peak, both the published one and the
  one at the shader clock measured while that workload ran;
* `gpu_clock_mhz`: the shader clock read from `amd-smi metric --clock` by a
  child process started before the GPU is touched, over a window of
  back-to-back steps (the timed region itself is too short for the tool's
  refresh period);
* `roofline`: the call that takes the most time per step (fa_bwd), timed
  with HIP events on the stream the library launches on, with the HBM bytes
  per launch recorded from rocprofv3 counters for the same kernel sources;
* `cpu_baseline`: the fp64 CPU oracle on a bounded sample of the step's
  workload (plus a sample of every other workload under `per_config`), with
  the CPU model and the BLAS library and thread count.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu] [--no-configs] [--no-clock]
       python bench.py --workload NAME | --varlen | --sweep | --persistent | --fp8   (extra measurements)
"""

from __future__ import annotations

import argparse
import json
import os
import subprocess
import sys
import threading
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
# Per-launch kernel durations and HBM bytes of the step's calls, written by
# --summarize-profiles from rocprofv3 runs of this benchmark.
PROFILE_JSON = os.path.join(ROOT, "profiles", "fa_step_b4_h16_n4096_d128_profile.json")
sys.path.insert(0, ROOT)

from exact_tiled_attention_28_amd import binding  # noqa: E402
from exact_tiled_attention_28_amd.inputs import make_inputs  # noqa: E402
from exact_tiled_attention_28_amd.workloads import (  # noqa: E402
    MI355X_BF16_PEAK_TFLOPS, MI355X_HBM_GBPS, WORKLOAD_ORDER, WORKLOADS, bwd_bytes, bwd_flops, fwd_bytes, fwd_flops,
    workload_bytes, workload_flops)

METRIC = "attention fwd/bwd TFLOPS (causal-adjusted) and % of MI355X bf16 MFMA peak"
STEP_WORKLOAD = "bwd_bf16_causal_b4_h16_n4096_d128"
# Dense bf16 MFMA flops per clock of the whole chip: 256 CUs x 4096.
BF16_FLOPS_PER_CLK = 256 * 4096
# (batch, head) slices of each workload timed on the CPU oracle: about 20 s
# of fp64 work in all on 16 host threads.
CPU_SLICES = {
    "fwd_f32_b1_h1_n128_d64": 1,
    "fwd_bf16_causal_b8_h16_n2048_d128": 16,
    "fwd_bf16_causal_b1_h8_n16384_d128": 2,
    "fwd_bf16_causal_gqa_b4_hq32_hkv8_n4096_d128_outliers": 4,
    "bwd_bf16_causal_b4_h16_n4096_d128": 32,
}
CACHE_NOTE = ("inputs resident in HBM before timing; L2 and MALL are not flushed between timed calls (the step "
              "reads 256 MiB of Q, K, V, dO, as large as the 256 MiB MALL before its outputs are counted)")


def parse(argv=None):
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=100)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    p.add_argument("--no-configs", action="store_true",
                   help="skip timing the named workloads one by one after the step (profiled runs use this)")
    p.add_argument("--no-clock", action="store_true",
                   help="do not sample the shader clock (profiled runs use this: no child process)")
    p.add_argument("--config-calls", type=int, default=50, help="timed calls per named workload")
    p.add_argument("--clock-window", type=float, default=2.0,
                   help="seconds of back-to-back steps over which the shader clock is read (half of it per "
                        "named workload)")
    p.add_argument("--workload", default=None, help="time one named workload (fwd or bwd only)")
    p.add_argument("--varlen", action="store_true", help="time fa_fwd_varlen + fa_bwd_varlen on a packed batch")
    p.add_argument("--sweep", action="store_true",
                   help="fa_fwd / fa_bwd throughput over head dim 64/128, N 1K-32K, causal and not, MHA and GQA")
    p.add_argument("--persistent", action="store_true",
                   help="time fa_fwd_persistent beside fa_fwd (forward workload B8 H16 N2048, or --workload)")
    p.add_argument("--fp8", action="store_true",
                   help="time fa_quantize_fp8 (Q and K) + fa_fwd_fp8 beside fa_fwd (B8 H16 N2048, or --workload)")
    p.add_argument("--fp8-d64", action="store_true",
                   help="with --fp8: the head-dim-64 shape B8 H32 N2048 causal (seed 2) instead")
    p.add_argument("--summarize-profiles", default=None, metavar="DIR",
                   help="summarise rocprofv3 output under DIR/{trace,fetch,write,rdreq,tcc} (no GPU needed) and "
                        "record per-launch durations and HBM bytes for the current kernel sources")
    p.add_argument("--profile-out", default=PROFILE_JSON, metavar="PATH",
                   help="where --summarize-profiles records the per-launch figures (default: the step's record "
                        "under profiles/, which the benchmark line reads)")
    p.add_argument("--summarize-pmc", default=None, metavar="DIR",
                   help="summarise a rocprofv3 --pmc run of the SQ counters under DIR (no GPU needed)")
    p.add_argument("--machine-limits", action="store_true",
                   help="run the in-bounds microbenchmarks of tests/hw/machine_limits.hip (matrix-core rate, exp "
                        "beside it, LDS read patterns, shader clock) and print their table")
    p.add_argument("--calibration-mib", type=int, default=256, help="copy size used by the counter runs")
    p.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                   help="after the run, copy a MIB-MiB buffer 3 times (a plain copy kernel of known size, to "
                        "scale the HBM byte counters of a profiler run)")
    p.add_argument("--poll-clock", type=float, default=None, metavar="SECONDS", help=argparse.SUPPRESS)
    return p.parse_args(argv)


# ---------------------------------------------------------------- shader clock

def read_amd_smi_clock(text):
    """Per-XCD shader clocks (MHz) from `amd-smi metric -g 0 --clock --json`
    output, or None when the text holds none."""
    starts = [i for i in (text.find("{"), text.find("[")) if i >= 0]
    if not starts:
        return None
    try:
        d = json.loads(text[min(starts):])
    except json.JSONDecodeError:
        return None
    gpus = d.get("gpu_data", []) if isinstance(d, dict) else d
    if not gpus or not isinstance(gpus[0], dict):
        return None
    clk = gpus[0].get("clock", {})
    mhz = []
    for key in sorted(k for k in clk if k.startswith("gfx_")):
        v = clk[key].get("clk", {}) if isinstance(clk[key], dict) else {}
        v = v.get("value") if isinstance(v, dict) else None
        if isinstance(v, (int, float)):
            mhz.append(float(v))
    return mhz or None


def poll_clock_main(period):
    """Child-process loop: print `time mean min max` (MHz over the XCDs) about
    every `period` seconds until the parent goes away. Touches no HIP API."""
    parent = os.getppid()
    t_stop = time.time() + 1800
    while time.time() < t_stop and os.getppid() == parent:
        t0 = time.time()
        try:
            r = subprocess.run(["amd-smi", "metric", "-g", "0", "--clock", "--json"], capture_output=True,
                               text=True, timeout=10)
        except (OSError, subprocess.SubprocessError):
            return
        mhz = read_amd_smi_clock(r.stdout)
        if mhz:
            t = (t0 + time.time()) / 2
            print(f"{t:.3f} {np.mean(mhz):.1f} {min(mhz):.1f} {max(mhz):.1f}", flush=True)
        time.sleep(max(0.0, period - (time.time() - t0)))


class ClockPoller:
    """Shader-clock samples from a child process running amd-smi. Started
    before this process touches the GPU, so no process that holds a GPU
    context ever forks or execs."""

    def __init__(self, period=0.1):
        self.samples = []  # (time, mean MHz, min MHz, max MHz)
        self.proc = subprocess.Popen([sys.executable, os.path.abspath(__file__), "--poll-clock", str(period)],
                                     stdout=subprocess.PIPE, stderr=subprocess.DEVNULL, text=True)
        self.reader = threading.Thread(target=self._read, daemon=True)
        self.reader.start()

    def _read(self):
        for line in self.proc.stdout:
            f = line.split()
            if len(f) == 4:
                self.samples.append(tuple(float(x) for x in f))

    def window(self, t0, t1):
        """Clock statistics over the samples taken between t0 and t1."""
        return clock_window(self.samples, t0, t1)

    def stop(self):
        if self.proc.poll() is None:
            self.proc.terminate()
            try:
                self.proc.wait(timeout=5)
            except subprocess.TimeoutExpired:
                self.proc.kill()


def clock_window(samples, t0, t1):
    """Median of the per-sample XCD-mean clocks taken between t0 and t1, the
    lowest and highest single-XCD reading, and the sample count; None when
    no sample falls in the window."""
    s = [x for x in samples if t0 <= x[0] <= t1]
    if not s:
        return None
    return {"median": round(float(np.median([x[1] for x in s])), 1), "min_xcd": round(min(x[2] for x in s), 1),
            "max_xcd": round(max(x[3] for x in s), 1), "samples": len(s)}


def peak_at_clock(mhz):
    """Dense bf16 MFMA peak (TFLOP/s) at a shader clock of `mhz`."""
    return BF16_FLOPS_PER_CLK * mhz * 1e6 / 1e12


def run_for(calls, seconds):
    """Issue `calls` back to back for about `seconds` (untimed load under
    which the clock is read); returns (start, end) wall times."""
    import torch
    t0 = time.time()
    while time.time() - t0 < seconds:
        for _ in range(10):
            for c in calls:
                c()
        torch.cuda.synchronize()
    return t0, time.time()


# ---------------------------------------------------------------- device state

def device_inputs(w, with_do):
    import torch
    inp = make_inputs(w.seed, w.batch, w.n_q_heads, w.n_kv_heads, w.seqlen, w.seqlen, w.head_dim, w.dtype,
                      with_do=with_do, n_outlier_channels=w.n_outlier_channels)

    def up(bits, vals):
        if w.dtype == "bf16":
            return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).cuda()
        return torch.from_numpy(vals).cuda()

    q = up(inp.q_bits, inp.q)
    k = up(inp.k_bits, inp.k)
    v = up(inp.v_bits, inp.v)
    do = up(inp.do_bits, inp.do) if with_do else None
    return inp, q, k, v, do


class Step:
    """The hot path with every output buffer allocated once, up front."""

    def __init__(self, w, q, k, v, do):
        import torch
        self.w = w
        self.q, self.k, self.v, self.do = q, k, v, do
        B, Hq, Hkv, N, d = w.batch, w.n_q_heads, w.n_kv_heads, w.seqlen, w.head_dim
        dev = q.device
        self.o = torch.empty((B, Hq, N, d), dtype=q.dtype, device=dev)
        self.lse = torch.empty((B, Hq, N), dtype=torch.float32, device=dev)
        self.dq = torch.empty((B, Hq, N, d), dtype=torch.float32, device=dev)
        self.dk = torch.empty((B, Hkv, N, d), dtype=q.dtype, device=dev)
        self.dv = torch.empty((B, Hkv, N, d), dtype=q.dtype, device=dev)
        self.ws = torch.empty(binding.fa_bwd_workspace_bytes(B, Hq, N) // 4, dtype=torch.float32, device=dev)
        self.code = binding.FA_DTYPE_BF16 if w.dtype == "bf16" else binding.FA_DTYPE_F32
        self.stream = torch.cuda.current_stream()
        self.sh = self.stream.cuda_stream
        self.precision = binding.FA_PRECISION_BF16

    def fwd(self):
        w = self.w
        rc = binding.fa_fwd(self.q.data_ptr(), self.k.data_ptr(), self.v.data_ptr(), self.o.data_ptr(),
                            self.lse.data_ptr(), w.batch, w.n_q_heads, w.n_kv_heads, w.seqlen, w.seqlen,
                            w.head_dim, w.scale, int(w.causal), self.code, self.code, self.sh)
        if rc:
            raise binding.FAError(rc, "fa_fwd", binding.fa_last_error())

    def bwd_atomic(self):
        self.bwd(binding.fa_bwd_atomic)

    def bwd(self, fn=None):
        w = self.w
        fn = fn or binding.fa_bwd
        rc = fn(self.q.data_ptr(), self.k.data_ptr(), self.v.data_ptr(), self.o.data_ptr(),
                self.lse.data_ptr(), self.do.data_ptr(), self.dq.data_ptr(), self.dk.data_ptr(),
                self.dv.data_ptr(), self.ws.data_ptr(), w.batch, w.n_q_heads, w.n_kv_heads, w.seqlen,
                w.seqlen, w.head_dim, w.scale, int(w.causal), self.code, self.code, self.code,
                self.precision, self.sh)
        if rc:
            raise binding.FAError(rc, fn.__name__, binding.fa_last_error())


def time_calls(step, calls, steps, warmup):
    """Run `calls` (a list of callables) per step; return the step times and
    per-call times (ms) from HIP events recorded on the launch stream, and
    the wall-clock ms per step over the synchronised timed region."""
    import torch
    stream = step.stream if step is not None else torch.cuda.current_stream()
    for _ in range(warmup):
        for c in calls:
            c()
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(calls) + 1)] for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(steps):
        ev[s][0].record(stream)
        for i, c in enumerate(calls):
            c()
            ev[s][i + 1].record(stream)
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) * 1e3 / steps
    per_call = np.array([[ev[s][i].elapsed_time(ev[s][i + 1]) for i in range(len(calls))] for s in range(steps)])
    per_step = per_call.sum(axis=1)
    return per_step, per_call, wall


def time_stats(ms, flops, nbytes, clock):
    """Summary of one call's timed durations (ms): median, min, p90, mean,
    throughput at the median, and % of peak (published, and at `clock`)."""
    ms = np.asarray(ms, dtype=np.float64)
    med = float(np.median(ms))
    tf = flops / (med * 1e-3) / 1e12
    out = {"calls": int(len(ms)), "ms_median": round(med, 4), "ms_min": round(float(ms.min()), 4),
           "ms_p90": round(float(np.percentile(ms, 90)), 4), "ms_mean": round(float(ms.mean()), 4),
           "tflops": round(tf, 2), "pct_of_bf16_peak": round(100 * tf / MI355X_BF16_PEAK_TFLOPS, 2),
           "gbps_algorithmic": round(nbytes / (med * 1e-3) / 1e9, 1)}
    if clock:
        out["clock_mhz"] = clock["median"]
        out["pct_of_bf16_peak_at_clock"] = round(100 * tf / peak_at_clock(clock["median"]), 2)
    return out


def time_config(w, calls_n, warmup, poller, window_s):
    """Time one named workload's pass (`calls_n` calls after `warmup`), then
    read the clock under `window_s` seconds of the same calls."""
    inp, q, k, v, do = device_inputs(w, with_do=w.passes == "bwd")
    step = Step(w, q, k, v, do if do is not None else q)
    if w.passes == "bwd":
        step.fwd()
        calls = [step.bwd]
    else:
        calls = [step.fwd]
    per_step, _, _ = time_calls(step, calls, calls_n, warmup)
    clock = None
    if poller is not None:
        t0, t1 = run_for(calls, window_s)
        clock = poller.window(t0 + 0.25 * window_s, t1)
    res = time_stats(per_step, workload_flops(w), workload_bytes(w), clock)
    res["pass"] = "fa_bwd" if w.passes == "bwd" else "fa_fwd"
    return inp, res


# ---------------------------------------------------------------- CPU oracle

def host_description():
    """CPU model, logical CPUs this process may use, and the BLAS numpy calls."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    blas, threads = "unknown", len(os.sched_getaffinity(0))
    try:
        from threadpoolctl import threadpool_info
        info = [i for i in threadpool_info() if i.get("user_api") == "blas"]
        if info:
            i = info[0]
            threads = int(i.get("num_threads", threads))
            blas = (f"{i.get('internal_api')} {i.get('version')} ({i.get('architecture')} kernels, "
                    f"{i.get('threading_layer')} threads)")
    except Exception:
        pass
    return {"cpu_model": model, "logical_cpus": len(os.sched_getaffinity(0)), "blas": blas,
            "blas_threads": threads}


def cpu_oracle_sample(w, inp, slices, with_bwd):
    """Time the fp64 oracle, untuned, on the first `slices` (batch, head)
    slices of workload `w`: forward, plus backward when `with_bwd`.
    Returns (TFLOPS on the causal-adjusted count, seconds, slices)."""
    import oracle
    sel = [(b, h) for b in range(w.batch) for h in range(w.n_q_heads)][:slices]
    t0 = time.perf_counter()
    for b, h in sel:
        g = h // w.group
        oracle.forward_head(inp.q[b, h], inp.k[b, g], inp.v[b, g], w.scale, w.causal)
        if with_bwd:
            oracle.backward_head(inp.q[b, h], inp.k[b, g], inp.v[b, g], inp.do[b, h], w.scale, w.causal)
    dt = time.perf_counter() - t0
    fl = fwd_flops(1, 1, w.seqlen, w.seqlen, w.head_dim, w.causal)
    if with_bwd:
        fl += bwd_flops(1, 1, w.seqlen, w.seqlen, w.head_dim, w.causal)
    return len(sel) * fl / dt / 1e12, dt, len(sel)


# ---------------------------------------------------------------- extra modes

# Packed variable-length batch timed by --varlen: 16 causal sequences whose
# lengths are drawn uniformly from [256, 4096] (seed 11), Hq = Hkv = 16,
# d = 128, bf16 (a mix like the unequal-length batches the FlashAttention-3
# news page names; no dataset is involved).
VARLEN_SEED, VARLEN_SEQS, VARLEN_MIN, VARLEN_MAX, VARLEN_H, VARLEN_D = 11, 16, 256, 4096, 16, 128
DEFAULT_FWD = "fwd_bf16_causal_b8_h16_n2048_d128"


def bench_varlen(args):
    """Time fa_fwd_varlen + fa_bwd_varlen on the packed batch above; prints
    one JSON line (TFLOPS on the causal-adjusted count summed over the
    sequences)."""
    import torch
    from exact_tiled_attention_28_amd.inputs import make_varlen_inputs
    rng = np.random.default_rng(VARLEN_SEED)
    lengths = rng.integers(VARLEN_MIN, VARLEN_MAX + 1, size=VARLEN_SEQS)
    inp = make_varlen_inputs(VARLEN_SEED, lengths, lengths, VARLEN_H, VARLEN_H, VARLEN_D, with_do=True)
    dev = torch.device("cuda")
    up = lambda x: torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(dev).bfloat16()
    q, k, v, do = up(inp.q), up(inp.k), up(inp.v), up(inp.do)
    cu = torch.from_numpy(inp.cu_q).to(dev)
    H, T, d = q.shape
    scale = float(np.float32(1 / np.sqrt(d)))
    o = torch.empty_like(q)
    lse = torch.empty((H, T), dtype=torch.float32, device=dev)
    dq = torch.empty((H, T, d), dtype=torch.float32, device=dev)
    dk, dv = torch.empty_like(k), torch.empty_like(v)
    ws = torch.empty(binding.fa_bwd_workspace_bytes(1, H, T) // 4, dtype=torch.float32, device=dev)
    sh = torch.cuda.current_stream().cuda_stream
    bf = binding.FA_DTYPE_BF16
    B, mx = len(lengths), int(inp.max_q)

    def fwd():
        rc = binding.fa_fwd_varlen(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                                   cu.data_ptr(), cu.data_ptr(), B, mx, mx, T, T, H, H, d, scale, 1, bf, bf, sh)
        if rc:
            raise binding.FAError(rc, "fa_fwd_varlen", binding.fa_last_error())

    def bwd():
        rc = binding.fa_bwd_varlen(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                                   do.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), ws.data_ptr(),
                                   cu.data_ptr(), cu.data_ptr(), B, mx, mx, T, T, H, H, d, scale, 1, bf, bf, bf,
                                   binding.FA_PRECISION_BF16, sh)
        if rc:
            raise binding.FAError(rc, "fa_bwd_varlen", binding.fa_last_error())

    _, per_call, _ = time_calls(None, [fwd, bwd], args.steps, args.warmup)
    fwd_ms, bwd_ms = float(np.median(per_call[:, 0])), float(np.median(per_call[:, 1]))
    ff = sum(fwd_flops(1, H, int(n), int(n), d, True) for n in lengths)
    bfl = sum(bwd_flops(1, H, int(n), int(n), d, True) for n in lengths)
    out = {"workload": f"varlen causal bf16: {B} sequences, lengths U[{VARLEN_MIN},{VARLEN_MAX}] (seed {VARLEN_SEED}), "
                       f"total {T} tokens, max {mx}, H={H}, d={d}",
           "fwd_ms": round(fwd_ms, 4), "fwd_tflops": round(ff / (fwd_ms * 1e-3) / 1e12, 2),
           "bwd_ms": round(bwd_ms, 4), "bwd_tflops": round(bfl / (bwd_ms * 1e-3) / 1e12, 2)}
    out["fwd_pct_of_bf16_peak"] = round(100 * out["fwd_tflops"] / MI355X_BF16_PEAK_TFLOPS, 2)
    out["bwd_pct_of_bf16_peak"] = round(100 * out["bwd_tflops"] / MI355X_BF16_PEAK_TFLOPS, 2)
    print(json.dumps(out), flush=True)


SWEEP_TOKENS, SWEEP_HD = 16384, 2048  # B * N tokens and Hq * d per shape


def bench_sweep(args):
    """Throughput of fa_fwd (bf16 O) and fa_bwd (fp32 dQ, bf16 dK/dV) over
    head dim 64/128, N = 128..32K, causal and non-causal, MHA and GQA (G = 4),
    with B = max(1, 16384 / N) and Hq = 2048 / d: N(0, 1) bf16 inputs drawn on
    the GPU from a seeded generator. One JSON line per shape (median of
    --steps timed calls after --warmup): TFLOP/s and % of the bf16 peak, and
    the algorithmic HBM rate (fwd_bytes / bwd_bytes over the time) with its %
    of 8 TB/s, the bound that matters for the short sequences; then a summary
    line."""
    import torch
    rows = []
    for d in (64, 128):
        for n in (128, 256, 512, 1024, 2048, 4096, 8192, 16384, 32768):
            for causal in (True, False):
                for group in (1, 4):
                    B, Hq = max(1, SWEEP_TOKENS // n), SWEEP_HD // d
                    Hkv = Hq // group
                    g = torch.Generator(device="cuda").manual_seed(1000 + n + d + group)
                    q = torch.randn(B, Hq, n, d, device="cuda", generator=g).bfloat16()
                    k = torch.randn(B, Hkv, n, d, device="cuda", generator=g).bfloat16()
                    v = torch.randn(B, Hkv, n, d, device="cuda", generator=g).bfloat16()
                    do = torch.randn(B, Hq, n, d, device="cuda", generator=g).bfloat16()
                    scale = float(np.float32(1 / np.sqrt(d)))
                    o = torch.empty_like(q)
                    lse = torch.empty((B, Hq, n), dtype=torch.float32, device="cuda")
                    dq = torch.empty((B, Hq, n, d), dtype=torch.float32, device="cuda")
                    dk, dv = torch.empty_like(k), torch.empty_like(v)
                    ws = torch.empty(binding.fa_bwd_workspace_bytes(B, Hq, n) // 4, dtype=torch.float32,
                                     device="cuda")
                    sh = torch.cuda.current_stream().cuda_stream
                    bf = binding.FA_DTYPE_BF16

                    def fwd():
                        rc = binding.fa_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                                            B, Hq, Hkv, n, n, d, scale, int(causal), bf, bf, sh)
                        if rc:
                            raise binding.FAError(rc, "fa_fwd", binding.fa_last_error())

                    def bwd():
                        rc = binding.fa_bwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                                            do.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), ws.data_ptr(),
                                            B, Hq, Hkv, n, n, d, scale, int(causal), bf, bf, bf,
                                            binding.FA_PRECISION_BF16, sh)
                        if rc:
                            raise binding.FAError(rc, "fa_bwd", binding.fa_last_error())

                    _, per_call, _ = time_calls(None, [fwd, bwd], args.steps, args.warmup)
                    fm, bm = float(np.median(per_call[:, 0])), float(np.median(per_call[:, 1]))
                    ff, bfl = fwd_flops(B, Hq, n, n, d, causal), bwd_flops(B, Hq, n, n, d, causal)
                    row = {"d": d, "N": n, "B": B, "Hq": Hq, "Hkv": Hkv, "causal": causal,
                           "fwd_ms": round(fm, 4), "fwd_tflops": round(ff / (fm * 1e-3) / 1e12, 1),
                           "bwd_ms": round(bm, 4), "bwd_tflops": round(bfl / (bm * 1e-3) / 1e12, 1)}
                    row["fwd_pct"] = round(100 * row["fwd_tflops"] / MI355X_BF16_PEAK_TFLOPS, 1)
                    row["bwd_pct"] = round(100 * row["bwd_tflops"] / MI355X_BF16_PEAK_TFLOPS, 1)
                    fb, bb = fwd_bytes(B, Hq, Hkv, n, n, d), bwd_bytes(B, Hq, Hkv, n, n, d)
                    row["fwd_gbps"] = round(fb / (fm * 1e-3) / 1e9, 1)
                    row["bwd_gbps"] = round(bb / (bm * 1e-3) / 1e9, 1)
                    row["fwd_pct_hbm"] = round(100 * row["fwd_gbps"] / MI355X_HBM_GBPS, 1)
                    row["bwd_pct_hbm"] = round(100 * row["bwd_gbps"] / MI355X_HBM_GBPS, 1)
                    rows.append(row)
                    print(json.dumps(row), flush=True)
                    del q, k, v, do, o, lse, dq, dk, dv, ws
    best = max(rows, key=lambda r: r["fwd_tflops"] if r["causal"] and r["d"] == 128 else 0)
    best_short = max(rows, key=lambda r: r["fwd_gbps"] if r["N"] <= 512 else 0)
    print(json.dumps({"sweep_shapes": len(rows), "best_causal_d128_fwd": best, "best_short_fwd_gbps": best_short}),
          flush=True)


def bench_persistent(args):
    """Time fa_fwd_persistent (work-queue grid) and fa_fwd (one workgroup per
    item) on the same forward workload; prints one JSON line."""
    import torch
    w = WORKLOADS[args.workload or DEFAULT_FWD]
    if w.passes != "fwd" or w.dtype != "bf16":
        raise SystemExit(f"--persistent needs a bf16 forward workload, not {w.name}")
    _, q, k, v, _ = device_inputs(w, with_do=False)
    step = Step(w, q, k, v, q)
    sched = binding.new_sched()
    o = torch.empty(q.shape, dtype=torch.bfloat16, device=q.device)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=q.device)
    stream = torch.cuda.current_stream()

    def persist():
        binding.forward_persistent(q, k, v, w.scale, w.causal, sched, o=o, lse=lse, stream=stream)

    _, per_call, _ = time_calls(None, [persist, step.fwd], args.steps, args.warmup)
    med = [float(np.median(per_call[:, i])) for i in range(2)]
    ff = fwd_flops(w.batch, w.n_q_heads, w.seqlen, w.seqlen, w.head_dim, w.causal)
    out = {"workload": f"{w.name}: fa_fwd_persistent vs fa_fwd", "persistent_ms": round(med[0], 4),
           "persistent_tflops": round(ff / (med[0] * 1e-3) / 1e12, 2), "fa_fwd_ms": round(med[1], 4),
           "fa_fwd_tflops": round(ff / (med[1] * 1e-3) / 1e12, 2),
           "persistent_pct_of_bf16_peak": round(100 * ff / (med[0] * 1e-3) / 1e12 / MI355X_BF16_PEAK_TFLOPS, 2)}
    print(json.dumps(out), flush=True)


MI355X_FP8_PEAK_TFLOPS = 5000.0  # dense fp8 MFMA


def bench_fp8(args):
    """Time the FP8 forward path on one forward workload: fa_quantize_fp8 of
    Q and of K (random-sign Hadamard transform, seed = the workload's) and
    fa_fwd_fp8 (bf16 O), with fa_fwd on the same inputs beside it, then
    fa_quantize_vt_fp8 of V and fa_fwd_fp8_pv (P V in FP8 too), and
    fa_fwd_fp8_quantize_q (Q quantized inside the forward) with either V.
    Prints one JSON line. The roofline of fa_fwd_fp8 counts S = Q K^T at the fp8 peak
    and O = P V at the bf16 peak (half of the flops each); that of
    fa_fwd_fp8_pv counts both at the fp8 peak."""
    import torch
    from exact_tiled_attention_28_amd.inputs import make_signs
    from exact_tiled_attention_28_amd.workloads import Workload
    if args.fp8_d64:
        w = Workload("fwd_bf16_causal_b8_h32_n2048_d64", 8, 32, 32, 2048, 64, True, "bf16", "fwd", 2)
    else:
        w = WORKLOADS[args.workload or DEFAULT_FWD]
    if w.passes != "fwd" or w.dtype != "bf16":
        raise SystemExit(f"--fp8 needs a bf16 forward workload, not {w.name}")
    _, q, k, v, _ = device_inputs(w, with_do=False)
    step = Step(w, q, k, v, q)
    signs = torch.from_numpy(make_signs(w.seed, w.head_dim)).cuda()
    qc, qs = binding.quantize_fp8(q, signs)
    kc, ks = binding.quantize_fp8(k, signs)
    o = torch.empty(q.shape, dtype=torch.bfloat16, device=q.device)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=q.device)
    stream = torch.cuda.current_stream()

    def quant_q():
        binding.quantize_fp8(q, signs, qc, qs, stream=stream)

    def quant_k():
        binding.quantize_fp8(k, signs, kc, ks, stream=stream)

    def fwd8():
        binding.forward_fp8(qc, qs, kc, ks, v, w.scale, w.causal, o=o, lse=lse, stream=stream)

    vt, vs = binding.quantize_vt_fp8(v)

    def quant_v():
        binding.quantize_vt_fp8(v, vt, vs, stream=stream)

    def fwd8pv():
        binding.forward_fp8_pv(qc, qs, kc, ks, vt, vs, w.scale, w.causal, o=o, lse=lse, stream=stream)

    def fwd8q():
        binding.forward_fp8_quantize_q(q, kc, ks, v, w.scale, w.causal, signs=signs, o=o, lse=lse, stream=stream)

    def fwd8qpv():
        binding.forward_fp8_quantize_q(q, kc, ks, vt, w.scale, w.causal, signs=signs, v_scales=vs, o=o, lse=lse,
                                       stream=stream)

    _, per_call, _ = time_calls(None, [quant_q, quant_k, fwd8, step.fwd, quant_v, fwd8pv, fwd8q, fwd8qpv], args.steps,
                                args.warmup)
    med = [float(np.median(per_call[:, i])) for i in range(8)]
    avgpv = float(np.mean(per_call[:, 5]))
    avg8 = float(np.mean(per_call[:, 2]))
    ff = fwd_flops(w.batch, w.n_q_heads, w.seqlen, w.seqlen, w.head_dim, w.causal)
    peak_mixed = 2.0 / (1.0 / MI355X_FP8_PEAK_TFLOPS + 1.0 / MI355X_BF16_PEAK_TFLOPS)
    tf8 = ff / (med[2] * 1e-3) / 1e12
    ach = ff / (avg8 * 1e-3) / 1e12
    el = w.batch * w.n_q_heads * w.seqlen * w.head_dim
    qbytes = el * 2 + el + w.batch * w.n_q_heads * (-(-w.seqlen // 64)) * 4  # bf16 in, codes + scales out
    out = {"workload": f"{w.name}: fa_quantize_fp8(Q), fa_quantize_fp8(K), fa_fwd_fp8 (bf16 O)",
           "quantize_q_ms": round(med[0], 4), "quantize_q_gbps": round(qbytes / (med[0] * 1e-3) / 1e9, 1),
           "quantize_k_ms": round(med[1], 4),
           "fwd_fp8_ms": round(med[2], 4), "fwd_fp8_tflops": round(tf8, 2),
           "fp8_path_ms": round(sum(med[:3]), 4),
           "fp8_path_tflops": round(ff / (sum(med[:3]) * 1e-3) / 1e12, 2),
           "fwd_bf16_ms": round(med[3], 4), "fwd_bf16_tflops": round(ff / (med[3] * 1e-3) / 1e12, 2),
           "quantize_vt_ms": round(med[4], 4),
           "fwd_fp8_pv_ms": round(med[5], 4), "fwd_fp8_pv_tflops": round(ff / (med[5] * 1e-3) / 1e12, 2),
           "fp8_pv_path_ms": round(med[0] + med[1] + med[4] + med[5], 4),
           "fwd_fp8_quantize_q_ms": round(med[6], 4),
           "fwd_fp8_quantize_q_tflops": round(ff / (med[6] * 1e-3) / 1e12, 2),
           "fwd_fp8_quantize_q_pv_ms": round(med[7], 4),
           "fwd_fp8_quantize_q_pv_tflops": round(ff / (med[7] * 1e-3) / 1e12, 2),
           "fp8_fused_q_path_ms": round(med[1] + med[6], 4),
           "fp8_fused_q_pv_path_ms": round(med[1] + med[4] + med[7], 4),
           "roofline_fp8_pv": {"kernel": "fa_fwd_fp8_pv (fwd_fp8_kernel, P V in FP8)", "bound": "mfma",
                               "achieved": round(ff / (avgpv * 1e-3) / 1e12, 2), "peak": MI355X_FP8_PEAK_TFLOPS,
                               "unit": "TFLOP/s",
                               "frac": round(ff / (avgpv * 1e-3) / 1e12 / MI355X_FP8_PEAK_TFLOPS, 4),
                               "avg_launch_ms": round(avgpv, 4)},
           "roofline": {"kernel": "fa_fwd_fp8 (fwd_fp8_kernel)", "bound": "mfma", "achieved": round(ach, 2),
                        "peak": round(peak_mixed, 1), "unit": "TFLOP/s", "frac": round(ach / peak_mixed, 4),
                        "peak_note": "half the flops (Q K^T) at the 5.0 PFLOP/s fp8 peak, half (P V) at the "
                                     "2.5166 PFLOP/s bf16 peak", "avg_launch_ms": round(avg8, 4)}}
    print(json.dumps(out), flush=True)


def bench_one(args):
    """Time one named workload's pass (fwd or bwd); prints one JSON line."""
    _, res = time_config(WORKLOADS[args.workload], args.steps, args.warmup, None, 0)
    res["workload"] = args.workload
    print(json.dumps(res), flush=True)


# ---------------------------------------------------------------- profiles

def csrc_sha256():
    """sha256 over the kernel sources (file names and contents, sorted)."""
    import hashlib
    csrc = os.path.join(ROOT, "exact_tiled_attention_28_amd", "csrc")
    h = hashlib.sha256()
    for f in sorted(os.listdir(csrc)):
        h.update(f.encode())
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


# Kernels of each C entry point, by the name rocprofv3 reports (demangled,
# or mangled for the preprocess kernel, whose last template argument says
# whether it also zeroes dQ: only fa_bwd_atomic's does).
CALL_KERNELS = {
    "fa_fwd": ("void fa::fwd_kernel<",),
    "fa_bwd": ("void fa::bwd_dkdv_kernel<", "void fa::bwd_dkdv4_kernel<", "void fa::bwd_dq_kernel<"),
    "fa_bwd_atomic": ("void fa::bwd_kernel<",),
    "fa_quantize_fp8": ("void fa::quantize_fp8_kernel<",),
    "fa_quantize_vt_fp8": ("void fa::quantize_vt_fp8_kernel<",),
    "fa_fwd_fp8": ("void fa::fwd_fp8_kernel<",),
}


def _template_args(kernel):
    """Template arguments of a demangled kernel name, as strings."""
    if "<" not in kernel or ">(" not in kernel:
        return []
    return [t.strip() for t in kernel[kernel.index("<") + 1:kernel.rindex(">(")].split(",")]


# Position of the VARLEN / PERSIST / PV8 template argument of each kernel template
# (fwd_kernel<F32IN, D, CAUSAL, OUTF32, NW, VARLEN, PERSIST>,
# bwd_dkdv_kernel<D, CAUSAL, GF32, VARLEN, HILO>, bwd_dkdv4_kernel<D, CAUSAL, GF32, VARLEN>,
# bwd_dq_kernel<D, CAUSAL, VARLEN, NW, HILO>, fwd_fp8_kernel<D, CAUSAL, OUTF32, PV8, QBF16>).
_VARLEN_ARG = {
    "void fa::fwd_kernel<": 5,
    "void fa::bwd_dkdv_kernel<": 3,
    "void fa::bwd_dkdv4_kernel<": 3,
    "void fa::bwd_dq_kernel<": 2,
}
_PERSIST_ARG = {"void fa::fwd_kernel<": 6}
_PV8_ARG = {"void fa::fwd_fp8_kernel<": 3}
_QBF16_ARG = {"void fa::fwd_fp8_kernel<": 4}


def _call_of(kernel):
    t = _template_args(kernel)
    for prefix, pos in _QBF16_ARG.items():
        if kernel.startswith(prefix) and len(t) > pos and t[pos] == "true":
            return "fa_fwd_fp8_quantize_q"
    for prefix, pos in _PV8_ARG.items():
        if kernel.startswith(prefix) and len(t) > pos and t[pos] == "true":
            return "fa_fwd_fp8_pv"
    for prefix, pos in _PERSIST_ARG.items():
        if kernel.startswith(prefix) and len(t) > pos and t[pos] == "true":
            return "fa_fwd_persistent"
    for prefix, pos in _VARLEN_ARG.items():
        if kernel.startswith(prefix) and len(t) > pos and t[pos] == "true":
            return "fa_fwd_varlen" if prefix == "void fa::fwd_kernel<" else "fa_bwd_varlen"
    if "bwd_preprocess_kernel" in kernel:
        zero_dq = kernel.rstrip().endswith(", true>(fa::BwdArgs)") or "Lb1EEEv" in kernel or ", true>" in kernel
        return "fa_bwd_atomic" if zero_dq else "fa_bwd"
    for call, prefixes in CALL_KERNELS.items():
        if kernel.startswith(prefixes):
            return call
    return None


def _csv_rows(prof_dir, sub, suffix):
    import csv
    import glob
    files = glob.glob(os.path.join(prof_dir, sub, "*" + suffix))
    if not files:
        return None
    with open(files[0]) as fh:
        return list(csv.DictReader(fh))


def _counter_means(rows, names):
    """Mean over dispatches of each counter in `names`, per kernel name."""
    acc = {}
    for r in rows:
        if r["Counter_Name"] not in names:
            continue
        k = acc.setdefault(r["Kernel_Name"], {}).setdefault(r["Counter_Name"], {})
        k[r["Dispatch_Id"]] = k.get(r["Dispatch_Id"], 0.0) + float(r["Counter_Value"])
    return {kern: {c: sum(v.values()) / len(v) for c, v in per.items()} for kern, per in acc.items()}


RDREQ_COUNTERS = ("TCC_EA0_RDREQ_sum", "TCC_EA0_RDREQ_32B_sum", "TCC_EA0_RDREQ_64B_sum", "TCC_EA0_RDREQ_128B_sum")
TCC_COUNTERS = ("TCC_HIT_sum", "TCC_MISS_sum", "TCC_EA0_RDREQ_DRAM_sum")


def summarize_profiles(prof_dir, calib_mib, out_path=None):
    """Turn the rocprofv3 output of one kernel-trace run (prof_dir/trace) and
    the counter runs (prof_dir/fetch: FETCH_SIZE, prof_dir/write: WRITE_SIZE,
    prof_dir/rdreq: RDREQ_COUNTERS, prof_dir/tcc: TCC_COUNTERS; each with
    --copy-calibration calib_mib) into markdown tables on stdout, and record
    per-launch kernel durations and HBM bytes of each entry point for the
    current kernel sources in PROFILE_JSON (or out_path). Counter runs that
    are absent are skipped."""
    stats = _csv_rows(prof_dir, "trace", "kernel_stats.csv")
    if stats is None:
        raise SystemExit(f"no *kernel_stats.csv under {os.path.join(prof_dir, 'trace')}")
    total = sum(float(r["TotalDurationNs"]) for r in stats)
    print("| kernel | entry point | calls | average µs | min µs | max µs | share |")
    print("|---|---|---|---|---|---|---|")
    per_call = {}
    for r in stats:
        name = r["Name"]
        call = _call_of(name)
        avg = float(r["AverageNs"]) / 1e3
        print(f"| `{name}` | {call or '-'} | {r['Calls']} | {avg:.1f} | {float(r['MinNs']) / 1e3:.1f} | "
              f"{float(r['MaxNs']) / 1e3:.1f} | {100 * float(r['TotalDurationNs']) / total:.1f}% |")
        if call:
            c = per_call.setdefault(call, {"kernel_avg_us": 0.0})
            c["kernel_avg_us"] = round(c["kernel_avg_us"] + avg, 2)
    print()
    for call, c in sorted(per_call.items()):
        print(f"- `{call}`: sum of its kernels' average durations {c['kernel_avg_us']:.1f} µs")
    print()
    rec = {"note": "per launch of each entry point: the sum of its kernels' average durations (rocprofv3 "
                   "--kernel-trace --stats); HBM bytes from rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE (KiB per "
                   "dispatch) scaled by the same counters on a copy of known size; read bytes counted from "
                   "TCC_EA0_RDREQ by request size; L2 hits and misses",
           "kernel_sources_sha256": csrc_sha256(), "workload": STEP_WORKLOAD}

    calib_kib = calib_mib * 1024

    def copy_scale(per, cname):
        copies = [v[cname] for name, v in per.items() if "copyBuffer" in name and cname in v]
        if not copies:
            raise SystemExit(f"{cname}: no copy kernel in the counter run (run it with --copy-calibration)")
        return calib_kib / (sum(copies) / len(copies))

    fetch_scaled = {}  # kernel name -> copy-calibrated FETCH_SIZE bytes per dispatch
    fetch = _csv_rows(prof_dir, "fetch", "counter_collection.csv")
    write = _csv_rows(prof_dir, "write", "counter_collection.csv")
    if fetch is not None and write is not None:
        fmeans = _counter_means(fetch, {"FETCH_SIZE"})
        wmeans = _counter_means(write, {"WRITE_SIZE"})
        sf, sw = copy_scale(fmeans, "FETCH_SIZE"), copy_scale(wmeans, "WRITE_SIZE")
        print(f"Calibration: a copy of {calib_mib} MiB reads {calib_kib / sf:.0f} KiB of FETCH_SIZE "
              f"(scale x{sf:.4f}) and {calib_kib / sw:.0f} KiB of WRITE_SIZE (scale x{sw:.4f}).")
        print()
        print("| kernel | entry point | FETCH_SIZE KiB | WRITE_SIZE KiB | HBM MB (scaled) |")
        print("|---|---|---|---|---|")
        for name in sorted(set(fmeans) | set(wmeans)):
            call = _call_of(name)
            if call is None:
                continue
            f = fmeans.get(name, {}).get("FETCH_SIZE", 0.0)
            wr = wmeans.get(name, {}).get("WRITE_SIZE", 0.0)
            fb, wb = f * 1024 * sf, wr * 1024 * sw
            fetch_scaled[name] = fb
            print(f"| `{name}` | {call} | {f:.0f} | {wr:.0f} | {(fb + wb) / 1e6:.0f} |")
            c = per_call.setdefault(call, {})
            c["fetch_bytes"] = c.get("fetch_bytes", 0) + int(round(fb))
            c["write_bytes"] = c.get("write_bytes", 0) + int(round(wb))
        print()
        rec["fetch_scale"], rec["write_scale"] = round(sf, 4), round(sw, 4)

    rdreq = _csv_rows(prof_dir, "rdreq", "counter_collection.csv")
    if rdreq is not None:
        means = _counter_means(rdreq, set(RDREQ_COUNTERS))
        print("Read bytes counted from the requests the L2 sends to the fabric, by size "
              "(32 x n32 + 64 x n64 + 128 x n128; 'unsized' = requests minus the three sized counts):")
        print()
        print("| kernel | entry point | requests | 32 B | 64 B | 128 B | unsized | read MB | "
              "FETCH_SIZE-scaled MB |")
        print("|---|---|---|---|---|---|---|---|---|")
        for name, m in sorted(means.items()):
            call = _call_of(name) or ("copy" if "copyBuffer" in name else None)
            if call is None:
                continue
            n, n32, n64, n128 = (m.get(s, 0.0) for s in RDREQ_COUNTERS)
            rb = 32 * n32 + 64 * n64 + 128 * n128
            fs = fetch_scaled.get(name)
            print(f"| `{name}` | {call} | {n:.0f} | {n32:.0f} | {n64:.0f} | {n128:.0f} | "
                  f"{max(0, round(n - n32 - n64 - n128))} | {rb / 1e6:.0f} | {'-' if fs is None else f'{fs / 1e6:.0f}'} |")
            if call != "copy":
                c = per_call.setdefault(call, {})
                c["read_bytes_by_request_size"] = c.get("read_bytes_by_request_size", 0) + int(round(rb))
        print()

    tcc = _csv_rows(prof_dir, "tcc", "counter_collection.csv")
    if tcc is not None:
        means = _counter_means(tcc, set(TCC_COUNTERS))
        print("L2 (TCC) hits and misses, and read requests sent towards DRAM (the memory-side MALL sits "
              "behind this point, so a DRAM request may still be served by the MALL):")
        print()
        print("| kernel | entry point | L2 hits | L2 misses | L2 hit rate | DRAM read requests |")
        print("|---|---|---|---|---|---|")
        for name, m in sorted(means.items()):
            call = _call_of(name) or ("copy" if "copyBuffer" in name else None)
            if call is None:
                continue
            hit, miss, dram = (m.get(s, 0.0) for s in TCC_COUNTERS)
            rate = hit / (hit + miss) if hit + miss else float("nan")
            print(f"| `{name}` | {call} | {hit:.0f} | {miss:.0f} | {100 * rate:.1f}% | {dram:.0f} |")
            if call != "copy":
                c = per_call.setdefault(call, {})
                c["l2_hits"] = c.get("l2_hits", 0) + int(round(hit))
                c["l2_misses"] = c.get("l2_misses", 0) + int(round(miss))
                c["dram_read_requests"] = c.get("dram_read_requests", 0) + int(round(dram))
        print()

    for call, c in sorted(per_call.items()):
        if "fetch_bytes" in c:
            print(f"- `{call}`: {(c['fetch_bytes'] + c['write_bytes']) / 1e6:.0f} MB of HBM traffic per launch "
                  f"(copy-calibrated FETCH_SIZE + WRITE_SIZE)")
    rec.update(per_call)
    out_path = out_path or PROFILE_JSON
    with open(out_path, "w") as fh:
        json.dump(rec, fh, indent=1)
    print(f"\nkernel sources sha256 {rec['kernel_sources_sha256']}")


SQ_COUNTERS = ("GRBM_GUI_ACTIVE", "SQ_WAVES", "SQ_INSTS_VALU", "SQ_INSTS_MFMA", "SQ_INSTS_LDS",
               "SQ_VALU_MFMA_BUSY_CYCLES", "SQ_LDS_BANK_CONFLICT", "SQ_VALU_MFMA_COEXEC_CYCLES",
               "SQ_ACTIVE_INST_VALU")


# The second counter pass: LDS activity and where the wavefronts wait.
LDS_WAIT_COUNTERS = ("GRBM_GUI_ACTIVE", "SQ_WAVES", "SQ_WAVE_CYCLES", "SQ_WAIT_ANY", "SQ_WAIT_INST_ANY",
                     "SQ_WAIT_INST_LDS", "SQ_LDS_IDX_ACTIVE", "SQ_LDS_DATA_FIFO_FULL", "SQ_BUSY_CYCLES")


def summarize_pmc(prof_dir, n_xcd=8, n_simd=1024, n_cu=256):
    """Per-kernel averages of one rocprofv3 --pmc run of SQ_COUNTERS: clock
    (GRBM_GUI_ACTIVE, summed over the n_xcd XCD instances, over the
    dispatch's duration), MFMA busy (SQ_VALU_MFMA_BUSY_CYCLES over n_simd
    SIMDs x the kernel's cycles, rocprofv3's MfmaUtil expression), VALU busy
    (rocprofv3's VALUBusy expression: SQ_ACTIVE_INST_VALU / n_cu / cycles),
    co-execution (SQ_VALU_MFMA_COEXEC_CYCLES, cycles in which a SIMD issued a
    VALU instruction while its MFMA unit was busy, as a share of the MFMA
    busy cycles), instructions per wavefront and LDS bank-conflict cycles.
    Counters absent from the run read as zero. A run of LDS_WAIT_COUNTERS
    (recognised by SQ_LDS_IDX_ACTIVE) is summarised instead as: LDS busy
    (rocprofv3's LdsUtil expression: SQ_LDS_IDX_ACTIVE / n_cu / cycles),
    the shares of the wavefronts' lifetime (SQ_WAVE_CYCLES) spent waiting on
    a dependency or s_waitcnt/barrier (SQ_WAIT_ANY), waiting to issue
    (SQ_WAIT_INST_ANY) and waiting to issue an LDS instruction
    (SQ_WAIT_INST_LDS), all in the same quad-cycle unit, and the cycles the
    LDS data FIFO was full per CU."""
    import collections
    import csv
    import glob

    files = glob.glob(os.path.join(prof_dir, "*counter_collection.csv"))
    if not files:
        raise SystemExit(f"no *counter_collection.csv under {prof_dir}")
    disp = collections.defaultdict(lambda: collections.defaultdict(dict))
    with open(files[0]) as fh:
        for r in csv.DictReader(fh):
            d = disp[r["Kernel_Name"]][r["Dispatch_Id"]]
            d[r["Counter_Name"]] = d.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
            d["_ns"] = float(r["End_Timestamp"]) - float(r["Start_Timestamp"])
    if any("SQ_LDS_IDX_ACTIVE" in d for ds in disp.values() for d in ds.values()):
        print("| kernel | entry point | dispatches | µs | clock GHz | LDS busy % | wave cycles / wave | waiting % | "
              "waiting to issue % | waiting to issue LDS % | LDS data FIFO full cycles / CU |")
        print("|---|---|---|---|---|---|---|---|---|---|---|")
        for name, ds in disp.items():
            call = _call_of(name)
            if call is None:
                continue
            n = len(ds)
            avg = {k: sum(d.get(k, 0.0) for d in ds.values()) / n for k in ("_ns",) + LDS_WAIT_COUNTERS}
            cyc = avg["GRBM_GUI_ACTIVE"] / n_xcd
            waves = max(avg["SQ_WAVES"], 1.0)
            wc = max(avg["SQ_WAVE_CYCLES"], 1.0)
            lds_busy = 100.0 * avg["SQ_LDS_IDX_ACTIVE"] / n_cu / cyc if cyc else 0.0
            print(f"| `{name}` | {call} | {n} | {avg['_ns'] / 1e3:.1f} | {cyc / avg['_ns']:.2f} | {lds_busy:.1f} | "
                  f"{4 * wc / waves:.0f} | {100 * avg['SQ_WAIT_ANY'] / wc:.1f} | "
                  f"{100 * avg['SQ_WAIT_INST_ANY'] / wc:.1f} | {100 * avg['SQ_WAIT_INST_LDS'] / wc:.1f} | "
                  f"{avg['SQ_LDS_DATA_FIFO_FULL'] / n_cu:.0f} |")
        return
    print("| kernel | entry point | dispatches | µs | clock GHz | MFMA busy % | VALU busy % | co-exec % of MFMA "
          "busy | VALU instr / wave | MFMA instr / wave | VALU / MFMA | LDS instr / wave | LDS bank-conflict "
          "cycles |")
    print("|---|---|---|---|---|---|---|---|---|---|---|---|---|")
    for name, ds in disp.items():
        call = _call_of(name)
        if call is None:
            continue
        n = len(ds)
        avg = {k: sum(d.get(k, 0.0) for d in ds.values()) / n for k in ("_ns",) + SQ_COUNTERS}
        cyc = avg["GRBM_GUI_ACTIVE"] / n_xcd
        waves = max(avg["SQ_WAVES"], 1.0)
        mfma_busy = 100.0 * avg["SQ_VALU_MFMA_BUSY_CYCLES"] / (cyc * n_simd) if cyc else 0.0
        valu_busy = 100.0 * avg["SQ_ACTIVE_INST_VALU"] / n_cu / cyc if cyc else 0.0
        coexec = (100.0 * avg["SQ_VALU_MFMA_COEXEC_CYCLES"] / avg["SQ_VALU_MFMA_BUSY_CYCLES"]
                  if avg["SQ_VALU_MFMA_BUSY_CYCLES"] else float("nan"))
        v_per_m = avg["SQ_INSTS_VALU"] / avg["SQ_INSTS_MFMA"] if avg["SQ_INSTS_MFMA"] else float("nan")
        print(f"| `{name}` | {call} | {n} | {avg['_ns'] / 1e3:.1f} | {cyc / avg['_ns']:.2f} | {mfma_busy:.1f} | "
              f"{valu_busy:.1f} | {coexec:.1f} | {avg['SQ_INSTS_VALU'] / waves:.0f} | "
              f"{avg['SQ_INSTS_MFMA'] / waves:.0f} | {v_per_m:.2f} | {avg['SQ_INSTS_LDS'] / waves:.0f} | "
              f"{avg['SQ_LDS_BANK_CONFLICT']:.0f} |")


def profile_record(call, path=None):
    """The recorded profile of entry point `call` (kernel durations and HBM
    bytes per launch), or None when the kernel sources have changed since
    the profile was taken."""
    path = path or PROFILE_JSON
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        rec = json.load(fh)
    if rec.get("kernel_sources_sha256") != csrc_sha256() or call not in rec:
        return None
    return rec[call]


def copy_calibration(mib):
    """dst.copy_(src) of `mib` MiB, three times: reads and writes exactly that
    many bytes per launch."""
    import torch
    src = torch.ones(mib << 18, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": mib << 20}), flush=True)


# ---------------------------------------------------------------- main

def main():
    args = parse()
    if args.poll_clock is not None:
        return poll_clock_main(args.poll_clock)
    if args.summarize_profiles:
        return summarize_profiles(args.summarize_profiles, args.calibration_mib, args.profile_out)
    if args.summarize_pmc:
        return summarize_pmc(args.summarize_pmc)
    if args.machine_limits:
        from tests.hw import machine_limits
        print(machine_limits.markdown(machine_limits.run()))
        return 0
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: --gpus {args.gpus} is not supported "
              "(the attention path runs on one GPU)", file=sys.stderr)
        sys.exit(2)
    extra = args.fp8 or args.persistent or args.sweep or args.workload or args.varlen
    # The clock poller is a child process, started before this process
    # touches the GPU.
    poller = None if (args.no_clock or extra) else ClockPoller()
    try:
        run(args, poller)
    finally:
        if poller is not None:
            poller.stop()


def run(args, poller):
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    binding.load_library()

    if args.fp8:
        return bench_fp8(args)
    if args.persistent:
        return bench_persistent(args)
    if args.sweep:
        return bench_sweep(args)
    if args.workload:
        return bench_one(args)
    if args.varlen:
        return bench_varlen(args)

    w = WORKLOADS[STEP_WORKLOAD]
    B, H, Hkv, N, d = w.batch, w.n_q_heads, w.n_kv_heads, w.seqlen, w.head_dim
    inp, q, k, v, do = device_inputs(w, with_do=True)
    step = Step(w, q, k, v, do)
    per_step, per_call, wall = time_calls(step, [step.fwd, step.bwd], args.steps, args.warmup)
    clock = None
    if poller is not None:
        t0, t1 = run_for([step.fwd, step.bwd], args.clock_window)
        clock = poller.window(t0 + 0.25 * args.clock_window, t1)
    ff = fwd_flops(B, H, N, N, d, w.causal)
    bf = bwd_flops(B, H, N, N, d, w.causal)
    tflops = (ff + bf) / (wall * 1e-3) / 1e12

    # Roofline of the call that takes the most time per step.
    avg_fwd, avg_bwd = float(np.mean(per_call[:, 0])), float(np.mean(per_call[:, 1]))
    if avg_bwd >= avg_fwd:
        dom = {"call": "fa_bwd", "kernel": "fa_bwd (bwd_dq_kernel forming D and dQ, then bwd_dkdv_kernel)",
               "flops": bf, "ms": avg_bwd, "bytes": bwd_bytes(B, H, Hkv, N, N, d)}
    else:
        dom = {"call": "fa_fwd", "kernel": "fa_fwd (fwd_kernel)", "flops": ff, "ms": avg_fwd,
               "bytes": fwd_bytes(B, H, Hkv, N, N, d)}
    prof = profile_record(dom["call"])
    traffic = prof["fetch_bytes"] + prof["write_bytes"] if prof and "fetch_bytes" in prof else None
    achieved = dom["flops"] / (dom["ms"] * 1e-3) / 1e12
    roofline = {"kernel": dom["kernel"], "bound": "mfma", "achieved": round(achieved, 2),
                "peak": MI355X_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": round(achieved / MI355X_BF16_PEAK_TFLOPS, 4), "traffic": traffic,
                "traffic_unit": "HBM bytes per launch (rocprofv3 FETCH_SIZE + WRITE_SIZE, copy-calibrated)",
                "algorithmic_bytes": dom["bytes"], "algorithmic_flops": dom["flops"],
                "avg_launch_ms": round(dom["ms"], 4),
                "profiled_avg_launch_ms": round(prof["kernel_avg_us"] / 1e3, 4) if prof else None}
    if clock:
        roofline["peak_at_clock"] = round(peak_at_clock(clock["median"]), 1)
        roofline["frac_at_clock"] = round(achieved / roofline["peak_at_clock"], 4)

    out = {
        "metric": METRIC,
        "value": round(tflops, 2),
        "unit": "TFLOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "backward config B4 H16 N4096 d128 causal bf16 (seed 5): fa_fwd producing O and L, "
                               "then fa_bwd",
                   "batch": B, "n_q_heads": H, "n_kv_heads": Hkv, "seqlen": N, "head_dim": d,
                   "causal": w.causal, "parallelism": "single GPU"},
        "pct_of_bf16_peak": round(100 * tflops / MI355X_BF16_PEAK_TFLOPS, 2),
        "ms_per_step_events_median": round(float(np.median(per_step)), 4),
        "gpu_clock_mhz": clock,
        "gpu_clock_source": "amd-smi metric -g 0 --clock (mean of the 8 XCD shader clocks), sampled every 0.1 s "
                            f"over {args.clock_window:.1f} s of back-to-back steps after the timed region, the "
                            "first quarter dropped",
        "fwd": time_stats(per_call[:, 0], ff, fwd_bytes(B, H, Hkv, N, N, d), clock),
        "bwd": time_stats(per_call[:, 1], bf, bwd_bytes(B, H, Hkv, N, N, d), clock),
        "caches": CACHE_NOTE,
        "roofline": roofline,
    }
    if clock:
        out["pct_of_bf16_peak_at_clock"] = round(100 * tflops / peak_at_clock(clock["median"]), 2)
    del step, q, k, v, do
    torch.cuda.empty_cache()

    cpu = {}
    if not args.no_cpu:
        tf, dt, n = cpu_oracle_sample(w, inp, CPU_SLICES[STEP_WORKLOAD], with_bwd=True)
        cpu[STEP_WORKLOAD] = {"value": round(tf, 5), "seconds": round(dt, 2), "slices": n}
    del inp

    if not args.no_configs:
        configs = {}
        for name in WORKLOAD_ORDER:
            cw = WORKLOADS[name]
            cinp, configs[name] = time_config(cw, args.config_calls, max(3, args.warmup // 2), poller,
                                              args.clock_window / 2)
            torch.cuda.empty_cache()
            if not args.no_cpu and name != STEP_WORKLOAD:
                tf, dt, n = cpu_oracle_sample(cw, cinp, CPU_SLICES[name], with_bwd=False)
                cpu[name] = {"value": round(tf, 5), "seconds": round(dt, 2), "slices": n, "pass": "forward"}
            del cinp
        out["configs"] = configs

        # fa_bwd_atomic (single pass, dQ by fp32 atomics) on the step's workload, as context.
        _, q, k, v, do = device_inputs(w, with_do=True)
        st = Step(w, q, k, v, do)
        st.fwd()
        per_a, _, _ = time_calls(st, [st.bwd_atomic], args.config_calls, 3)
        out["bwd_atomic_dq"] = time_stats(per_a, bf, bwd_bytes(B, H, Hkv, N, N, d), clock)
        out["bwd_atomic_dq"]["note"] = "fa_bwd_atomic on the step's workload (not in the timed step)"
        del st, q, k, v, do
        torch.cuda.empty_cache()

    if not args.no_cpu:
        host = host_description()
        s = cpu[STEP_WORKLOAD]
        out["cpu_baseline"] = {
            "value": s["value"], "unit": "TFLOPS", "cores": host["blas_threads"], "kind": "oracle",
            "sample": f"fp64 oracle forward+backward of {s['slices']} of {B * H} (batch, head) slices of the step's "
                      f"workload (N={N}, d={d}, causal), {s['seconds']:.1f} s wall, same causal-adjusted flop count; "
                      "BLAS calls run on the threads counted in cores, the elementwise work on one",
            **host,
            "per_config": {k2: v2 for k2, v2 in cpu.items() if k2 != STEP_WORKLOAD},
        }
    print(json.dumps(out), flush=True)
    if args.copy_calibration:
        copy_calibration(args.copy_calibration)


if __name__ == "__main__":
    main()
