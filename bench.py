#!/usr/bin/env python3
"""Benchmark of the attention hot path on one MI355X.

One step = one pass of the whole hot path over one batch of synthetic input:
fa_fwd (bf16 O, fp32 L) followed by fa_bwd (D preprocess, dK/dV kernel,
dQ kernel; fp32 dQ, bf16 dK/dV) on the causal bf16 workload B=8, H=16, N=2048, d=128
(seed 2), inputs resident in HBM. Prints ONE JSON line.

value = causal-adjusted TFLOPS of the step: forward 4*B*H*N^2*d/2 plus
backward 2.5x that, divided by the step time. Forward and backward TFLOPS
and their fractions of the dense bf16 MFMA peak are reported separately.

`roofline` covers the call that takes the most time per step, timed with HIP
events recorded on the stream the library launches on. `cpu_baseline` times
the fp64 CPU oracle (forward + backward) on a bounded sample of the same
workload: a few (batch, head) slices.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu]
       python bench.py --workload NAME   (one of the named workloads, extra)
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
# Copy-calibrated HBM bytes per launch of the step's calls, written by
# --summarize-profiles from rocprofv3 FETCH_SIZE / WRITE_SIZE runs.
TRAFFIC_JSON = os.path.join(ROOT, "profiles", "fa_step_b8_h16_n2048_d128_hbm_bytes.json")
sys.path.insert(0, ROOT)

from exact_tiled_attention_28_amd import binding  # noqa: E402
from exact_tiled_attention_28_amd.inputs import make_inputs  # noqa: E402
from exact_tiled_attention_28_amd.workloads import (  # noqa: E402
    MI355X_BF16_PEAK_TFLOPS, MI355X_HBM_GBPS, WORKLOADS, bwd_bytes, bwd_flops, fwd_bytes, fwd_flops)

METRIC = "attention fwd/bwd TFLOPS (causal-adjusted) and % of MI355X bf16 MFMA peak"
STEP_WORKLOAD = "fwd_bf16_causal_b8_h16_n2048_d128"


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=30)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    p.add_argument("--no-others", action="store_true",
                   help="skip timing the other named workloads after the step (profiled runs of the step use this)")
    p.add_argument("--cpu-heads", type=int, default=128, help="(batch, head) slices timed on the CPU oracle")
    p.add_argument("--workload", default=None, help="time one named workload (fwd or bwd only)")
    p.add_argument("--varlen", action="store_true", help="time fa_fwd_varlen + fa_bwd_varlen on a packed batch")
    p.add_argument("--sweep", action="store_true",
                   help="fa_fwd / fa_bwd throughput over head dim 64/128, N 1K-32K, causal and not, MHA and GQA")
    p.add_argument("--persistent", action="store_true",
                   help="time fa_fwd_persistent beside fa_fwd (default forward workload, or --workload)")
    p.add_argument("--fp8", action="store_true",
                   help="time fa_quantize_fp8 (Q and K) + fa_fwd_fp8 beside fa_fwd (default workload, or --workload)")
    p.add_argument("--summarize-profiles", default=None, metavar="DIR",
                   help="summarise rocprofv3 output under DIR/{trace,fetch,write} (no GPU needed) and record "
                        "the HBM bytes per launch for the current kernel sources")
    p.add_argument("--summarize-pmc", default=None, metavar="DIR",
                   help="summarise a rocprofv3 --pmc run of SQ_WAVES SQ_INSTS_VALU SQ_INSTS_MFMA SQ_INSTS_LDS "
                        "SQ_VALU_MFMA_BUSY_CYCLES SQ_LDS_BANK_CONFLICT GRBM_GUI_ACTIVE under DIR (no GPU needed)")
    p.add_argument("--calibration-mib", type=int, default=256, help="copy size used by the counter runs")
    p.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                   help="after the run, copy a MIB-MiB buffer 3 times (a plain copy kernel of known size, to "
                        "scale the HBM byte counters of a profiler run)")
    return p.parse_args()


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
    per-call times (ms) from HIP events recorded on the launch stream."""
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


# Packed variable-length batch timed by --varlen: 16 causal sequences whose
# lengths are drawn uniformly from [256, 4096] (seed 11), Hq = Hkv = 16,
# d = 128, bf16 (a mix like the unequal-length batches the FlashAttention-3
# news page names; no dataset is involved).
VARLEN_SEED, VARLEN_SEQS, VARLEN_MIN, VARLEN_MAX, VARLEN_H, VARLEN_D = 11, 16, 256, 4096, 16, 128


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
    head dim 64/128, N = 1K..32K, causal and non-causal, MHA and GQA (G = 4),
    with B = max(1, 16384 / N) and Hq = 2048 / d: N(0, 1) bf16 inputs drawn on
    the GPU from a seeded generator. One JSON line per shape (median of
    --steps timed calls after --warmup), then a summary line."""
    import torch
    rows = []
    for d in (64, 128):
        for n in (1024, 2048, 4096, 8192, 16384, 32768):
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
                    rows.append(row)
                    print(json.dumps(row), flush=True)
                    del q, k, v, do, o, lse, dq, dk, dv, ws
    best = max(rows, key=lambda r: r["fwd_tflops"] if r["causal"] and r["d"] == 128 else 0)
    print(json.dumps({"sweep_shapes": len(rows), "best_causal_d128_fwd": best}), flush=True)


def bench_persistent(args):
    """Time fa_fwd_persistent (work-queue grid) and fa_fwd (one workgroup per
    item) on the same forward workload; prints one JSON line."""
    import torch
    w = WORKLOADS[args.workload or STEP_WORKLOAD]
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
    fa_fwd_fp8 (bf16 O), with fa_fwd on the same inputs beside it. Prints one
    JSON line. The roofline of fa_fwd_fp8 counts S = Q K^T at the fp8 peak
    and O = P V at the bf16 peak: half of the flops each."""
    import torch
    from exact_tiled_attention_28_amd.inputs import make_signs
    w = WORKLOADS[args.workload or STEP_WORKLOAD]
    if w.passes != "fwd" or w.head_dim != 128 or w.dtype != "bf16":
        raise SystemExit(f"--fp8 needs a bf16 forward workload with head_dim 128, not {w.name}")
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

    _, per_call, _ = time_calls(None, [quant_q, quant_k, fwd8, step.fwd], args.steps, args.warmup)
    med = [float(np.median(per_call[:, i])) for i in range(4)]
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
           "roofline": {"kernel": "fa_fwd_fp8 (fwd_fp8_kernel)", "bound": "mfma", "achieved": round(ach, 2),
                        "peak": round(peak_mixed, 1), "unit": "TFLOP/s", "frac": round(ach / peak_mixed, 4),
                        "peak_note": "half the flops (Q K^T) at the 5.0 PFLOP/s fp8 peak, half (P V) at the "
                                     "2.5166 PFLOP/s bf16 peak", "avg_launch_ms": round(avg8, 4)}}
    print(json.dumps(out), flush=True)


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
    "fa_bwd": ("void fa::bwd_dkdv_kernel<", "void fa::bwd_dq_kernel<"),
    "fa_bwd_atomic": ("void fa::bwd_kernel<",),
    "fa_quantize_fp8": ("void fa::quantize_fp8_kernel<",),
    "fa_fwd_fp8": ("void fa::fwd_fp8_kernel<",),
}


def _template_args(kernel):
    """Template arguments of a demangled kernel name, as strings."""
    if "<" not in kernel or ">(" not in kernel:
        return []
    return [t.strip() for t in kernel[kernel.index("<") + 1:kernel.rindex(">(")].split(",")]


# Position of the VARLEN / PERSIST template argument of each kernel template
# (fwd_kernel<F32IN, D, CAUSAL, OUTF32, NW, VARLEN, PERSIST>,
# bwd_dkdv_kernel<D, CAUSAL, GF32, VARLEN>, bwd_dq_kernel<D, CAUSAL, VARLEN, NW>).
_VARLEN_ARG = {
    "void fa::fwd_kernel<": 5,
    "void fa::bwd_dkdv_kernel<": 3,
    "void fa::bwd_dq_kernel<": 2,
}
_PERSIST_ARG = {"void fa::fwd_kernel<": 6}


def _call_of(kernel):
    t = _template_args(kernel)
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


def summarize_profiles(prof_dir, calib_mib, out_path=None):
    """Turn the rocprofv3 output of one kernel-trace run (prof_dir/trace) and
    two counter runs (prof_dir/fetch: FETCH_SIZE, prof_dir/write: WRITE_SIZE,
    each with --copy-calibration calib_mib) into markdown tables, and record
    the copy-calibrated HBM bytes per launch of fa_fwd / fa_bwd for the
    current kernel sources in TRAFFIC_JSON."""
    import csv
    import glob

    def rows(sub, suffix):
        files = glob.glob(os.path.join(prof_dir, sub, "*" + suffix))
        if not files:
            raise SystemExit(f"no *{suffix} under {os.path.join(prof_dir, sub)}")
        with open(files[0]) as fh:
            return list(csv.DictReader(fh))

    stats = rows("trace", "kernel_stats.csv")
    total = sum(float(r["TotalDurationNs"]) for r in stats)
    print("| kernel | entry point | calls | average µs | min µs | max µs | share |")
    print("|---|---|---|---|---|---|---|")
    per_call_us = {}
    for r in stats:
        name = r["Name"]
        call = _call_of(name)
        avg = float(r["AverageNs"]) / 1e3
        print(f"| `{name}` | {call or '-'} | {r['Calls']} | {avg:.1f} | {float(r['MinNs']) / 1e3:.1f} | "
              f"{float(r['MaxNs']) / 1e3:.1f} | {100 * float(r['TotalDurationNs']) / total:.1f}% |")
        if call:
            per_call_us[call] = per_call_us.get(call, 0.0) + avg
    print()
    for call, us in sorted(per_call_us.items()):
        print(f"- `{call}`: sum of its kernels' average durations {us:.1f} µs")
    print()

    if not os.path.isdir(os.path.join(prof_dir, "fetch")):
        return  # a kernel-trace-only run
    counters = {}
    for sub, cname in (("fetch", "FETCH_SIZE"), ("write", "WRITE_SIZE")):
        acc = {}
        for r in rows(sub, "counter_collection.csv"):
            if r["Counter_Name"] != cname:
                continue
            k = acc.setdefault(r["Kernel_Name"], {})
            k[r["Dispatch_Id"]] = k.get(r["Dispatch_Id"], 0.0) + float(r["Counter_Value"])
        counters[cname] = {name: sum(v.values()) / len(v) for name, v in acc.items()}
    calib_kib = calib_mib * 1024
    scale = {}
    for cname, per in counters.items():
        copies = [v for name, v in per.items() if "copyBuffer" in name]
        if not copies:
            raise SystemExit(f"{cname}: no copy kernel in the counter run (run it with --copy-calibration)")
        scale[cname] = calib_kib / (sum(copies) / len(copies))
    print(f"Calibration: a copy of {calib_mib} MiB reads {calib_kib / scale['FETCH_SIZE']:.0f} KiB of FETCH_SIZE "
          f"(scale x{scale['FETCH_SIZE']:.4f}) and {calib_kib / scale['WRITE_SIZE']:.0f} KiB of WRITE_SIZE "
          f"(scale x{scale['WRITE_SIZE']:.4f}).")
    print()
    print("| kernel | entry point | FETCH_SIZE KiB | WRITE_SIZE KiB | HBM MB (scaled) |")
    print("|---|---|---|---|---|")
    per_call = {}
    names = sorted(set(counters["FETCH_SIZE"]) | set(counters["WRITE_SIZE"]))
    for name in names:
        call = _call_of(name)
        if call is None:
            continue
        f = counters["FETCH_SIZE"].get(name, 0.0)
        wr = counters["WRITE_SIZE"].get(name, 0.0)
        fb, wb = f * 1024 * scale["FETCH_SIZE"], wr * 1024 * scale["WRITE_SIZE"]
        print(f"| `{name}` | {call} | {f:.0f} | {wr:.0f} | {(fb + wb) / 1e6:.0f} |")
        c = per_call.setdefault(call, {"fetch_bytes": 0, "write_bytes": 0})
        c["fetch_bytes"] += int(round(fb))
        c["write_bytes"] += int(round(wb))
    print()
    for call, c in sorted(per_call.items()):
        print(f"- `{call}`: {(c['fetch_bytes'] + c['write_bytes']) / 1e6:.0f} MB per launch")
    rec = {"note": "HBM bytes per launch from rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE (KiB per dispatch), "
                   "scaled by the same counters on a copy of known size",
           "kernel_sources_sha256": csrc_sha256(), "workload": "fwd_bf16_causal_b8_h16_n2048_d128",
           "fetch_scale": round(scale["FETCH_SIZE"], 4), "write_scale": round(scale["WRITE_SIZE"], 4)}
    rec.update({k: v for k, v in per_call.items() if k in ("fa_fwd", "fa_bwd")})
    out_path = out_path or TRAFFIC_JSON
    with open(out_path, "w") as fh:
        json.dump(rec, fh, indent=1)
    print(f"\nkernel sources sha256 {rec['kernel_sources_sha256']}")


def summarize_pmc(prof_dir, n_xcd=8, n_simd=1024):
    """Per-kernel averages of one rocprofv3 --pmc run: clock (GRBM_GUI_ACTIVE,
    summed over the n_xcd XCD instances, over the dispatch's duration), MFMA
    utilisation (SQ_VALU_MFMA_BUSY_CYCLES over n_simd SIMDs x the kernel's
    cycles, the rocprofv3 MfmaUtil expression), instructions per wavefront,
    and LDS bank-conflict cycles."""
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
    print("| kernel | entry point | dispatches | µs | clock GHz | MFMA busy % | VALU instr / wave | "
          "MFMA instr / wave | VALU / MFMA | LDS instr / wave | LDS bank-conflict cycles |")
    print("|---|---|---|---|---|---|---|---|---|---|---|")
    for name, ds in disp.items():
        call = _call_of(name)
        if call is None:
            continue
        n = len(ds)
        avg = {k: sum(d.get(k, 0.0) for d in ds.values()) / n
               for k in ("_ns", "GRBM_GUI_ACTIVE", "SQ_VALU_MFMA_BUSY_CYCLES", "SQ_WAVES", "SQ_INSTS_VALU",
                         "SQ_INSTS_MFMA", "SQ_INSTS_LDS", "SQ_LDS_BANK_CONFLICT")}
        cyc = avg["GRBM_GUI_ACTIVE"] / n_xcd
        waves = max(avg["SQ_WAVES"], 1.0)
        mfma_busy = 100.0 * avg["SQ_VALU_MFMA_BUSY_CYCLES"] / (cyc * n_simd) if cyc else 0.0
        v_per_m = avg["SQ_INSTS_VALU"] / avg["SQ_INSTS_MFMA"] if avg["SQ_INSTS_MFMA"] else float("nan")
        print(f"| `{name}` | {call} | {n} | {avg['_ns'] / 1e3:.1f} | {cyc / avg['_ns']:.2f} | {mfma_busy:.1f} | "
              f"{avg['SQ_INSTS_VALU'] / waves:.0f} | {avg['SQ_INSTS_MFMA'] / waves:.0f} | {v_per_m:.2f} | "
              f"{avg['SQ_INSTS_LDS'] / waves:.0f} | {avg['SQ_LDS_BANK_CONFLICT']:.0f} |")


def measured_traffic(call):
    """HBM bytes per launch of `call` ("fa_fwd" / "fa_bwd") recorded from
    rocprofv3 FETCH_SIZE / WRITE_SIZE runs, or None when the kernel sources
    have changed since they were taken."""
    rec_path = TRAFFIC_JSON
    if not os.path.exists(rec_path):
        return None
    with open(rec_path) as fh:
        rec = json.load(fh)
    if rec.get("kernel_sources_sha256") != csrc_sha256() or call not in rec:
        return None
    return rec[call]["fetch_bytes"] + rec[call]["write_bytes"]


def cpu_baseline(w, inp, heads):
    """The fp64 oracle, untuned, on `heads` (batch, head) slices of the
    workload: forward + backward. Returns the JSON object."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"] or [1])
    except Exception:
        threads = len(os.sched_getaffinity(0))
    sel = [(b, h) for b in range(w.batch) for h in range(w.n_q_heads)][:heads]
    t0 = time.perf_counter()
    for b, h in sel:
        g = h // w.group
        oracle.forward_head(inp.q[b, h], inp.k[b, g], inp.v[b, g], w.scale, w.causal)
        oracle.backward_head(inp.q[b, h], inp.k[b, g], inp.v[b, g], inp.do[b, h], w.scale, w.causal)
    dt = time.perf_counter() - t0
    flops = heads * (fwd_flops(1, 1, w.seqlen, w.seqlen, w.head_dim, w.causal)
                     + bwd_flops(1, 1, w.seqlen, w.seqlen, w.head_dim, w.causal))
    return {"value": flops / dt / 1e12, "unit": "TFLOPS", "cores": int(threads), "kind": "oracle",
            "sample": f"fp64 oracle forward+backward of {heads} of {w.batch * w.n_q_heads} (batch, head) slices "
                      f"(N={w.seqlen}, d={w.head_dim}, causal), {dt:.1f} s wall, same causal-adjusted flop count"}


def main():
    args = parse()
    if args.summarize_profiles:
        return summarize_profiles(args.summarize_profiles, args.calibration_mib)
    if args.summarize_pmc:
        return summarize_pmc(args.summarize_pmc)
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: --gpus {args.gpus} is not supported "
              "(the attention path runs on one GPU)", file=sys.stderr)
        sys.exit(2)
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
    inp, q, k, v, do = device_inputs(w, with_do=True)
    if do is None:
        raise RuntimeError("dO missing")
    step = Step(w, q, k, v, do)
    per_step, per_call, wall = time_calls(step, [step.fwd, step.bwd], args.steps, args.warmup)
    _, per_call_atomic, _ = time_calls(step, [step.bwd_atomic], args.steps, args.warmup)
    ms_bwd_atomic = float(np.median(per_call_atomic[:, 0]))
    ms_step = float(np.median(per_step))
    ms_fwd = float(np.median(per_call[:, 0]))
    ms_bwd = float(np.median(per_call[:, 1]))
    ff = fwd_flops(w.batch, w.n_q_heads, w.seqlen, w.seqlen, w.head_dim, w.causal)
    bf = bwd_flops(w.batch, w.n_q_heads, w.seqlen, w.seqlen, w.head_dim, w.causal)
    tflops = (ff + bf) / (ms_step * 1e-3) / 1e12
    fwd_tf = ff / (ms_fwd * 1e-3) / 1e12
    bwd_tf = bf / (ms_bwd * 1e-3) / 1e12
    avg_fwd = float(np.mean(per_call[:, 0]))
    avg_bwd = float(np.mean(per_call[:, 1]))
    if avg_bwd >= avg_fwd:
        dom = {"kernel": "fa_bwd (bwd_dq_kernel with D + bwd_dkdv_kernel, one call)", "flops": bf,
               "ms": avg_bwd, "traffic": measured_traffic("fa_bwd")}
    else:
        dom = {"kernel": "fa_fwd (fwd_kernel)", "flops": ff, "ms": avg_fwd, "traffic": measured_traffic("fa_fwd")}
    achieved = dom["flops"] / (dom["ms"] * 1e-3) / 1e12
    out = {
        "metric": METRIC,
        "value": round(tflops, 2),
        "unit": "TFLOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "fa_fwd + fa_bwd, bf16, causal, B=8 Hq=Hkv=16 N=2048 d=128 (seed 2)",
                   "batch": w.batch, "n_q_heads": w.n_q_heads, "n_kv_heads": w.n_kv_heads,
                   "seqlen": w.seqlen, "head_dim": w.head_dim, "causal": w.causal, "parallelism": "single GPU"},
        "pct_of_bf16_peak": round(100 * tflops / MI355X_BF16_PEAK_TFLOPS, 2),
        "fwd": {"ms": round(ms_fwd, 4), "tflops": round(fwd_tf, 2),
                "pct_of_bf16_peak": round(100 * fwd_tf / MI355X_BF16_PEAK_TFLOPS, 2),
                "gbps_algorithmic": round(fwd_bytes(w.batch, w.n_q_heads, w.n_kv_heads, w.seqlen, w.seqlen,
                                                    w.head_dim) / (ms_fwd * 1e-3) / 1e9, 1)},
        "bwd": {"ms": round(ms_bwd, 4), "tflops": round(bwd_tf, 2),
                "pct_of_bf16_peak": round(100 * bwd_tf / MI355X_BF16_PEAK_TFLOPS, 2),
                "gbps_algorithmic": round(bwd_bytes(w.batch, w.n_q_heads, w.n_kv_heads, w.seqlen, w.seqlen,
                                                    w.head_dim) / (ms_bwd * 1e-3) / 1e9, 1)},
        "bwd_atomic_dq": {"ms": round(ms_bwd_atomic, 4),
                          "tflops": round(bf / (ms_bwd_atomic * 1e-3) / 1e12, 2),
                          "note": "fa_bwd_atomic: single pass, dQ by fp32 atomics (not in the timed step)"},
        "wall_ms_per_step": round(wall, 4),
        "roofline": {"kernel": dom["kernel"], "bound": "mfma", "achieved": round(achieved, 2),
                     "peak": MI355X_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / MI355X_BF16_PEAK_TFLOPS, 4), "traffic": dom["traffic"],
                     "traffic_unit": "bytes per launch (HBM, rocprofv3 FETCH_SIZE+WRITE_SIZE, copy-calibrated)",
                     "avg_launch_ms": round(dom["ms"], 4)},
    }
    # The other named workloads, each pass timed on its own after the step
    # (context for the same run; not part of value).
    if not args.no_others:
        out["other_workloads"] = {name: {k2: v2 for k2, v2 in time_workload(WORKLOADS[name], 10, 3).items()
                                         if k2 != "workload"}
                                  for name in WORKLOADS if name != STEP_WORKLOAD}
    if not args.no_cpu:
        out["cpu_baseline"] = cpu_baseline(w, inp, args.cpu_heads)
    print(json.dumps(out), flush=True)
    if args.copy_calibration:
        copy_calibration(args.copy_calibration)


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


def bench_one(args):
    """Time one named workload's pass (fwd or bwd); prints one JSON line."""
    print(json.dumps(time_workload(WORKLOADS[args.workload], args.steps, args.warmup)), flush=True)


def time_workload(w, steps, warmup):
    """Median time of one named workload's pass (fwd or bwd), as a dict."""
    inp, q, k, v, do = device_inputs(w, with_do=w.passes == "bwd")
    step = Step(w, q, k, v, do if do is not None else q)
    if w.passes == "bwd":
        step.fwd()
        calls, fl = [step.bwd], bwd_flops(w.batch, w.n_q_heads, w.seqlen, w.seqlen, w.head_dim, w.causal)
        by = bwd_bytes(w.batch, w.n_q_heads, w.n_kv_heads, w.seqlen, w.seqlen, w.head_dim)
    else:
        calls, fl = [step.fwd], fwd_flops(w.batch, w.n_q_heads, w.seqlen, w.seqlen, w.head_dim, w.causal)
        eb = 4 if w.dtype == "f32" else 2
        by = fwd_bytes(w.batch, w.n_q_heads, w.n_kv_heads, w.seqlen, w.seqlen, w.head_dim, eb, eb)
    per_step, _, _ = time_calls(step, calls, steps, warmup)
    ms = float(np.median(per_step))
    tf = fl / (ms * 1e-3) / 1e12
    return {"workload": w.name, "ms": round(ms, 4), "ms_min": round(float(per_step.min()), 4),
            "tflops": round(tf, 2), "pct_of_bf16_peak": round(100 * tf / MI355X_BF16_PEAK_TFLOPS, 2),
            "gbps_algorithmic": round(by / (ms * 1e-3) / 1e9, 1),
            "pct_of_hbm": round(100 * by / (ms * 1e-3) / 1e9 / MI355X_HBM_GBPS, 2)}


if __name__ == "__main__":
    main()
