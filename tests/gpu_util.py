"""Helpers for the GPU tests: upload seeded inputs, run the library, compare
with the oracle."""

from __future__ import annotations

import sys

import numpy as np

from exact_tiled_attention_28_amd.inputs import make_inputs


def announce(msg: str) -> None:
    """Name the case before a GPU step, flushed, so a fault names it."""
    sys.stdout.write(f"\n[case] {msg}\n")
    sys.stdout.flush()


def to_device(x, bits, dtype):
    import torch
    if dtype == "bf16":
        return torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).cuda()


def upload(inp):
    q = to_device(inp.q, inp.q_bits, inp.dtype)
    k = to_device(inp.k, inp.k_bits, inp.dtype)
    v = to_device(inp.v, inp.v_bits, inp.dtype)
    do = to_device(inp.do, inp.do_bits, inp.dtype) if inp.do is not None else None
    return q, k, v, do


def host(t):
    import torch
    return t.detach().float().cpu().numpy().astype(np.float64) if t.dtype != torch.float32 \
        else t.detach().cpu().numpy().astype(np.float64)


def gen(seed, B, Hq, Hkv, Nq, Nk, d, dtype="bf16", with_do=False, outliers=0):
    return make_inputs(seed, B, Hq, Hkv, Nq, Nk, d, dtype, with_do=with_do, n_outlier_channels=outliers)


def bf16_half_ulp(x):
    """Half a bfloat16 ulp at |x| (for bf16-rounded outputs)."""
    ax = np.maximum(np.abs(x), np.finfo(np.float32).tiny)
    e = np.floor(np.log2(ax))
    return 2.0 ** (e - 8)
