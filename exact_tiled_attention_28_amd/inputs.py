"""Seeded synthetic inputs for the attention workloads.

This module only draws random numbers and rounds them to bfloat16; it holds
none of the attention arithmetic, so both the HIP path and the CPU oracle can
take their inputs from it without sharing any of the method.

Recipe (the same for every workload):

* ``numpy.random.default_rng(seed)`` (PCG64);
* float32 standard normal draws, in the order Q, K, V, then dO when the
  workload has a backward pass, then (for the outlier workload) the outlier
  channel indices, drawn without replacement;
* outlier channels of Q and K are multiplied by the outlier factor in float32
  before rounding (the FlashAttention-3 news page, section on FP8 and
  incoherent processing, simulates activation outliers with a few
  large-magnitude entries in N(0,1) data);
* bfloat16 workloads round every float32 value once, round-to-nearest-even.

Layouts are row-major: Q, dO are [B, Hq, Nq, d]; K, V are [B, Hkv, Nk, d].

Packed variable-length batches (``make_varlen_inputs``) draw Q, K, V, dO the
same way with shapes [Hq, total_q, d] / [Hkv, total_k, d], where sequence b
owns rows cu[b]..cu[b+1]-1 and cu is the running sum of the given lengths.
"""

from __future__ import annotations

from dataclasses import dataclass

import numpy as np


def round_to_bf16(x: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """Round float32 values to bfloat16, round-to-nearest-even.

    Returns ``(values, bits)``: ``values`` is float32 holding exactly the
    bfloat16 numbers, ``bits`` the uint16 bfloat16 encodings. Inputs are
    finite (standard normal draws), so NaN handling is not needed here.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    r = (u + bias) & np.uint32(0xFFFF0000)
    return r.view(np.float32), (r >> np.uint32(16)).astype(np.uint16)


@dataclass
class AttentionInputs:
    """Host copies of one workload's inputs.

    ``q``, ``k``, ``v``, ``do`` are float32 arrays holding the exact input
    values (bfloat16-representable for bf16 workloads). ``*_bits`` hold the
    uint16 bfloat16 encodings for bf16 workloads and are ``None`` for fp32.
    """

    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    do: np.ndarray | None
    dtype: str
    q_bits: np.ndarray | None = None
    k_bits: np.ndarray | None = None
    v_bits: np.ndarray | None = None
    do_bits: np.ndarray | None = None
    outlier_channels: np.ndarray | None = None


def make_inputs(
    seed: int,
    batch: int,
    n_q_heads: int,
    n_kv_heads: int,
    seqlen_q: int,
    seqlen_k: int,
    head_dim: int,
    dtype: str = "bf16",
    with_do: bool = False,
    n_outlier_channels: int = 0,
    outlier_factor: float = 20.0,
) -> AttentionInputs:
    """Draw one workload's inputs following the recipe in the module doc."""
    if dtype not in ("bf16", "f32"):
        raise ValueError(f"dtype must be 'bf16' or 'f32', got {dtype!r}")
    rng = np.random.default_rng(seed)
    qs = (batch, n_q_heads, seqlen_q, head_dim)
    ks = (batch, n_kv_heads, seqlen_k, head_dim)
    q = rng.standard_normal(qs, dtype=np.float32)
    k = rng.standard_normal(ks, dtype=np.float32)
    v = rng.standard_normal(ks, dtype=np.float32)
    do = rng.standard_normal(qs, dtype=np.float32) if with_do else None
    channels = None
    if n_outlier_channels:
        channels = np.sort(rng.choice(head_dim, size=n_outlier_channels, replace=False))
        f = np.float32(outlier_factor)
        q[..., channels] *= f
        k[..., channels] *= f
    if dtype == "f32":
        return AttentionInputs(q, k, v, do, dtype, outlier_channels=channels)
    qv, qb = round_to_bf16(q)
    kv, kb = round_to_bf16(k)
    vv, vb = round_to_bf16(v)
    if do is not None:
        dov, dob = round_to_bf16(do)
    else:
        dov, dob = None, None
    return AttentionInputs(qv, kv, vv, dov, dtype, qb, kb, vb, dob, channels)


@dataclass
class VarlenInputs:
    """Host copies of a packed variable-length batch: ``q``, ``do``
    [Hq, total_q, d], ``k``, ``v`` [Hkv, total_k, d] (float32 holding
    bfloat16 values), the int32 offsets ``cu_q``, ``cu_k`` [batch + 1] and the
    longest lengths."""

    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    do: np.ndarray | None
    cu_q: np.ndarray
    cu_k: np.ndarray
    max_q: int
    max_k: int


def make_varlen_inputs(seed: int, lengths_q, lengths_k, n_q_heads: int, n_kv_heads: int, head_dim: int,
                       with_do: bool = False) -> VarlenInputs:
    """Draw a packed batch with the given per-sequence lengths (bf16 values)."""
    lq = np.asarray(lengths_q, dtype=np.int64)
    lk = np.asarray(lengths_k, dtype=np.int64)
    if lq.shape != lk.shape or lq.ndim != 1 or np.any(lq < 0) or np.any(lk < 0):
        raise ValueError("lengths must be two equal-size lists of non-negative integers")
    cu_q = np.concatenate([[0], np.cumsum(lq)]).astype(np.int32)
    cu_k = np.concatenate([[0], np.cumsum(lk)]).astype(np.int32)
    rng = np.random.default_rng(seed)
    tq, tk = int(cu_q[-1]), int(cu_k[-1])
    q = rng.standard_normal((n_q_heads, tq, head_dim), dtype=np.float32)
    k = rng.standard_normal((n_kv_heads, tk, head_dim), dtype=np.float32)
    v = rng.standard_normal((n_kv_heads, tk, head_dim), dtype=np.float32)
    do = rng.standard_normal((n_q_heads, tq, head_dim), dtype=np.float32) if with_do else None
    q, k, v = round_to_bf16(q)[0], round_to_bf16(k)[0], round_to_bf16(v)[0]
    if do is not None:
        do = round_to_bf16(do)[0]
    return VarlenInputs(q, k, v, do, cu_q, cu_k, int(lq.max(initial=0)), int(lk.max(initial=0)))


def make_signs(seed: int, head_dim: int) -> np.ndarray:
    """Random +1/-1 per channel (int8 [head_dim]) for the random-sign Hadamard
    transform of the FP8 path, drawn once and passed to both sides."""
    rng = np.random.default_rng(seed)
    return np.where(rng.random(head_dim) < 0.5, -1, 1).astype(np.int8)
