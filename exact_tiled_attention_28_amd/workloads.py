"""The attention workloads this library is measured and checked on, plus the
algorithmic work (FLOPs and HBM bytes) each one must do.

FLOP count: a visible (query, key) pair costs 4*d multiply-add flops in the
forward pass (two dense contractions of length d: Q K^T and P V; the
FlashAttention-3 news page notes that at head dim 128 the matmul flops are
512 times the exponentials). Causal attention is counted as half the square.
The backward pass does five contractions per pair (the recomputed S = Q K^T,
then dV, dP, dQ and dK; the CSDN FlashAttention-2 page, backward equations)
instead of two, so it is counted as 2.5 times the forward.

HBM bytes are the minimum the method has to move: every input read once and
every output written once (no N^2 traffic).
"""

from __future__ import annotations

from dataclasses import dataclass
import math

import numpy as np

# Dense bf16 MFMA peak of one MI355X: 256 CUs x 4096 flop/clk/CU x 2.4 GHz.
MI355X_BF16_PEAK_TFLOPS = 2516.58
# Dense fp32 MFMA peak of one MI355X.
MI355X_F32_MFMA_PEAK_TFLOPS = 157.3
# HBM3E bandwidth of one MI355X.
MI355X_HBM_GBPS = 8000.0


@dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    n_q_heads: int
    n_kv_heads: int
    seqlen: int
    head_dim: int
    causal: bool
    dtype: str  # "bf16" or "f32"
    passes: str  # "fwd" or "bwd"
    seed: int
    n_outlier_channels: int = 0
    outlier_factor: float = 20.0

    @property
    def scale(self) -> float:
        """The float32 softmax scale 1/sqrt(d), as the kernels receive it."""
        return float(np.float32(1.0 / math.sqrt(self.head_dim)))

    @property
    def group(self) -> int:
        return self.n_q_heads // self.n_kv_heads


WORKLOADS = {
    w.name: w
    for w in [
        Workload("fwd_f32_b1_h1_n128_d64", 1, 1, 1, 128, 64, False, "f32", "fwd", 1),
        Workload("fwd_bf16_causal_b8_h16_n2048_d128", 8, 16, 16, 2048, 128, True, "bf16", "fwd", 2),
        Workload("fwd_bf16_causal_b1_h8_n16384_d128", 1, 8, 8, 16384, 128, True, "bf16", "fwd", 3),
        Workload("fwd_bf16_causal_gqa_b4_hq32_hkv8_n4096_d128_outliers", 4, 32, 8, 4096, 128, True,
                 "bf16", "fwd", 4, n_outlier_channels=2),
        Workload("bwd_bf16_causal_b4_h16_n4096_d128", 4, 16, 16, 4096, 128, True, "bf16", "bwd", 5),
    ]
}
WORKLOAD_ORDER = list(WORKLOADS)


def fwd_flops(batch, n_q_heads, seqlen_q, seqlen_k, head_dim, causal) -> float:
    """Forward flops: 4*d per visible pair, causal counted as half the square."""
    f = 4.0 * batch * n_q_heads * seqlen_q * seqlen_k * head_dim
    return f * 0.5 if causal else f


def bwd_flops(batch, n_q_heads, seqlen_q, seqlen_k, head_dim, causal) -> float:
    """Backward flops: five contractions per pair instead of two (x2.5)."""
    return 2.5 * fwd_flops(batch, n_q_heads, seqlen_q, seqlen_k, head_dim, causal)


def fwd_bytes(batch, n_q_heads, n_kv_heads, seqlen_q, seqlen_k, head_dim, in_bytes=2, out_bytes=2) -> int:
    """Minimum forward HBM traffic: read Q, K, V once; write O and fp32 L once."""
    q = batch * n_q_heads * seqlen_q * head_dim
    kv = batch * n_kv_heads * seqlen_k * head_dim
    return in_bytes * (q + 2 * kv) + out_bytes * q + 4 * batch * n_q_heads * seqlen_q


def bwd_bytes(batch, n_q_heads, n_kv_heads, seqlen_q, seqlen_k, head_dim, in_bytes=2, grad_bytes=2) -> int:
    """Minimum backward HBM traffic: read Q, K, V, O, dO, L once; write and
    read D once; write fp32 dQ and dK, dV once."""
    q = batch * n_q_heads * seqlen_q * head_dim
    kv = batch * n_kv_heads * seqlen_k * head_dim
    rows = batch * n_q_heads * seqlen_q
    return (in_bytes * (3 * q + 2 * kv) + 4 * rows + 2 * 4 * rows
            + 4 * q + grad_bytes * 2 * kv)


def workload_flops(w: Workload) -> float:
    f = bwd_flops if w.passes == "bwd" else fwd_flops
    return f(w.batch, w.n_q_heads, w.seqlen, w.seqlen, w.head_dim, w.causal)


def workload_bytes(w: Workload) -> int:
    eb = 4 if w.dtype == "f32" else 2
    if w.passes == "bwd":
        return bwd_bytes(w.batch, w.n_q_heads, w.n_kv_heads, w.seqlen, w.seqlen, w.head_dim, eb, eb)
    return fwd_bytes(w.batch, w.n_q_heads, w.n_kv_heads, w.seqlen, w.seqlen, w.head_dim, eb, eb)
