"""Forward parity on the GPU: libfa.so (through the C ABI) against the fp64
oracle on the same seeded inputs.

Tolerances: max-abs 1e-2 on O and 1e-3 on L for bf16 inputs (O requested in
fp32 so the bound measures the kernel's arithmetic, not the final rounding);
bf16 O is checked against 1e-2 plus half a bf16 ulp of the exact value; the
fp32 path must match O within 1e-5.
"""

import math

import numpy as np
import pytest

import oracle
from exact_tiled_attention_28_amd import binding
from exact_tiled_attention_28_amd.workloads import WORKLOADS
from tests.gpu_util import announce, bf16_half_ulp, gen, host, upload

pytestmark = pytest.mark.gpu

O_TOL_BF16 = 1e-2
L_TOL_BF16 = 1e-3
O_TOL_F32 = 1e-5


def run_fwd(inp, scale, causal, out_f32=True):
    import torch
    q, k, v, _ = upload(inp)
    o, lse = binding.forward(q, k, v, scale, causal, out_dtype=torch.float32 if out_f32 else torch.bfloat16)
    torch.cuda.synchronize()
    return host(o), host(lse)


CASES = [
    # (B, Hq, Hkv, Nq, Nk, d, causal)
    (1, 1, 1, 1, 1, 64, False),
    (1, 1, 1, 1, 1, 128, True),
    (1, 2, 2, 17, 17, 64, True),
    (1, 2, 1, 127, 127, 128, True),
    (2, 2, 2, 129, 129, 128, False),
    (1, 4, 2, 300, 300, 64, True),
    (1, 4, 1, 257, 257, 128, True),
    (1, 2, 2, 100, 257, 128, False),
    (1, 2, 2, 333, 65, 64, False),
    (2, 8, 2, 512, 512, 128, True),
    (1, 1, 1, 1000, 1000, 128, True),
    # non-causal d=128 with 1 and 5 unmasked steps: the three-buffer main
    # loop leaves after phases 1 and 5 of its six
    (1, 2, 2, 64, 192, 128, False),
    (1, 2, 1, 200, 448, 128, False),
]


@pytest.mark.parametrize("case", CASES, ids=[f"B{c[0]}Hq{c[1]}Hkv{c[2]}Nq{c[3]}Nk{c[4]}d{c[5]}{'c' if c[6] else 'n'}" for c in CASES])
def test_fwd_bf16_parity(case):
    B, Hq, Hkv, Nq, Nk, d, causal = case
    announce(f"fwd bf16 {case}")
    inp = gen(100 + Nq + d, B, Hq, Hkv, Nq, Nk, d)
    scale = float(np.float32(1 / math.sqrt(d)))
    O, L = run_fwd(inp, scale, causal)
    Or, Lr = oracle.forward(inp.q, inp.k, inp.v, scale, causal)
    assert np.max(np.abs(O - Or)) <= O_TOL_BF16
    assert np.max(np.abs(L - Lr)) <= L_TOL_BF16


@pytest.mark.parametrize("case", CASES[:6], ids=[f"B{c[0]}Hq{c[1]}Hkv{c[2]}Nq{c[3]}Nk{c[4]}d{c[5]}{'c' if c[6] else 'n'}" for c in CASES[:6]])
def test_fwd_f32_parity(case):
    B, Hq, Hkv, Nq, Nk, d, causal = case
    announce(f"fwd f32 {case}")
    inp = gen(200 + Nq + d, B, Hq, Hkv, Nq, Nk, d, dtype="f32")
    scale = float(np.float32(1 / math.sqrt(d)))
    O, L = run_fwd(inp, scale, causal)
    Or, Lr = oracle.forward(inp.q, inp.k, inp.v, scale, causal)
    assert np.max(np.abs(O - Or)) <= O_TOL_F32
    assert np.max(np.abs(L - Lr)) <= O_TOL_F32


def test_fwd_f32_workload_b1_h1_n128_d64():
    w = WORKLOADS["fwd_f32_b1_h1_n128_d64"]
    announce(w.name)
    inp = gen(w.seed, w.batch, w.n_q_heads, w.n_kv_heads, w.seqlen, w.seqlen, w.head_dim, dtype="f32")
    O, L = run_fwd(inp, w.scale, w.causal)
    Or, Lr = oracle.forward(inp.q, inp.k, inp.v, w.scale, w.causal)
    assert np.max(np.abs(O - Or)) <= O_TOL_F32
    assert np.max(np.abs(L - Lr)) <= O_TOL_F32


def test_fwd_bf16_output_rounding():
    announce("fwd bf16 out")
    inp = gen(7, 1, 4, 4, 300, 300, 128)
    scale = float(np.float32(1 / math.sqrt(128)))
    O, L = run_fwd(inp, scale, True, out_f32=False)
    Or, Lr = oracle.forward(inp.q, inp.k, inp.v, scale, True)
    assert np.all(np.abs(O - Or) <= O_TOL_BF16 + bf16_half_ulp(Or))
    assert np.max(np.abs(L - Lr)) <= L_TOL_BF16


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("scale", [0.0, -0.2, 0.5])
def test_fwd_scale_edge_cases(scale, d):
    # A zero scale also checks the masked tiles' -inf scores under the
    # kernels' smallest-normal multiplier (probability 0, not NaN).
    announce(f"fwd scale {scale} d {d}")
    inp = gen(8, 1, 2, 2, 200, 200, d)
    for causal in (False, True):
        O, L = run_fwd(inp, scale, causal)
        Or, Lr = oracle.forward(inp.q, inp.k, inp.v, scale, causal)
        assert np.all(np.isfinite(O)) and np.all(np.isfinite(L))
        assert np.max(np.abs(O - Or)) <= O_TOL_BF16
        assert np.max(np.abs(L - Lr)) <= L_TOL_BF16


# Longer key sequences: the three-K-buffer main loop over many phases, ragged
# last tiles in both head dims, GQA and Nq != Nk (the 8-wavefront causal
# kernel at d = 128, from 16K keys, is covered by the long-sequence and
# workload tests).
LONG_CASES = [
    (1, 2, 1, 4097, 4097, 128, True),
    (1, 1, 1, 8300, 8300, 128, True),   # ragged last Q tile
    (1, 2, 2, 4500, 4500, 128, False),  # ragged
    (1, 2, 2, 4100, 4100, 64, True),
    (1, 2, 1, 333, 4200, 128, False),
    (1, 1, 1, 4096, 4096, 64, False),
    # 8-wavefront kernel without the causal mask (from 8192 keys): ragged
    # 256-row Q tiles and a ragged last K/V tile, MHA and GQA
    (1, 1, 1, 300, 8300, 128, False),
    (1, 4, 1, 520, 8200, 128, False),
    # the same kernel at d = 64: ragged Q tiles without the mask, and a
    # causal run from 16384 keys with a ragged last tile
    (1, 2, 1, 300, 8300, 64, False),
    (1, 1, 1, 16400, 16400, 64, True),
]


@pytest.mark.parametrize("case", LONG_CASES,
                         ids=[f"B{c[0]}Hq{c[1]}Hkv{c[2]}Nq{c[3]}Nk{c[4]}d{c[5]}{'c' if c[6] else 'n'}" for c in LONG_CASES])
def test_fwd_long_keys_parity(case):
    B, Hq, Hkv, Nq, Nk, d, causal = case
    announce(f"fwd bf16 long {case}")
    inp = gen(400 + Nq + d, B, Hq, Hkv, Nq, Nk, d)
    scale = float(np.float32(1 / math.sqrt(d)))
    O, L = run_fwd(inp, scale, causal)
    Or, Lr = oracle.forward(inp.q, inp.k, inp.v, scale, causal)
    assert np.max(np.abs(O - Or)) <= O_TOL_BF16
    assert np.max(np.abs(L - Lr)) <= L_TOL_BF16
