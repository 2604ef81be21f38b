"""Backward parity on the GPU: fa_bwd (through the C ABI) against the fp64
oracle's analytic gradients on the same seeded inputs, at the stated flat
bound: max-abs 1e-2 on dQ, dK and dV (bf16 dK, dV outputs: 1e-2 plus half a
bf16 ulp of the exact value).

The backward is fed O and L from fa_fwd with fp32 O (the backward's D is
rowsum(dO o O), so a bf16-rounded O would add its rounding to D; parity runs
request fp32 outputs from the same kernels; test_bwd_with_bf16_o covers the
bf16 O of the timed configuration).

Schemes: "bf16" is fa_bwd with FA_PRECISION_BF16 (P and dS rounded once to
bf16 before the gradient products, the 16-bit products of the pages), "hilo"
fa_bwd with FA_PRECISION_HILO (P and dS as bf16 pairs hi + lo), "atomic"
fa_bwd_atomic (bf16). The bf16 rounding of P alone moves dV by up to
2^-9 * sum_{h,i} P_hij |dO_hic|; where query heads are summed over a group on
short causal rows, that exceeds the flat bound (1.4e-2 on dV at G = 4,
N = 512), so those cases run with the hilo scheme only (BF16_OVER_BOUND).
"""

import math

import numpy as np
import pytest

import oracle
from exact_tiled_attention_28_amd import binding
from tests.gpu_util import announce, bf16_half_ulp, gen, host, upload

pytestmark = pytest.mark.gpu

TOL = 1e-2
SCHEMES = ["bf16", "hilo", "atomic"]


def run_fwd_bwd(inp, scale, causal, grad_f32=True, scheme="bf16"):
    import torch
    q, k, v, do = upload(inp)
    o, lse = binding.forward(q, k, v, scale, causal, out_dtype=torch.float32)
    dq, dk, dv, dvec = binding.backward(q, k, v, o, lse, do, scale, causal,
                                        grad_dtype=torch.float32 if grad_f32 else torch.bfloat16,
                                        atomic_dq=scheme == "atomic", hilo=scheme == "hilo")
    torch.cuda.synchronize()
    return host(o), host(lse), host(dq), host(dk), host(dv), host(dvec)


def check_flat(dQ, dK, dV, dQr, dKr, dVr, what, tol=TOL):
    e = (np.max(np.abs(dQ - dQr)), np.max(np.abs(dK - dKr)), np.max(np.abs(dV - dVr)))
    print(f"{what}: max|d dQ|={e[0]:.3e} max|d dK|={e[1]:.3e} max|d dV|={e[2]:.3e}")
    assert e[0] <= tol, "dQ"
    assert e[1] <= tol, "dK"
    assert e[2] <= tol, "dV"


CASES = [
    # (B, Hq, Hkv, Nq, Nk, d, causal)
    (1, 1, 1, 1, 1, 128, True),
    (1, 1, 1, 17, 17, 64, True),
    (1, 2, 2, 127, 127, 128, True),
    (1, 2, 1, 129, 129, 128, False),
    (2, 4, 2, 200, 200, 64, True),
    (1, 4, 1, 300, 300, 128, True),
    (1, 2, 2, 100, 257, 128, False),
    (1, 2, 2, 333, 65, 64, False),
    (1, 8, 2, 512, 512, 128, True),
    (1, 8, 1, 256, 256, 128, True),   # G = 8
    (1, 16, 2, 200, 200, 64, False),  # G = 8, d = 64, non-causal
]
# Grouped causal cases where the bf16 rounding of P and dS alone reaches the
# flat bound (a CPU simulation of that rounding: dV 9.9e-3 at G=4 N=300,
# 1.4e-2 at G=4 N=512; G=8 sums twice as many heads): hilo only.
BF16_OVER_BOUND = {(1, 4, 1, 300, 300, 128, True), (1, 8, 2, 512, 512, 128, True),
                   (1, 8, 1, 256, 256, 128, True)}
PARAMS = [(c, sc) for c in CASES for sc in SCHEMES if sc == "hilo" or c not in BF16_OVER_BOUND]


def _cid(c):
    return f"B{c[0]}Hq{c[1]}Hkv{c[2]}Nq{c[3]}Nk{c[4]}d{c[5]}{'c' if c[6] else 'n'}"


@pytest.mark.parametrize("case,scheme", PARAMS, ids=[f"{_cid(c)}-{sc}" for c, sc in PARAMS])
def test_bwd_parity(case, scheme):
    B, Hq, Hkv, Nq, Nk, d, causal = case
    announce(f"bwd {case} scheme={scheme}")
    inp = gen(300 + Nq + d, B, Hq, Hkv, Nq, Nk, d, with_do=True)
    scale = float(np.float32(1 / math.sqrt(d)))
    O, L, dQ, dK, dV, Dv = run_fwd_bwd(inp, scale, causal, scheme=scheme)
    dQr, dKr, dVr = oracle.backward(inp.q, inp.k, inp.v, inp.do, scale, causal)
    check_flat(dQ, dK, dV, dQr, dKr, dVr, f"{_cid(case)} {scheme}")
    # D = rowsum(dO o O) of the O the kernel was given.
    assert np.max(np.abs(Dv - oracle.row_dot(inp.do, O))) <= 1e-4
    # Sum rules: sum_j dK_j = 0, sum_j dV_j = group sum of sum_i dO_i.
    G = Hq // Hkv
    assert np.max(np.abs(dK.sum(axis=2))) <= 0.05
    ref = inp.do.astype(np.float64).reshape(B, Hkv, G, Nq, d).sum(axis=(2, 3))
    assert np.max(np.abs(dV.sum(axis=2) - ref)) <= 0.05 + 1e-3 * np.max(np.abs(ref))


# From 8192 keys the d = 128 dQ pass runs with 8 wavefronts (256-row Q
# tiles): a causal run with a ragged last Q tile, and ragged Q tiles without
# the mask (Nq = 300).
WIDE_DQ_CASES = [(1, 1, 1, 8300, 8300, 128, True), (1, 2, 1, 300, 8300, 128, False)]
WIDE_PARAMS = [(c, sc) for c in WIDE_DQ_CASES for sc in ("bf16", "hilo")]


@pytest.mark.parametrize("case,scheme", WIDE_PARAMS, ids=[f"{_cid(c)}-{sc}" for c, sc in WIDE_PARAMS])
def test_bwd_wide_dq_parity(case, scheme):
    B, Hq, Hkv, Nq, Nk, d, causal = case
    announce(f"bwd wide dQ {case} scheme={scheme}")
    inp = gen(500 + Nq + d, B, Hq, Hkv, Nq, Nk, d, with_do=True)
    scale = float(np.float32(1 / math.sqrt(d)))
    O, L, dQ, dK, dV, Dv = run_fwd_bwd(inp, scale, causal, scheme=scheme)
    dQr, dKr, dVr = oracle.backward(inp.q, inp.k, inp.v, inp.do, scale, causal)
    check_flat(dQ, dK, dV, dQr, dKr, dVr, f"{_cid(case)} {scheme}")
    assert np.max(np.abs(Dv - oracle.row_dot(inp.do, O))) <= 1e-4


# Causal d = 128 rows without query-head groups run the four-wavefront dK/dV
# kernel up to 1024 keys and the eight-wavefront one above: both sides of
# that switch, with a ragged last key block below it.
SHORT_ROW_CASES = [(1, 2, 2, 1023, 1023, 128, True), (1, 2, 2, 1024, 1024, 128, True),
                   (1, 2, 2, 1025, 1025, 128, True)]


@pytest.mark.parametrize("case", SHORT_ROW_CASES, ids=[_cid(c) for c in SHORT_ROW_CASES])
def test_bwd_short_row_dispatch_parity(case):
    B, Hq, Hkv, Nq, Nk, d, causal = case
    announce(f"bwd short-row dispatch {case}")
    inp = gen(700 + Nq, B, Hq, Hkv, Nq, Nk, d, with_do=True)
    scale = float(np.float32(1 / math.sqrt(d)))
    O, L, dQ, dK, dV, Dv = run_fwd_bwd(inp, scale, causal)
    dQr, dKr, dVr = oracle.backward(inp.q, inp.k, inp.v, inp.do, scale, causal)
    check_flat(dQ, dK, dV, dQr, dKr, dVr, _cid(case))


@pytest.mark.parametrize("scheme", SCHEMES)
def test_bwd_bf16_grads(scheme):
    announce(f"bwd bf16 grads scheme={scheme}")
    inp = gen(41, 1, 4, 2, 300, 300, 128, with_do=True)
    scale = float(np.float32(1 / math.sqrt(128)))
    _, _, dQ, dK, dV, _ = run_fwd_bwd(inp, scale, True, grad_f32=False, scheme=scheme)
    dQr, dKr, dVr = oracle.backward(inp.q, inp.k, inp.v, inp.do, scale, True)
    print(f"bf16 outputs {scheme}: max|d dQ|={np.max(np.abs(dQ - dQr)):.3e} "
          f"max|d dK|={np.max(np.abs(dK - dKr)):.3e} max|d dV|={np.max(np.abs(dV - dVr)):.3e}")
    assert np.max(np.abs(dQ - dQr)) <= TOL
    assert np.all(np.abs(dK - dKr) <= TOL + bf16_half_ulp(dKr))
    assert np.all(np.abs(dV - dVr) <= TOL + bf16_half_ulp(dVr))


@pytest.mark.parametrize("scheme", SCHEMES)
def test_bwd_zero_scale(scheme):
    announce(f"bwd scale 0 scheme={scheme}")
    inp = gen(42, 1, 2, 1, 150, 150, 64, with_do=True)
    for causal in (False, True):
        _, _, dQ, dK, dV, _ = run_fwd_bwd(inp, 0.0, causal, scheme=scheme)
        assert np.all(dQ == 0.0) and np.all(dK == 0.0)
        _, _, dVr = oracle.backward(inp.q, inp.k, inp.v, inp.do, 0.0, causal)
        assert np.max(np.abs(dV - dVr)) <= TOL


@pytest.mark.parametrize("hilo", [False, True], ids=["bf16", "hilo"])
def test_bwd_two_pass_is_deterministic(hilo):
    """fa_bwd uses no atomics: two runs give bitwise identical gradients."""
    import torch
    announce(f"bwd determinism hilo={hilo}")
    inp = gen(43, 2, 4, 2, 700, 700, 128, with_do=True)
    scale = float(np.float32(1 / math.sqrt(128)))
    q, k, v, do = upload(inp)
    o, lse = binding.forward(q, k, v, scale, True, out_dtype=torch.float32)
    r1 = binding.backward(q, k, v, o, lse, do, scale, True, grad_dtype=torch.float32, hilo=hilo)
    r2 = binding.backward(q, k, v, o, lse, do, scale, True, grad_dtype=torch.float32, hilo=hilo)
    torch.cuda.synchronize()
    for a, b in zip(r1, r2):
        assert torch.equal(a, b)


BF16_O_CASES = [
    (1, 4, 2, 300, 300, 128, True),
    (1, 2, 2, 129, 200, 64, False),
    (2, 2, 1, 257, 257, 128, False),
]


@pytest.mark.parametrize("case", BF16_O_CASES, ids=[_cid(c) for c in BF16_O_CASES])
def test_bwd_with_bf16_o(case):
    """fa_bwd given the bf16 O of the forward (the timed configuration). D
    must be rowsum(dO o O) of that O, and the gradients must equal, within the
    flat bound, the exact gradients of the definition evaluated with that D:
    with dD_i = rowsum(dO_i o (O16_i - O_i)), dS_ij = P_ij (dP_ij - D_i)
    moves by exactly -P_ij dD_i, so dQ_i moves by -s dD_i (P K)_i and dK_j by
    -s sum_i P_ij dD_i Q_i, and dV does not move (hilo scheme, so that the
    bound measures the kernel and not the bf16 rounding of P and dS)."""
    import torch
    B, Hq, Hkv, Nq, Nk, d, causal = case
    announce(f"bwd with bf16 O {case}")
    inp = gen(500 + Nq + d, B, Hq, Hkv, Nq, Nk, d, with_do=True)
    scale = float(np.float32(1 / math.sqrt(d)))
    q, k, v, do = upload(inp)
    o16, lse = binding.forward(q, k, v, scale, causal, out_dtype=torch.bfloat16)
    dq, dk, dv, dvec = binding.backward(q, k, v, o16, lse, do, scale, causal, grad_dtype=torch.float32, hilo=True)
    torch.cuda.synchronize()
    O16 = host(o16).astype(np.float64)
    dQ, dK, dV, Dv = host(dq), host(dk), host(dv), host(dvec)
    assert np.max(np.abs(Dv - oracle.row_dot(inp.do, O16))) <= 1e-4
    dQr, dKr, dVr = oracle.backward(inp.q, inp.k, inp.v, inp.do, scale, causal)
    qq, kk, vv, dd = (x.astype(np.float64) for x in (inp.q, inp.k, inp.v, inp.do))
    G = Hq // Hkv
    for b in range(B):
        for h in range(Hq):
            g = h // G
            P = oracle.probabilities_head(qq[b, h], kk[b, g], scale, causal)
            dD = oracle.row_dot(dd[b, h], O16[b, h] - P @ vv[b, g])
            dQr[b, h] -= scale * dD[:, None] * (P @ kk[b, g])
            dKr[b, g] -= scale * P.T @ (dD[:, None] * qq[b, h])
    check_flat(dQ, dK, dV, dQr, dKr, dVr, f"{_cid(case)} bf16 O")


@pytest.mark.parametrize("hkv", [1, 2], ids=["gqa", "mha"])
@pytest.mark.parametrize("d", [128, 64])
@pytest.mark.parametrize("hilo", [False, True], ids=["bf16", "hilo"])
def test_bwd_nan_in_one_q_row(hilo, d, hkv):
    """A NaN in query row i of one head (causal, the K/V head shared by two
    query heads). The outputs that depend on that row become NaN: O_i, L_i,
    D_i, dQ_i, and dV_j, dK_j of every key j <= i it sees. The K/V-outer pass
    forms dK_j = s sum_i dS_ij Q_i over aligned blocks of query rows (64 rows
    at head dim 64 with bf16 P and dS, and at head dim 128 with bf16 P and dS
    for causal rows of up to 1024 keys without query-head groups, else 32
    rows), so a NaN in Q_i (and in
    D_i, through dS_ij = P_ij (dP_ij - D_i) with P_ij = 0) also reaches dK_j
    for the keys after i up to the end of i's block, j <= 64 floor(i / 64) + 63
    (j <= 32 floor(i / 32) + 31), which do not depend on it. Every other output
    is finite and matches the oracle evaluated with the row set to zero."""
    import torch
    B, Hq, Hkv, N = 1, 2, hkv, 300
    i = 77
    announce(f"bwd NaN Q row hilo={hilo} d={d} Hkv={hkv}")
    inp = gen(71, B, Hq, Hkv, N, N, d, with_do=True)
    clean_q = inp.q.copy()
    clean_q[0, 1, i] = 0.0
    inp.q[0, 1, i] = np.nan
    inp.q_bits[0, 1, i] = np.uint16(0x7FC0)
    scale = float(np.float32(1 / math.sqrt(d)))
    q, k, v, do = upload(inp)
    o, lse = binding.forward(q, k, v, scale, True, out_dtype=torch.float32)
    dq, dk, dv, dvec = binding.backward(q, k, v, o, lse, do, scale, True, grad_dtype=torch.float32, hilo=hilo)
    torch.cuda.synchronize()
    dQ, dK, dV, Dv = host(dq), host(dk), host(dv), host(dvec)
    rows_nan = np.zeros((B, Hq, N), dtype=bool)
    rows_nan[0, 1, i] = True
    keys = np.arange(N)
    kvh = 1 // (Hq // Hkv)  # the K/V head of query head 1
    dv_nan = np.zeros((B, Hkv, N), dtype=bool)
    dv_nan[0, kvh] = keys <= i
    dk_nan = np.zeros((B, Hkv, N), dtype=bool)
    blk = 64 if (not hilo and (d == 64 or Hq == Hkv)) else 32
    dk_nan[0, kvh] = keys <= blk * (i // blk) + blk - 1
    assert np.array_equal(np.isnan(Dv), rows_nan)
    assert np.array_equal(np.isnan(dQ).any(axis=-1), rows_nan) and np.all(np.isnan(dQ[rows_nan]))
    assert np.array_equal(np.isnan(dV).any(axis=-1), dv_nan) and np.all(np.isnan(dV[dv_nan]))
    assert np.array_equal(np.isnan(dK).any(axis=-1), dk_nan) and np.all(np.isnan(dK[dk_nan]))
    dQr, dKr, dVr = oracle.backward(clean_q, inp.k, inp.v, inp.do, scale, True)
    e = (np.max(np.abs(dQ[~rows_nan] - dQr[~rows_nan])), np.max(np.abs(dK[~dk_nan] - dKr[~dk_nan])),
         np.max(np.abs(dV[~dv_nan] - dVr[~dv_nan])))
    print(f"NaN Q row, finite outputs: max|d dQ|={e[0]:.3e} max|d dK|={e[1]:.3e} max|d dV|={e[2]:.3e}")
    assert max(e) <= TOL
