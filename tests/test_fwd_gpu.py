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
    # 8-wavefront kernel without the causal mask (from 4096 keys): ragged
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


# ---------------------------------------------------------------------------
# edge cases: NaN rows, identical keys, repeatability, streams, tile shapes
# ---------------------------------------------------------------------------

BF16_NAN = np.uint16(0x7FC0)


def _plant_nan(inp, which, index):
    """Make one row of Q or K (index = (b, h, row)) NaN in both the value and
    the bf16 bit arrays."""
    getattr(inp, which)[index] = np.nan
    getattr(inp, which + "_bits")[index] = BF16_NAN


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True], ids=["noncausal", "causal"])
def test_fwd_nan_in_one_q_row(causal, d):
    """A NaN in query row i of one head makes exactly O_i and L_i of that head
    NaN (nothing else depends on that row); every other output is finite and
    matches the oracle (evaluated with the row set to zero, which the other
    outputs do not depend on)."""
    B, Hq, Hkv, N = 1, 2, 1, 300
    i = 77
    announce(f"fwd NaN Q row causal={causal} d={d}")
    inp = gen(61, B, Hq, Hkv, N, N, d)
    clean_q = inp.q.copy()
    clean_q[0, 1, i] = 0.0
    _plant_nan(inp, "q", (0, 1, i))
    scale = float(np.float32(1 / math.sqrt(d)))
    O, L = run_fwd(inp, scale, causal)
    expect_nan = np.zeros((B, Hq, N), dtype=bool)
    expect_nan[0, 1, i] = True
    assert np.array_equal(np.isnan(L), expect_nan)
    assert np.array_equal(np.isnan(O).any(axis=-1), expect_nan) and np.all(np.isnan(O[0, 1, i]))
    Or, Lr = oracle.forward(clean_q, inp.k, inp.v, scale, causal)
    ok = ~expect_nan
    assert np.all(np.isfinite(O[ok])) and np.all(np.isfinite(L[ok]))
    assert np.max(np.abs(O[ok] - Or[ok])) <= O_TOL_BF16
    assert np.max(np.abs(L[ok] - Lr[ok])) <= L_TOL_BF16


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True], ids=["noncausal", "causal"])
def test_fwd_nan_in_one_k_row(causal, d):
    """A NaN in key row j of a K/V head reaches every query of its group that
    sees key j: with the causal mask exactly the rows i >= j of the group's
    query heads (the masked scores of rows i < j are replaced, not
    multiplied), without it every row of the group. Other outputs match the
    oracle."""
    B, Hq, Hkv, N = 1, 4, 2, 300
    j = 150
    announce(f"fwd NaN K row causal={causal} d={d}")
    inp = gen(62, B, Hq, Hkv, N, N, d)
    clean_k = inp.k.copy()
    clean_k[0, 0, j] = 0.0
    _plant_nan(inp, "k", (0, 0, j))
    scale = float(np.float32(1 / math.sqrt(d)))
    O, L = run_fwd(inp, scale, causal)
    expect_nan = np.zeros((B, Hq, N), dtype=bool)
    rows = np.arange(N) >= j if causal else np.ones(N, dtype=bool)
    expect_nan[0, 0:2] = rows  # query heads 0 and 1 use K/V head 0
    assert np.array_equal(np.isnan(L), expect_nan)
    assert np.array_equal(np.isnan(O).any(axis=-1), expect_nan)
    assert np.all(np.isnan(O[expect_nan]))
    Or, Lr = oracle.forward(inp.q, clean_k, inp.v, scale, causal)
    ok = ~expect_nan
    assert np.max(np.abs(O[ok] - Or[ok])) <= O_TOL_BF16
    assert np.max(np.abs(L[ok] - Lr[ok])) <= L_TOL_BF16


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True], ids=["noncausal", "causal"])
def test_fwd_identical_keys_closed_form(causal, d):
    """Every key row equal to one vector k: each score row is constant, so O_i
    is the mean of the value rows row i sees and L_i = s q_i . k + ln n_i
    (n_i = i + 1 causal, Nk otherwise). Checked against that closed form, not
    the oracle."""
    from exact_tiled_attention_28_amd.inputs import round_to_bf16
    B, Hq, Hkv, N = 1, 4, 2, 333
    announce(f"fwd identical keys causal={causal} d={d}")
    inp = gen(63, B, Hq, Hkv, N, N, d)
    rng = np.random.default_rng(64)
    kv, kb = round_to_bf16(rng.standard_normal(d, dtype=np.float32))
    inp.k[:] = kv
    inp.k_bits[:] = kb
    scale = float(np.float32(1 / math.sqrt(d)))
    O, L = run_fwd(inp, scale, causal)
    v = inp.v.astype(np.float64)
    n = np.arange(1, N + 1) if causal else np.full(N, N)
    for h in range(Hq):
        g = h // (Hq // Hkv)
        Oc = (np.cumsum(v[0, g], axis=0) if causal else np.broadcast_to(v[0, g].sum(axis=0), (N, d))) / n[:, None]
        Lc = scale * (inp.q[0, h].astype(np.float64) @ kv.astype(np.float64)) + np.log(n)
        assert np.max(np.abs(O[0, h] - Oc)) <= O_TOL_BF16
        assert np.max(np.abs(L[0, h] - Lc)) <= L_TOL_BF16


@pytest.mark.parametrize("shape", [(2, 4, 2, 2048, 128, True), (1, 2, 2, 16400, 128, True),
                                   (2, 2, 2, 1500, 64, False)], ids=["n2048_d128c", "n16400_d128c_8wave",
                                                                     "n1500_d64n"])
def test_fwd_bitwise_repeatable(shape):
    """The forward has no atomics and a fixed reduction order: two calls give
    identical bits (O and L)."""
    import torch
    B, Hq, Hkv, N, d, causal = shape
    announce(f"fwd repeatability {shape}")
    inp = gen(65, B, Hq, Hkv, N, N, d)
    q, k, v, _ = upload(inp)
    scale = float(np.float32(1 / math.sqrt(d)))
    o1, l1 = binding.forward(q, k, v, scale, causal)
    o2, l2 = binding.forward(q, k, v, scale, causal)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_non_default_stream():
    """fa_fwd and fa_bwd enqueue on the stream they are given: results on a
    fresh stream equal those on the default stream bit for bit, and are
    complete once that stream is synchronised."""
    import torch
    announce("non-default stream")
    inp = gen(66, 2, 4, 2, 700, 700, 128, with_do=True)
    scale = float(np.float32(1 / math.sqrt(128)))
    q, k, v, do = upload(inp)
    o, lse = binding.forward(q, k, v, scale, True, out_dtype=torch.float32)
    ref = binding.backward(q, k, v, o, lse, do, scale, True, grad_dtype=torch.float32)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        o_s, lse_s = binding.forward(q, k, v, scale, True, out_dtype=torch.float32, stream=s)
        got = binding.backward(q, k, v, o_s, lse_s, do, scale, True, grad_dtype=torch.float32, stream=s)
    s.synchronize()
    assert torch.equal(o_s, o) and torch.equal(lse_s, lse)
    for a, b in zip(got, ref):
        assert torch.equal(a, b)


@pytest.mark.parametrize("d", [64, 128])
def test_tile_shapes_agree(d):
    """From 16384 causal keys fa_fwd runs 256-row Q tiles (8 wavefronts);
    the packed variable-length path runs the same sequence in 128-row tiles
    (4 wavefronts). Each wavefront owns 32 query rows and visits the same key
    tiles in the same order in both, so O and L agree bit for bit; and from
    8192 keys at d = 128 the same holds for fa_bwd's dQ pass against
    fa_bwd_varlen's."""
    import torch
    N = 16400
    announce(f"tile shapes agree N={N} d={d}")
    inp = gen(67, 1, 2, 1, N, N, d, with_do=True)
    scale = float(np.float32(1 / math.sqrt(d)))
    q, k, v, do = upload(inp)
    o, lse = binding.forward(q, k, v, scale, True, out_dtype=torch.float32)
    cu = torch.tensor([0, N], dtype=torch.int32, device=q.device)
    o_v, l_v = binding.forward_varlen(q[0], k[0], v[0], cu, cu, N, N, scale, True, out_dtype=torch.float32)
    dq, dk, dv, _ = binding.backward(q, k, v, o, lse, do, scale, True, grad_dtype=torch.float32)
    dq_v, dk_v, dv_v, _ = binding.backward_varlen(q[0], k[0], v[0], o[0], lse[0], do[0], cu, cu, N, N, scale, True,
                                                  grad_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(o[0], o_v) and torch.equal(lse[0], l_v)
    assert torch.equal(dq[0], dq_v) and torch.equal(dk[0], dk_v) and torch.equal(dv[0], dv_v)
