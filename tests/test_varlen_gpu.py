"""Packed variable-length batches on the GPU: fa_fwd_varlen / fa_bwd_varlen
(through the C ABI) against the fp64 oracle's per-sequence definition on the
same seeded inputs.

Bounds as for the fixed-length shapes: O max-abs 1e-2 and L 1e-3 (fp32
outputs); dQ, dK, dV max-abs 1e-2. The backward runs with FA_PRECISION_HILO
(P and dS as bf16 pairs) on every case and also with FA_PRECISION_BF16 where
no query heads are summed into one K/V head (with a group, the bf16 rounding
of P alone can reach the flat bound on short causal rows; test_bwd_gpu.py).
Rows of a sequence without keys must be exactly O = 0, L = -inf, dQ = 0; keys
of a sequence without queries dK = dV = 0.
"""

import numpy as np
import pytest

import oracle
from exact_tiled_attention_28_amd import binding
from exact_tiled_attention_28_amd.inputs import make_varlen_inputs
from tests.gpu_util import announce, host

pytestmark = pytest.mark.gpu


def upload(x):
    import torch
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).cuda().bfloat16()


def cu_dev(cu):
    import torch
    return torch.from_numpy(np.ascontiguousarray(cu, dtype=np.int32)).cuda()


CASES = [
    # (lengths_q, lengths_k, Hq, Hkv, d, causal)
    ([1, 63, 64, 65, 129, 300, 2], None, 4, 2, 128, True),
    ([200, 1, 0, 257, 128], None, 2, 2, 64, True),
    ([100, 3, 77, 0, 64], [257, 40, 1, 9, 0], 4, 1, 128, False),
    ([5, 130, 33], [0, 65, 1000], 2, 2, 64, False),
    ([1000, 17, 513], None, 8, 2, 128, True),
]
IDS = [f"{'c' if c[5] else 'n'}d{c[4]}Hq{c[2]}Hkv{c[3]}b{len(c[0])}" for c in CASES]


def _run(case, seed, with_bwd, hilo=False):
    import torch
    lq, lk, Hq, Hkv, d, causal = case
    lk = lq if lk is None else lk
    inp = make_varlen_inputs(seed, lq, lk, Hq, Hkv, d, with_do=with_bwd)
    scale = float(np.float32(1 / np.sqrt(d)))
    q, k, v = upload(inp.q), upload(inp.k), upload(inp.v)
    cq = cu_dev(inp.cu_q)
    ck = cq if causal else cu_dev(inp.cu_k)
    o, lse = binding.forward_varlen(q, k, v, cq, ck, inp.max_q, inp.max_k, scale, causal, out_dtype=torch.float32)
    out = {"o": o, "lse": lse}
    if with_bwd:
        do = upload(inp.do)
        dq, dk, dv, _ = binding.backward_varlen(q, k, v, o, lse, do, cq, ck, inp.max_q, inp.max_k, scale, causal,
                                                grad_dtype=torch.float32, hilo=hilo)
        out.update(dq=dq, dk=dk, dv=dv)
    torch.cuda.synchronize()
    return inp, scale, {n: host(t) for n, t in out.items()}


def _no_key_rows(inp):
    rows = np.zeros(inp.q.shape[1], dtype=bool)
    for b in range(inp.cu_q.size - 1):
        if inp.cu_k[b + 1] == inp.cu_k[b]:
            rows[inp.cu_q[b]:inp.cu_q[b + 1]] = True
    return rows


@pytest.mark.parametrize("case", CASES, ids=IDS)
def test_varlen_forward_parity(case):
    announce(f"fwd varlen {case}")
    inp, scale, r = _run(case, 900 + len(case[0]), False)
    Or, Lr = oracle.forward_varlen(inp.q, inp.k, inp.v, inp.cu_q, inp.cu_k, scale, case[5])
    empty = _no_key_rows(inp)
    assert np.all(r["o"][:, empty] == 0) and np.all(r["lse"][:, empty] == -np.inf)
    assert np.max(np.abs(r["o"][:, ~empty] - Or[:, ~empty]), initial=0) <= 1e-2
    assert np.max(np.abs(r["lse"][:, ~empty] - Lr[:, ~empty]), initial=0) <= 1e-3


BWD_PARAMS = [(i, hilo) for i, c in enumerate(CASES) for hilo in (False, True) if hilo or c[2] == c[3]]


@pytest.mark.parametrize("ci,hilo", BWD_PARAMS, ids=[f"{IDS[i]}-{'hilo' if h else 'bf16'}" for i, h in BWD_PARAMS])
def test_varlen_backward_parity(ci, hilo):
    case = CASES[ci]
    announce(f"bwd varlen {case} hilo={hilo}")
    inp, scale, r = _run(case, 950 + len(case[0]), True, hilo=hilo)
    dQ, dK, dV = oracle.backward_varlen(inp.q, inp.k, inp.v, inp.do, inp.cu_q, inp.cu_k, scale, case[5])
    e = [np.max(np.abs(r["dq"] - dQ)), np.max(np.abs(r["dk"] - dK)), np.max(np.abs(r["dv"] - dV))]
    print(f"varlen {IDS[ci]} hilo={hilo}: max|d dQ|={e[0]:.3e} max|d dK|={e[1]:.3e} max|d dV|={e[2]:.3e}")
    assert max(e) <= 1e-2
    # exact zeros where there is nothing to attend to
    assert np.all(r["dq"][:, _no_key_rows(inp)] == 0)
    for b in range(inp.cu_q.size - 1):
        if inp.cu_q[b + 1] == inp.cu_q[b]:
            k0, k1 = inp.cu_k[b], inp.cu_k[b + 1]
            assert np.all(r["dk"][:, k0:k1] == 0) and np.all(r["dv"][:, k0:k1] == 0)


def test_varlen_equal_lengths_match_fixed_length_path():
    """Equal lengths: the packed path gives the fixed-length path's numbers
    bit for bit (same kernels, same tiling, only the addressing differs)."""
    import torch
    B, H, N, d = 3, 4, 200, 128
    announce("fwd varlen == fixed")
    inp = make_varlen_inputs(77, [N] * B, [N] * B, H, H, d)
    scale = float(np.float32(1 / np.sqrt(d)))
    q, k, v = upload(inp.q), upload(inp.k), upload(inp.v)
    cu = cu_dev(inp.cu_q)
    o_v, l_v = binding.forward_varlen(q, k, v, cu, cu, N, N, scale, True, out_dtype=torch.float32)
    to_bhsd = lambda x: x.view(H, B, N, d).permute(1, 0, 2, 3).contiguous()
    o_f, l_f = binding.forward(to_bhsd(q), to_bhsd(k), to_bhsd(v), scale, True, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(o_v.view(H, B, N, d).permute(1, 0, 2, 3), o_f)
    assert torch.equal(l_v.view(H, B, N).permute(1, 0, 2), l_f)
