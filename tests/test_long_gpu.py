"""Long sequences on the GPU, beyond the named workloads: 2^18 + 37 keys
(ragged last tile), causal GQA at d = 128 (the 8-wavefront forward and the
two backward passes) and non-causal at d = 64, against the fp64 oracle on
sampled rows: O and L of the forward (oracle.forward_head with rows) and dQ of
the backward (oracle.backward_dq_rows, exact per row). Bounds as for the
named workloads: O and dQ max-abs 1e-2, L 1e-3 (fp32 outputs). The sampled
rows include the first and last rows and tile boundaries; over 262181 keys
they exercise the online-softmax rescaling over long loops and the large
row offsets of every kernel.
"""

import math

import numpy as np
import pytest

import oracle
from exact_tiled_attention_28_amd import binding
from tests.gpu_util import announce, gen, host, upload

pytestmark = pytest.mark.gpu

N = (1 << 18) + 37


def _rows(rng, n):
    fixed = [0, 1, 63, 64, 127, 128, 255, 256, n // 2, n - 130, n - 65, n - 38, n - 37, n - 2, n - 1]
    return np.array(sorted(set(fixed) | set(rng.choice(n, size=9, replace=False).tolist())))


@pytest.mark.parametrize("case", [(2, 1, 128, True), (1, 1, 64, False)], ids=["causal_gqa_d128", "noncausal_d64"])
def test_long_sequence_forward_and_dq(case):
    import torch
    Hq, Hkv, d, causal = case
    announce(f"long sequence N={N} Hq={Hq} Hkv={Hkv} d={d} causal={causal}")
    inp = gen(4242 + d, 1, Hq, Hkv, N, N, d, with_do=True)
    q, k, v, do = upload(inp)
    scale = float(np.float32(1 / math.sqrt(d)))
    o, lse = binding.forward(q, k, v, scale, causal, out_dtype=torch.float32)
    dq, dk, dv, _ = binding.backward(q, k, v, o, lse, do, scale, causal, grad_dtype=torch.float32)
    torch.cuda.synchronize()
    O, L, dQ = host(o), host(lse), host(dq)
    assert np.all(np.isfinite(O)) and np.all(np.isfinite(dQ))
    dK, dV = host(dk), host(dv)
    assert np.all(np.isfinite(dK)) and np.all(np.isfinite(dV))
    # Sum rules over every key (the oracle's full columns are out of reach
    # here): sum_j dK_j = 0 since every row of dS sums to 0, and
    # sum_j dV_j = sum over the group's query heads and rows of dO.
    dO_sum = inp.do.astype(np.float64).reshape(1, Hkv, Hq // Hkv, N, d).sum(axis=(2, 3))
    rule_k = float(np.max(np.abs(dK.sum(axis=2))))
    rule_v = float(np.max(np.abs(dV.sum(axis=2) - dO_sum)))
    print(f"N={N}: sum rules max|sum dK|={rule_k:.3e} max|sum dV - sum dO|={rule_v:.3e}")
    assert rule_k <= 0.05 and rule_v <= 0.05 + 1e-4 * float(np.max(np.abs(dO_sum)))
    rng = np.random.default_rng(7)
    worst = [0.0, 0.0, 0.0]
    for h in range(Hq):
        g = h // (Hq // Hkv)
        rows = _rows(rng, N)
        Or, Lr = oracle.forward_head(inp.q[0, h], inp.k[0, g], inp.v[0, g], scale, causal, rows=rows)
        dQr = oracle.backward_dq_rows(inp.q[0, h], inp.k[0, g], inp.v[0, g], inp.do[0, h], scale, causal, rows)
        worst[0] = max(worst[0], float(np.max(np.abs(O[0, h][rows] - Or))))
        worst[1] = max(worst[1], float(np.max(np.abs(L[0, h][rows] - Lr))))
        worst[2] = max(worst[2], float(np.max(np.abs(dQ[0, h][rows] - dQr))))
    print(f"N={N}: max|dO|={worst[0]:.3e} max|dL|={worst[1]:.3e} max|d dQ|={worst[2]:.3e}")
    assert worst[0] <= 1e-2
    assert worst[1] <= 1e-3
    assert worst[2] <= 1e-2


def test_keys_past_two_gib_per_head():
    # 8392709 keys at d = 128: K and V of one head span more than 2^31 bytes
    # (keys from 2^23 on lie past that mark), so every K/V offset there must
    # be formed in 64 bits. Each query row i gets one planted key
    # j_i = 2^23 + 37 i past the mark with K[j_i] = 3 q_i (rounded to bf16):
    # its score (about 0.088 * 3 * |q_i|^2, above 25 for any row here)
    # dominates the 8.4M random ones (their exp-sum is about 1.4e7), so O_i is about
    # V[j_i] and the planted keys carry O(1) gradients, which a wrong offset
    # would change far beyond the bounds. 70 ragged query rows keep the full
    # fp64 oracle backward affordable (8 query rows at a time).
    import torch
    from exact_tiled_attention_28_amd.inputs import round_to_bf16
    nq, nk, d = 70, (1 << 23) + 4101, 128
    assert nk * d * 2 > 2 ** 31
    announce(f"keys past 2 GiB: Nq={nq} Nk={nk} d={d} non-causal")
    inp = gen(777, 1, 1, 1, nq, nk, d, with_do=True)
    planted = (1 << 23) + 37 * np.arange(nq)
    vals, bits = round_to_bf16(np.ascontiguousarray(3.0 * inp.q[0, 0], dtype=np.float32))
    inp.k[0, 0, planted], inp.k_bits[0, 0, planted] = vals, bits
    q, k, v, do = upload(inp)
    scale = float(np.float32(1 / math.sqrt(d)))
    o, lse = binding.forward(q, k, v, scale, False, out_dtype=torch.float32)
    dq, dk, dv, _ = binding.backward(q, k, v, o, lse, do, scale, False, grad_dtype=torch.float32)
    torch.cuda.synchronize()
    rng = np.random.default_rng(3)
    keys = np.array(sorted(set([0, 1, 63, 64, nk // 2, (1 << 23) - 1, nk - 2, nk - 1]) | set(planted[::3].tolist())
                           | set(rng.choice(nk, size=16, replace=False).tolist())))
    key_idx = torch.from_numpy(keys).cuda()
    dK_s, dV_s = host(dk[0, 0].index_select(0, key_idx)), host(dv[0, 0].index_select(0, key_idx))
    O, L, dQ = host(o), host(lse), host(dq)
    del q, k, v, do, o, lse, dq, dk, dv
    torch.cuda.empty_cache()
    Or, Lr = oracle.forward_head(inp.q[0, 0], inp.k[0, 0], inp.v[0, 0], scale, False, row_block=8)
    dQr, dKr, dVr = oracle.backward_head(inp.q[0, 0], inp.k[0, 0], inp.v[0, 0], inp.do[0, 0], scale, False,
                                         row_block=8)
    # the planted keys dominate: O_i is close to V[j_i], far from the mean of V
    assert np.max(np.abs(Or - inp.v[0, 0, planted])) < 0.1 and np.min(np.max(np.abs(Or), axis=1)) > 0.5
    errs = [np.max(np.abs(O[0, 0] - Or)), np.max(np.abs(L[0, 0] - Lr)), np.max(np.abs(dQ[0, 0] - dQr)),
            np.max(np.abs(dK_s - dKr[keys])), np.max(np.abs(dV_s - dVr[keys]))]
    print("O L dQ dK dV max-abs errors:", ", ".join(f"{e:.3e}" for e in errs),
          "| max |dV| at planted keys", f"{np.max(np.abs(dVr[planted])):.2f}")
    assert errs[0] <= 1e-2 and errs[1] <= 1e-3 and max(errs[2:]) <= 1e-2
