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
    assert np.all(np.isfinite(host(dk))) and np.all(np.isfinite(host(dv)))
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
