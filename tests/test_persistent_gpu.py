"""The persistent work-queue forward (fa_fwd_persistent through the C ABI):
the same per-item arithmetic as fa_fwd's 4-wavefront kernel, so for keys
below the length where fa_fwd switches to its 8-wavefront kernel the outputs
must be bit-identical to fa_fwd's; everywhere they must meet the forward's
bounds against the fp64 oracle (O max-abs 1e-2, L 1e-3, O requested in
fp32). The counter array must be back to zero after every call, including
calls of different sizes in a row and a grid smaller than the item count.
"""

import math

import numpy as np
import pytest

import oracle
from exact_tiled_attention_28_amd import binding
from tests.gpu_util import announce, gen, host, upload

pytestmark = pytest.mark.gpu

CASES = [
    # (B, Hq, Hkv, Nq, Nk, d, causal)
    (1, 1, 1, 1, 1, 128, True),
    (1, 2, 2, 17, 17, 64, True),
    (1, 4, 1, 257, 257, 128, True),
    (1, 2, 2, 100, 257, 128, False),
    (1, 2, 2, 333, 65, 64, False),
    (2, 8, 2, 512, 512, 128, True),
    (1, 1, 1, 1000, 1000, 64, True),
]


def _ids(c):
    return f"B{c[0]}Hq{c[1]}Hkv{c[2]}Nq{c[3]}Nk{c[4]}d{c[5]}{'c' if c[6] else 'n'}"


@pytest.mark.parametrize("case", CASES, ids=[_ids(c) for c in CASES])
def test_persistent_matches_oracle_and_fa_fwd(case):
    import torch
    B, Hq, Hkv, Nq, Nk, d, causal = case
    announce(f"fa_fwd_persistent {_ids(case)}")
    inp = gen(400 + Nq + d, B, Hq, Hkv, Nq, Nk, d)
    q, k, v, _ = upload(inp)
    scale = float(np.float32(1 / math.sqrt(d)))
    sched = binding.new_sched()
    o, lse = binding.forward_persistent(q, k, v, scale, causal, sched, out_dtype=torch.float32)
    o_ref, lse_ref = binding.forward(q, k, v, scale, causal, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert int(sched.abs().sum()) == 0, "work-queue counters must be zero after the call"
    assert torch.equal(o, o_ref) and torch.equal(lse, lse_ref), "must equal fa_fwd bit for bit"
    Or, Lr = oracle.forward(inp.q, inp.k, inp.v, scale, causal)
    assert np.max(np.abs(host(o) - Or)) <= 1e-2
    assert np.max(np.abs(host(lse) - Lr)) <= 1e-3


def test_persistent_calls_in_a_row_and_bf16_output():
    # a large call (more items than resident workgroups), then a small one,
    # then the large one again with bf16 output, on the same counter array
    import torch
    sched = binding.new_sched()
    scale = float(np.float32(1 / math.sqrt(128)))
    for i, (B, H, N, out) in enumerate([(8, 16, 1024, torch.float32), (1, 2, 130, torch.float32),
                                        (8, 16, 1024, torch.bfloat16)]):
        announce(f"fa_fwd_persistent call {i}: B{B} H{H} N{N} {out}")
        inp = gen(500 + i, B, H, H, N, N, 128)
        q, k, v, _ = upload(inp)
        o, lse = binding.forward_persistent(q, k, v, scale, True, sched, out_dtype=out)
        o_ref, lse_ref = binding.forward(q, k, v, scale, True, out_dtype=out)
        torch.cuda.synchronize()
        assert int(sched.abs().sum()) == 0
        assert torch.equal(o, o_ref) and torch.equal(lse, lse_ref)


def test_persistent_long_keys_against_oracle():
    # a longer key range than the bit-identity cases; both paths within the
    # bounds, on sampled rows
    import torch
    B, H, N, d = 1, 2, 4160, 128
    announce(f"fa_fwd_persistent long keys B{B} H{H} N{N}")
    inp = gen(777, B, H, H, N, N, d)
    q, k, v, _ = upload(inp)
    scale = float(np.float32(1 / math.sqrt(d)))
    sched = binding.new_sched()
    o, lse = binding.forward_persistent(q, k, v, scale, True, sched, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert int(sched.abs().sum()) == 0
    rows = np.array([0, 1, 127, 128, 2047, 4095, 4096, N - 1])
    O, L = host(o), host(lse)
    for h in range(H):
        Or, Lr = oracle.forward_head(inp.q[0, h], inp.k[0, h], inp.v[0, h], scale, True, rows=rows)
        assert np.max(np.abs(O[0, h][rows] - Or)) <= 1e-2
        assert np.max(np.abs(L[0, h][rows] - Lr)) <= 1e-3
