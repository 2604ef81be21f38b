"""fa_bwd_noalloc (through the C ABI) against fa_bwd on the same inputs:
the same kernels, with D in the library's static scratch instead of the
caller's workspace, so dQ, dK and dV must be identical bit for bit. Two
calls in a row, the second with a smaller input (the scratch keeps the first
call's D, which the second must not read), both precisions, and one
run on a non-default stream."""

import math

import numpy as np
import pytest

from exact_tiled_attention_28_amd import binding
from tests.gpu_util import announce, gen, upload

pytestmark = pytest.mark.gpu


def _noalloc(q, k, v, o, lse, do, scale, causal, hilo, stream=None):
    import torch
    B, Hq, N, d = q.shape
    Hkv, Nk = k.shape[1], k.shape[2]
    dq = torch.empty((B, Hq, N, d), dtype=torch.float32, device=q.device)
    dk = torch.empty((B, Hkv, Nk, d), dtype=torch.float32, device=q.device)
    dv = torch.empty((B, Hkv, Nk, d), dtype=torch.float32, device=q.device)
    s = stream if stream is not None else torch.cuda.current_stream()
    rc = binding.fa_bwd_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                                do.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), B, Hq, Hkv, N, Nk, d,
                                float(scale), int(causal), binding.FA_DTYPE_BF16, binding.FA_DTYPE_F32,
                                binding.FA_DTYPE_F32,
                                binding.FA_PRECISION_HILO if hilo else binding.FA_PRECISION_BF16, s.cuda_stream)
    assert rc == binding.FA_OK, binding.fa_last_error()
    return dq, dk, dv


@pytest.mark.parametrize("hilo", [False, True], ids=["bf16", "hilo"])
def test_bwd_noalloc_matches_fa_bwd_twice(hilo):
    import torch
    shapes = [(2, 8, 2, 1000, 128, True), (1, 2, 1, 300, 64, False)]  # second call smaller
    for B, Hq, Hkv, N, d, causal in shapes:
        announce(f"fa_bwd_noalloc B{B} Hq{Hq} Hkv{Hkv} N{N} d{d} causal={causal} hilo={hilo}")
        inp = gen(31 + N, B, Hq, Hkv, N, N, d, with_do=True)
        scale = float(np.float32(1 / math.sqrt(d)))
        q, k, v, do = upload(inp)
        o, lse = binding.forward(q, k, v, scale, causal, out_dtype=torch.float32)
        ref = binding.backward(q, k, v, o, lse, do, scale, causal, grad_dtype=torch.float32, hilo=hilo)
        got = _noalloc(q, k, v, o, lse, do, scale, causal, hilo)
        torch.cuda.synchronize()
        for a, b in zip(got, ref[:3]):
            assert torch.equal(a, b)


def test_bwd_noalloc_on_a_stream():
    import torch
    B, Hq, Hkv, N, d = 1, 4, 4, 700, 128
    announce("fa_bwd_noalloc on a non-default stream")
    inp = gen(55, B, Hq, Hkv, N, N, d, with_do=True)
    scale = float(np.float32(1 / math.sqrt(d)))
    q, k, v, do = upload(inp)
    o, lse = binding.forward(q, k, v, scale, True, out_dtype=torch.float32)
    ref = binding.backward(q, k, v, o, lse, do, scale, True, grad_dtype=torch.float32)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        got = _noalloc(q, k, v, o, lse, do, scale, True, False, stream=s)
    s.synchronize()
    for a, b in zip(got, ref[:3]):
        assert torch.equal(a, b)
