"""fa_fwd and fa_bwd inside a captured HIP graph (torch.cuda.CUDAGraph):
the library enqueues only kernels on the stream it is given (no allocation,
no memset, no host synchronisation), so both calls can be captured once and
replayed. Every replay, with eager work and synchronisations between
replays and the outputs overwritten with NaN before each, must give the
eager results bit for bit. All buffers are allocated before the capture;
inside it only the C-ABI entry points run."""

import math

import numpy as np
import pytest

from exact_tiled_attention_28_amd import binding
from tests.gpu_util import announce

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("causal", [True, False], ids=["causal", "noncausal"])
@pytest.mark.parametrize("d", [64, 128])
def test_fwd_bwd_replayed_from_a_captured_graph(causal, d):
    import torch
    B, Hq, Hkv, N = 2, 4, 2, 700
    announce(f"graph capture B{B} Hq{Hq} Hkv{Hkv} N{N} d{d} causal={causal}")
    g = torch.Generator(device="cuda").manual_seed(123 + d + int(causal))
    q = torch.randn(B, Hq, N, d, device="cuda", generator=g).bfloat16()
    k = torch.randn(B, Hkv, N, d, device="cuda", generator=g).bfloat16()
    v = torch.randn(B, Hkv, N, d, device="cuda", generator=g).bfloat16()
    do = torch.randn(B, Hq, N, d, device="cuda", generator=g).bfloat16()
    scale = float(np.float32(1 / math.sqrt(d)))
    o = torch.empty_like(q)
    lse = torch.empty(B, Hq, N, device="cuda", dtype=torch.float32)
    dq = torch.empty(B, Hq, N, d, device="cuda", dtype=torch.float32)
    dk, dv = torch.empty_like(k), torch.empty_like(v)
    ws = torch.empty(binding.fa_bwd_workspace_bytes(B, Hq, N) // 4, device="cuda", dtype=torch.float32)
    bf = binding.FA_DTYPE_BF16

    def calls(stream):
        rc = binding.fa_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), B, Hq, Hkv, N, N,
                            d, scale, int(causal), bf, bf, stream)
        assert rc == 0, binding.fa_last_error()
        rc = binding.fa_bwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), do.data_ptr(),
                            dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), ws.data_ptr(), B, Hq, Hkv, N, N, d, scale,
                            int(causal), bf, bf, bf, binding.FA_PRECISION_BF16, stream)
        assert rc == 0, binding.fa_last_error()

    outs = (o, lse, dq, dk, dv)
    calls(torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    ref = [t.clone() for t in outs]

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=s):
        calls(s.cuda_stream)
    torch.cuda.synchronize()

    for rep in range(4):
        for t in outs:
            t.fill_(float("nan"))
        x = torch.randn(512, 512, device="cuda", generator=g)
        y = (x @ x).sum()  # eager work between the replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.isfinite(y)
        for name, got, want in zip(("O", "L", "dQ", "dK", "dV"), outs, ref):
            assert torch.equal(got, want), f"replay {rep}: {name} differs from the eager call"
