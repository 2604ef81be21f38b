"""The seeded input generator: determinism, rounding and the outlier recipe."""

import numpy as np
import torch

from exact_tiled_attention_28_amd.inputs import make_inputs, round_to_bf16
from exact_tiled_attention_28_amd.workloads import (
    WORKLOADS, bwd_flops, fwd_bytes, fwd_flops, workload_flops)


def test_bf16_rounding_matches_torch_rne():
    rng = np.random.default_rng(0)
    x = np.concatenate([
        rng.standard_normal(100000).astype(np.float32),
        (rng.standard_normal(1000) * 1e30).astype(np.float32),
        (rng.standard_normal(1000) * 1e-30).astype(np.float32),
        np.array([0.0, -0.0, 1.0, 1.00390625, 1.01171875, 65504.0], np.float32),
    ])
    vals, bits = round_to_bf16(x)
    ref = torch.from_numpy(x).to(torch.bfloat16)
    assert np.array_equal(bits, ref.view(torch.int16).numpy().view(np.uint16))
    assert np.array_equal(vals, ref.float().numpy())


def test_same_seed_same_bytes():
    a = make_inputs(3, 1, 4, 2, 33, 33, 64, "bf16", with_do=True, n_outlier_channels=2)
    b = make_inputs(3, 1, 4, 2, 33, 33, 64, "bf16", with_do=True, n_outlier_channels=2)
    for x, y in [(a.q_bits, b.q_bits), (a.k_bits, b.k_bits), (a.v_bits, b.v_bits), (a.do_bits, b.do_bits)]:
        assert x.tobytes() == y.tobytes()
    c = make_inputs(4, 1, 4, 2, 33, 33, 64, "bf16", with_do=True)
    assert c.q_bits.tobytes() != a.q_bits.tobytes()


def test_shapes_and_f32_mode():
    x = make_inputs(1, 2, 6, 3, 17, 29, 64, "f32", with_do=True)
    assert x.q.shape == (2, 6, 17, 64) and x.k.shape == (2, 3, 29, 64) and x.v.shape == x.k.shape
    assert x.do.shape == x.q.shape and x.q_bits is None and x.q.dtype == np.float32


def test_outlier_channels_scaled_before_rounding():
    plain = make_inputs(9, 1, 2, 1, 64, 64, 128, "f32", n_outlier_channels=0)
    out = make_inputs(9, 1, 2, 1, 64, 64, 128, "f32", n_outlier_channels=2, outlier_factor=20.0)
    ch = out.outlier_channels
    assert ch.size == 2 and len(set(ch.tolist())) == 2
    assert np.array_equal(out.q[..., ch], plain.q[..., ch] * np.float32(20))
    assert np.array_equal(out.k[..., ch], plain.k[..., ch] * np.float32(20))
    rest = np.setdiff1d(np.arange(128), ch)
    assert np.array_equal(out.q[..., rest], plain.q[..., rest])
    assert np.array_equal(out.v, plain.v)
    bf = make_inputs(9, 1, 2, 1, 64, 64, 128, "bf16", n_outlier_channels=2, outlier_factor=20.0)
    assert np.array_equal(bf.q, round_to_bf16(out.q)[0])


def test_flop_and_byte_accounting():
    # 4*d flops per visible pair, causal halves the square.
    assert fwd_flops(1, 1, 128, 128, 64, False) == 4 * 128 * 128 * 64
    assert abs(workload_flops(WORKLOADS["fwd_bf16_causal_b8_h16_n2048_d128"]) - 137.44e9) < 0.01e9
    assert abs(workload_flops(WORKLOADS["fwd_bf16_causal_b1_h8_n16384_d128"]) - 549.76e9) < 0.01e9
    assert abs(workload_flops(WORKLOADS["bwd_bf16_causal_b4_h16_n4096_d128"]) - 687.19e9) < 0.01e9
    assert bwd_flops(1, 2, 8, 8, 4, True) == 2.5 * fwd_flops(1, 2, 8, 8, 4, True)
    assert fwd_bytes(1, 1, 1, 128, 128, 64, 4, 4) == 131584
