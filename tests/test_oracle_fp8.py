"""Pins of the FP8 oracle pieces (oracle/fp8.py) against definitions that do
not use them: the OCP E4M3 format written out value by value, brute-force
nearest-code search, the explicit Sylvester Hadamard matrix, and the plain
attention oracle on inputs that FP8 represents exactly."""

import math

import numpy as np
import pytest

import oracle
from oracle import fp8
from exact_tiled_attention_28_amd.inputs import make_inputs


def test_e4m3_known_values():
    cases = {0x00: 0.0, 0x01: 2.0 ** -9, 0x07: 7 * 2.0 ** -9, 0x08: 2.0 ** -6, 0x38: 1.0, 0x39: 1.125,
             0x40: 2.0, 0x7E: 448.0, 0xB8: -1.0, 0xFE: -448.0, 0x80: -0.0}
    for c, val in cases.items():
        assert fp8.e4m3_decode([c])[0] == val
    assert np.isnan(fp8.e4m3_decode([0x7F])[0]) and np.isnan(fp8.e4m3_decode([0xFF])[0])
    assert np.signbit(fp8.e4m3_decode([0x80])[0])


def _finite_codes():
    c = np.arange(256, dtype=np.uint8)
    v = fp8.e4m3_decode(c)
    keep = ~np.isnan(v)
    return c[keep], v[keep]


def test_e4m3_roundtrip_of_every_finite_code():
    c, v = _finite_codes()
    np.testing.assert_array_equal(fp8.e4m3_encode(v), c)


def _brute_force(x):
    """Nearest finite code of the same sign; ties to the even code."""
    c, v = _finite_codes()
    out = []
    for xi in x:
        neg = np.signbit(xi)
        sel = (c >= 0x80) if neg else (c < 0x80)
        cs, vs = c[sel], v[sel]
        dist = np.abs(vs - xi)
        best = np.flatnonzero(dist == dist.min())
        if best.size > 1:
            best = best[(cs[best] & 1) == 0]
        out.append(cs[best[0]])
    return np.array(out, dtype=np.uint8)


def test_e4m3_rounding_matches_brute_force():
    rng = np.random.default_rng(0)
    _, v = _finite_codes()
    pos = np.unique(v[v > 0])
    mids = (pos[:-1] + pos[1:]) / 2  # exact ties (fp32-representable)
    x = np.concatenate([
        rng.uniform(-448, 448, 3000), rng.uniform(-0.05, 0.05, 2000), mids, -mids,
        np.nextafter(mids, 0), np.nextafter(mids, 1e9), [0.0, -0.0, 448.0, -448.0, 2.0 ** -10, 3 * 2.0 ** -10]])
    x = x.astype(np.float32).astype(np.float64)
    x = x[np.abs(x) <= 448]
    np.testing.assert_array_equal(fp8.e4m3_encode(x), _brute_force(x))


def _sylvester(d):
    H = np.array([[1.0]])
    while H.shape[0] < d:
        H = np.block([[H, H], [H, -H]])
    return H


@pytest.mark.parametrize("d", [64, 128])
def test_hadamard_rows_match_the_explicit_matrix(d):
    rng = np.random.default_rng(d)
    x = rng.standard_normal((5, 33, d)).astype(np.float32)
    s = np.where(rng.random(d) < 0.5, -1, 1).astype(np.int8)
    y = fp8.hadamard_rows(x, s)
    ref = (x.astype(np.float64) * s) @ _sylvester(d) / math.sqrt(d)
    # fp32 butterflies: log2(d) roundings of partial sums bounded by sum |x|
    bound = (math.log2(d) + 2) * 2.0 ** -24 * np.abs(x).sum(axis=-1, keepdims=True)
    assert np.all(np.abs(y - ref) <= bound)
    # orthogonal: norms kept and inner products unchanged
    np.testing.assert_allclose(np.linalg.norm(y, axis=-1), np.linalg.norm(x, axis=-1), rtol=1e-5)
    q, k = x[0], x[1]
    np.testing.assert_allclose(fp8.hadamard_rows(q, s) @ fp8.hadamard_rows(k, s).T, q @ k.T, atol=1e-4)


def test_block_scale_is_the_smallest_fitting_power_of_two():
    rng = np.random.default_rng(3)
    for amax in np.concatenate([rng.lognormal(0, 4, 500), [448.0, 448.0 * 2 ** -5, 449.0, 1e-30, 1e30]]):
        e = fp8.block_scale_exponent(amax)
        assert amax <= 448.0 * 2.0 ** e
        assert amax > 448.0 * 2.0 ** (e - 1)
    assert fp8.block_scale_exponent(0.0) == 0
    # the scale stays a normal float32 number
    assert fp8.block_scale_exponent(2.0 ** -126) == -126
    assert fp8.block_scale_exponent(448.0 * 2.0 ** -126) == -126
    assert fp8.block_scale_exponent(448.0 * 2.0 ** -126 * 1.01) == -125


def test_quantize_is_exact_on_representable_blocks():
    # values in {-2..2} with a 2 in every 64-row block: 2^e = 2^-7 and every
    # y / 2^e is in {0, +-128, +-256}, so quantization changes nothing and the
    # FP8 forward equals the plain oracle exactly
    rng = np.random.default_rng(4)
    shape = (1, 2, 150, 128)
    q = rng.integers(-2, 3, shape).astype(np.float32)
    k = rng.integers(-2, 3, shape).astype(np.float32)
    q[..., ::64, 0] = 2
    k[..., ::64, 0] = -2
    v = make_inputs(4, 1, 2, 2, 150, 150, 128).v
    codes, scales = fp8.quantize(q)
    assert np.all(scales == 2.0 ** -7)
    np.testing.assert_array_equal(fp8.dequantize(codes, scales), q)
    O8, L8 = fp8.forward_fp8(q, k, v, 0.05, True)
    O, L = oracle.forward(q, k, v, 0.05, True)
    np.testing.assert_array_equal(O8, O)
    np.testing.assert_array_equal(L8, L)


def test_quantize_error_is_within_half_a_step():
    rng = np.random.default_rng(5)
    x = rng.standard_normal((1, 1, 200, 64)).astype(np.float32)
    codes, scales = fp8.quantize(x)
    err = np.abs(fp8.dequantize(codes, scales) - x)
    # relative half-ulp 2^-4 for normals, absolute 2^-10 * scale in the subnormal range
    rep = np.repeat(scales, 64, axis=-1)[..., :200, None]
    assert np.all(err <= np.maximum(2.0 ** -4 * np.abs(x), 2.0 ** -10 * rep))


def test_incoherent_processing_lowers_the_error_on_outlier_inputs():
    # The page's experiment: N(0,1) Q, K, V with 0.1% of the entries made
    # large; the random-sign Hadamard transform before quantization lowers
    # the error of the FP8 forward (the page reports 2.6x for its setup;
    # with 64-row power-of-two scales and bf16 V the reduction is smaller).
    rng = np.random.default_rng(6)
    shape = (1, 2, 256, 128)

    def draw():
        x = rng.standard_normal(shape).astype(np.float32)
        x[rng.random(shape) < 0.001] *= np.float32(30.0)
        return x

    q, k, v = draw(), draw(), draw()
    s = np.where(rng.random(128) < 0.5, -1, 1).astype(np.int8)
    O, _ = oracle.forward(q, k, v, 0.088, False)
    e_plain = np.sqrt(np.mean((fp8.forward_fp8(q, k, v, 0.088, False)[0] - O) ** 2))
    e_had = np.sqrt(np.mean((fp8.forward_fp8(q, k, v, 0.088, False, s)[0] - O) ** 2))
    assert e_had < e_plain
