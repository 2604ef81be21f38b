"""The FP8 path on the GPU (fa_quantize_fp8 and fa_fwd_fp8 through the C ABI)
against the oracle's FP8 definition (oracle/fp8.py) on the same seeded bf16
inputs and the same random signs.

* Codes and block scales must be bit-exact: the oracle takes every rounding
  decision in the kernel's precision (float32 butterflies, then e4m3 round
  to nearest even of an exact power-of-two quotient).
* O and L of fa_fwd_fp8 must match the oracle's FP8 forward (the plain fp64
  attention of the dequantized Q, K and the bf16 V) within the bounds of the
  bf16 forward, O max-abs 1e-2 and L 1e-3, plus a bound for the one step
  whose precision the hardware fixes: the FP8 matrix instruction sums its 64
  exact products in a fixed-point window anchored at the largest one
  (measured on gfx950: terms 2^-13 below the leading bit of the largest
  product are kept, 2^-14 are dropped), then adds the sum to the fp32
  accumulator. Each of the 64 terms of one instruction is then off by less
  than 2^(E - 12), E = floor(log2 max|product|) (one bit of margin for where
  the window is anchored), so a score is off by at most
  delta_ij = |scale| sq_i sk_j sum over the two 64-channel halves 64 * 2^(E - 12),
  L_i by at most max_j delta_ij and O_i by (exp(2 max_j delta_ij) - 1) max|v|
  (the softmax weights move by at most that factor). On inputs without
  outlier channels the bf16 bounds alone are asserted too.
* On inputs with outlier entries, the transform with random signs lowers
  the error against exact attention (the property the method is for).
"""

import numpy as np
import pytest

import oracle
from oracle import fp8 as ofp8
from exact_tiled_attention_28_amd import binding
from exact_tiled_attention_28_amd.inputs import make_signs, round_to_bf16
from exact_tiled_attention_28_amd.workloads import WORKLOADS
from tests.gpu_util import announce, bf16_half_ulp, gen, host, upload

pytestmark = pytest.mark.gpu


def _bf16_dev(x):
    import torch
    _, bits = round_to_bf16(np.ascontiguousarray(x, dtype=np.float32))
    return torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16).cuda()


def _signs_dev(signs):
    import torch
    return None if signs is None else torch.from_numpy(signs.copy()).cuda()


def window_bound(qc, qs, kc, ks, scale, causal, rows=None):
    """max_j delta_ij (see the module doc) for the query rows `rows` (all by
    default) of one head, over the keys each row sees."""
    qv, kv = ofp8.e4m3_decode(qc), ofp8.e4m3_decode(kc)
    rows = np.arange(qv.shape[0]) if rows is None else np.asarray(rows)
    sq = np.repeat(np.asarray(qs, dtype=np.float64), 64)[rows]
    sk = np.repeat(np.asarray(ks, dtype=np.float64), 64)[:kv.shape[0]]
    out = np.empty(rows.size)
    for n, i in enumerate(rows):
        keys = kv[:i + 1] if causal else kv
        tot = np.zeros(keys.shape[0])
        for c0 in range(0, qv.shape[1], 64):
            p = np.abs(qv[i, c0:c0 + 64] * keys[:, c0:c0 + 64]).max(axis=1)
            e = np.floor(np.log2(np.where(p > 0, p, 1.0)))
            tot += np.where(p > 0, 64 * np.exp2(e - 12), 0.0)
        out[n] = abs(scale) * sq[n] * np.max(tot * sk[:keys.shape[0]])
    return out


def _assert_within(O_got, L_got, O_ref, L_ref, v_absmax, bound, where):
    """O and L of one head (rows x d, rows) within 1e-2 / 1e-3 plus the window
    bound of each row."""
    dl = np.abs(L_got - L_ref)
    do = np.max(np.abs(O_got - O_ref), axis=-1)
    assert np.all(dl <= 1e-3 + bound), f"L {where}: worst excess {np.max(dl - 1e-3 - bound):.3e}"
    assert np.all(do <= 1e-2 + np.expm1(2 * bound) * v_absmax), f"O {where}"


def _quantize_both(x_host, x_dev, signs):
    codes, scales = binding.quantize_fp8(x_dev, _signs_dev(signs))
    oc, osc = ofp8.quantize(x_host, signs)
    return codes.cpu().numpy(), scales.cpu().numpy(), oc, osc


QUANT_CASES = [
    # (B, H, N, d, with signs, outlier channels)
    (2, 3, 200, 128, True, 2),
    (1, 2, 64, 64, True, 0),
    (1, 1, 1, 128, False, 0),
    (2, 2, 130, 64, False, 3),
    (1, 4, 333, 128, True, 0),
]


@pytest.mark.parametrize("case", QUANT_CASES, ids=[f"B{c[0]}H{c[1]}N{c[2]}d{c[3]}{'s' if c[4] else ''}"
                                                   for c in QUANT_CASES])
def test_quantize_fp8_bit_exact(case):
    B, H, N, d, with_signs, outl = case
    announce(f"fa_quantize_fp8 {case}")
    inp = gen(21 + N, B, H, H, N, N, d, outliers=outl)
    q, _, _, _ = upload(inp)
    signs = make_signs(5 + d, d) if with_signs else None
    codes, scales, oc, osc = _quantize_both(inp.q, q, signs)
    np.testing.assert_array_equal(scales, osc.astype(np.float32))
    np.testing.assert_array_equal(codes, oc)


def test_quantize_fp8_ties_subnormals_and_extreme_blocks():
    # No transform, so y = x: block 0 holds 448 (scale 1) with exact ties
    # between e4m3 values and subnormal-range values; block 1 is all zeros
    # (scale 1, codes 0); block 2 is tiny (the scale is clamped at 2^-126);
    # block 3 is huge; block 4 holds a single negative zero row.
    d, N = 64, 4 * 64 + 1
    x = np.zeros((1, 1, N, d), dtype=np.float32)
    ties = np.array([448, 1.0625, 1.1875, -1.0625, 2.0 ** -10, 3 * 2.0 ** -10, -5 * 2.0 ** -10, 2.0 ** -6 + 2.0 ** -10,
                     15 * 2.0 ** -4 + 2.0 ** -5, 240 + 8, 2.0 ** -11, 0.0], dtype=np.float32)
    rng = np.random.default_rng(8)
    x[0, 0, :64] = rng.choice(ties, size=(64, d))
    x[0, 0, 0, 0] = 448.0
    # normal fp32 values with max below 448 * 2^-126 = 1.75 * 2^-118
    mag = rng.uniform(2.0 ** -119, 1.5 * 2.0 ** -118, (64, d)) * rng.choice([-1.0, 1.0], (64, d))
    x[0, 0, 128:192] = mag.astype(np.float32)
    x[0, 0, 192:256] = rng.standard_normal((64, d)).astype(np.float32) * np.float32(1e30)
    x[0, 0, 256] = -0.0
    x = round_to_bf16(x)[0]
    announce("fa_quantize_fp8 ties/subnormals/extreme blocks")
    codes, scales, oc, osc = _quantize_both(x, _bf16_dev(x), None)
    assert osc[0, 0, 0] == 1.0 and osc[0, 0, 1] == 1.0 and osc[0, 0, 2] == 2.0 ** -126
    np.testing.assert_array_equal(scales, osc.astype(np.float32))
    np.testing.assert_array_equal(codes, oc)
    assert np.all(codes[0, 0, 64:128] == 0) and np.all(codes[0, 0, 256] == 0x80)


FWD_CASES = [
    # (B, Hq, Hkv, Nq, Nk, causal, with signs, outlier channels, scale)
    (1, 4, 2, 300, 300, True, True, 4, None),
    (2, 2, 2, 130, 257, False, False, 0, None),
    (1, 2, 1, 1, 1, True, True, 0, None),
    (1, 3, 1, 70, 600, False, True, 0, None),
    (1, 2, 2, 200, 200, True, True, 2, -0.1),
    (1, 2, 1, 64, 64, False, True, 0, 0.0),
    (1, 2, 1, 200, 200, True, True, 0, 0.0),  # zero scale on masked diagonal tiles
    # longer rows: several passes of the six-phase main loop, leaving after
    # phases 1, 4 and 5
    (1, 2, 1, 200, 1000, False, True, 0, None),
    (1, 1, 1, 1100, 1100, True, True, 0, None),
    (1, 2, 2, 100, 448, False, False, 0, None),
]
# head dim 64 (one FP8 product per 32-key block, 64-byte K rows)
FWD_CASES_D64 = [
    (1, 4, 2, 300, 300, True, True, 4, None),
    (2, 2, 2, 130, 257, False, False, 0, None),
    (1, 2, 1, 1, 1, True, True, 0, None),
    (1, 2, 2, 200, 200, True, True, 2, -0.1),
    (1, 1, 1, 1100, 1100, True, True, 0, None),
    (1, 2, 1, 200, 1000, False, True, 0, None),
]
FWD_CASES_ALL = [c + (128,) for c in FWD_CASES] + [c + (64,) for c in FWD_CASES_D64]


def _fwd_id(c):
    return f"B{c[0]}Hq{c[1]}Hkv{c[2]}Nq{c[3]}Nk{c[4]}{'c' if c[5] else 'n'}{'s' if c[6] else ''}o{c[7]}" + \
        ("" if c[8] is None else f"sc{c[8]}") + f"d{c[9]}"


@pytest.mark.parametrize("case", FWD_CASES_ALL, ids=[_fwd_id(c) for c in FWD_CASES_ALL])
def test_fwd_fp8_parity(case):
    import torch
    B, Hq, Hkv, Nq, Nk, causal, with_signs, outl, scale, d = case
    scale = float(np.float32(1 / np.sqrt(d))) if scale is None else scale
    announce(f"fa_fwd_fp8 {_fwd_id(case)}")
    inp = gen(31 + Nq + Nk, B, Hq, Hkv, Nq, Nk, d, outliers=outl)
    q, k, v, _ = upload(inp)
    signs = make_signs(7, d) if with_signs else None
    qc, qs, oqc, oqs = _quantize_both(inp.q, q, signs)
    kc, ks, okc, oks = _quantize_both(inp.k, k, signs)
    np.testing.assert_array_equal(qc, oqc)
    np.testing.assert_array_equal(kc, okc)
    dq_c, dq_s = binding.quantize_fp8(q, _signs_dev(signs))
    dk_c, dk_s = binding.quantize_fp8(k, _signs_dev(signs))
    o32, lse = binding.forward_fp8(dq_c, dq_s, dk_c, dk_s, v, scale, causal, out_dtype=torch.float32)
    o16, lse16 = binding.forward_fp8(dq_c, dq_s, dk_c, dk_s, v, scale, causal, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    O, L = ofp8.forward_fp8(inp.q, inp.k, inp.v, scale, causal, signs)
    O32, L32, O16 = host(o32), host(lse), host(o16)
    err_o = np.max(np.abs(O32 - O))
    err_l = np.max(np.abs(L32 - L))
    worst_bound = 0.0
    for b in range(B):
        for h in range(Hq):
            g = h // (Hq // Hkv)
            bound = window_bound(oqc[b, h], oqs[b, h], okc[b, g], oks[b, g], scale, causal)
            worst_bound = max(worst_bound, float(bound.max()))
            vmax = np.max(np.abs(inp.v[b, g]))
            _assert_within(O32[b, h], L32[b, h], O[b, h], L[b, h], vmax, bound, f"head {(b, h)}")
            assert np.all(np.abs(O16[b, h] - O[b, h]) <= 1e-2 + bf16_half_ulp(O[b, h])
                          + np.expm1(2 * bound)[:, None] * vmax), f"bf16 O head {(b, h)}"
    print(f"max|dO|={err_o:.3e} max|dL|={err_l:.3e} window bound on dS <= {worst_bound:.3e}")
    if outl == 0:
        assert err_o <= 1e-2
        assert err_l <= 1e-3
    assert np.array_equal(host(lse16), L32), "L must not depend on the output dtype"


def _sample_rows(rng, n, count):
    rows = set(rng.choice(n, size=min(n, count), replace=False).tolist())
    rows |= {0, 1, 63, 64, n - 1}
    return np.array(sorted(rows))


def test_fwd_fp8_outlier_workload_full_size():
    # the GQA workload with outlier channels at its full size, in the launch
    # configuration the FP8 benchmark times; sampled heads and rows
    import torch
    w = WORKLOADS["fwd_bf16_causal_gqa_b4_hq32_hkv8_n4096_d128_outliers"]
    announce(f"fa_fwd_fp8 full size {w.name}")
    inp = gen(w.seed, w.batch, w.n_q_heads, w.n_kv_heads, w.seqlen, w.seqlen, w.head_dim,
              outliers=w.n_outlier_channels)
    q, k, v, _ = upload(inp)
    signs = make_signs(w.seed, w.head_dim)
    sd = _signs_dev(signs)
    qc, qs = binding.quantize_fp8(q, sd)
    kc, ks = binding.quantize_fp8(k, sd)
    o, lse = binding.forward_fp8(qc, qs, kc, ks, v, w.scale, w.causal, out_dtype=torch.float32)
    torch.cuda.synchronize()
    O, L = host(o), host(lse)
    rng = np.random.default_rng(99)
    G = w.group
    worst_o = worst_l = 0.0
    for b, h in [(0, 0), (1, 9), (3, w.n_q_heads - 1)]:
        g = h // G
        oqc, oqs = ofp8.quantize(inp.q[b, h], signs)
        okc, oks = ofp8.quantize(inp.k[b, g], signs)
        np.testing.assert_array_equal(qc[b, h].cpu().numpy(), oqc)
        np.testing.assert_array_equal(kc[b, g].cpu().numpy(), okc)
        np.testing.assert_array_equal(qs[b, h].cpu().numpy(), oqs.astype(np.float32))
        rows = _sample_rows(rng, w.seqlen, 48)
        Or, Lr = oracle.forward_head(ofp8.dequantize(oqc, oqs), ofp8.dequantize(okc, oks), inp.v[b, g], w.scale,
                                     w.causal, rows=rows)
        bound = window_bound(oqc, oqs, okc, oks, w.scale, w.causal, rows)
        _assert_within(O[b, h][rows], L[b, h][rows], Or, Lr, np.max(np.abs(inp.v[b, g])), bound, f"head {(b, h)}")
        worst_o = max(worst_o, np.max(np.abs(O[b, h][rows] - Or)))
        worst_l = max(worst_l, np.max(np.abs(L[b, h][rows] - Lr)))
    print(f"{w.name} fp8: max|dO|={worst_o:.3e} max|dL|={worst_l:.3e}")
    assert np.all(np.isfinite(O)) and np.all(np.isfinite(L))


def test_fwd_fp8_incoherent_processing_lowers_the_error():
    # N(0,1) Q, K, V with 0.1% of the entries scaled by 30; the error of the
    # FP8 forward against exact attention, with and without the transform
    import torch
    rng = np.random.default_rng(6)
    shape = (1, 4, 512, 128)

    def draw():
        x = rng.standard_normal(shape).astype(np.float32)
        x[rng.random(shape) < 0.001] *= np.float32(30.0)
        return round_to_bf16(x)[0]

    qh, kh, vh = draw(), draw(), draw()
    q, k, v = _bf16_dev(qh), _bf16_dev(kh), _bf16_dev(vh)
    scale = float(np.float32(1 / np.sqrt(128)))
    O_exact, _ = oracle.forward(qh, kh, vh, scale, False)
    errs = {}
    for name, signs in (("plain", None), ("hadamard", make_signs(17, 128))):
        announce(f"fa_fwd_fp8 outlier error, {name}")
        sd = _signs_dev(signs)
        qc, qs = binding.quantize_fp8(q, sd)
        kc, ks = binding.quantize_fp8(k, sd)
        o, _ = binding.forward_fp8(qc, qs, kc, ks, v, scale, False, out_dtype=torch.float32)
        torch.cuda.synchronize()
        errs[name] = float(np.sqrt(np.mean((host(o) - O_exact) ** 2)))
    print(f"rmse plain={errs['plain']:.4e} hadamard={errs['hadamard']:.4e} ratio={errs['plain'] / errs['hadamard']:.3f}")
    assert errs["hadamard"] < errs["plain"]


# --- P V in FP8 (fa_quantize_vt_fp8, fa_fwd_fp8_pv) -------------------------

def _vt_key_of(pos):
    g, s = pos >> 5, pos & 31
    return 32 * (s >> 4) + 8 * ((s & 15) >> 2) + 4 * g + (s & 3)


def _untranspose_vt(vt, N):
    """[..., nb, d, 64] transposed codes -> [..., N, d] (keys in order)."""
    *lead, nb, d, _ = vt.shape
    keys = np.array([_vt_key_of(p) for p in range(64)])
    out = np.zeros(tuple(lead) + (nb * 64, d), dtype=vt.dtype)
    for j in range(nb):
        out[..., j * 64 + keys, :] = np.swapaxes(vt[..., j, :, :], -1, -2)
    return out[..., :N, :], out[..., N:, :]


VT_CASES = [(2, 3, 200, 128, 0), (1, 2, 64, 64, 0), (1, 1, 1, 128, 0), (2, 2, 130, 64, 3), (1, 4, 333, 128, 2)]


@pytest.mark.parametrize("case", VT_CASES, ids=[f"B{c[0]}H{c[1]}N{c[2]}d{c[3]}o{c[4]}" for c in VT_CASES])
def test_quantize_vt_fp8_bit_exact(case):
    B, H, N, d, outl = case
    announce(f"fa_quantize_vt_fp8 {case}")
    inp = gen(51 + N, B, H, H, N, N, d, outliers=outl)
    _, _, v, _ = upload(inp)
    vt, vs = binding.quantize_vt_fp8(v)
    codes, tail = _untranspose_vt(vt.cpu().numpy(), N)
    oc, osc = ofp8.quantize(inp.v)
    np.testing.assert_array_equal(vs.cpu().numpy(), osc.astype(np.float32))
    np.testing.assert_array_equal(codes, oc)
    assert np.all(tail == 0), "keys past the end must get code 0"


def test_quantize_vt_fp8_ties_subnormals_and_extreme_blocks():
    # the blocks of the Q/K quantize test, now as V (no transform either way)
    d, N = 64, 4 * 64 + 1
    x = np.zeros((1, 1, N, d), dtype=np.float32)
    ties = np.array([448, 1.0625, 1.1875, -1.0625, 2.0 ** -10, 3 * 2.0 ** -10, -5 * 2.0 ** -10, 2.0 ** -6 + 2.0 ** -10,
                     15 * 2.0 ** -4 + 2.0 ** -5, 240 + 8, 2.0 ** -11, 0.0], dtype=np.float32)
    rng = np.random.default_rng(9)
    x[0, 0, :64] = rng.choice(ties, size=(64, d))
    x[0, 0, 0, 0] = 448.0
    mag = rng.uniform(2.0 ** -119, 1.5 * 2.0 ** -118, (64, d)) * rng.choice([-1.0, 1.0], (64, d))
    x[0, 0, 128:192] = mag.astype(np.float32)
    x[0, 0, 192:256] = rng.standard_normal((64, d)).astype(np.float32) * np.float32(1e30)
    x[0, 0, 256] = -0.0
    x = round_to_bf16(x)[0]
    announce("fa_quantize_vt_fp8 ties/subnormals/extreme blocks")
    vt, vs = binding.quantize_vt_fp8(_bf16_dev(x))
    codes, _ = _untranspose_vt(vt.cpu().numpy(), N)
    oc, osc = ofp8.quantize(x)
    np.testing.assert_array_equal(vs.cpu().numpy(), osc.astype(np.float32))
    np.testing.assert_array_equal(codes, oc)


def _pv_bounds(qv, kv, vv, vc, vs, scale, causal, delta, tile=64, rows=None):
    """Per query row of one head: the flip bound (codes of P that the kernel
    may round the other way, since its P carries the relative error
    e^(2 delta) - 1 of its scores plus fp32 rounding) and the window bound of
    the FP8 P V products (64 terms each, every term off by less than
    2^(E - 12), E = floor(log2 max |term|)), both in units of O, and the
    largest |V|. qv, kv, vv: dequantized Q, K, V (one head); vc, vs: V codes
    [Nk, d] and block scales; delta: the score bound of each row."""
    rows = np.arange(qv.shape[0]) if rows is None else np.asarray(rows)
    qv = qv[rows]
    Nq, Nk = qv.shape[0], kv.shape[0]
    S = scale * (qv @ kv.T)
    if causal:
        S = np.where(np.arange(Nk)[None, :] > rows[:, None], -np.inf, S)
    m_fin = S.max(axis=1)
    ell = np.exp(S - m_fin[:, None]).sum(axis=1)
    vdec = ofp8.e4m3_decode(vc)  # V / 2^e
    flip = np.zeros(Nq)
    win = np.zeros(Nq)
    m = np.full(Nq, -np.inf)
    eps = np.expm1(2 * delta) + 2.0 ** -20
    for t, j0 in enumerate(range(0, Nk, tile)):
        cols = slice(j0, min(Nk, j0 + tile))
        St = S[:, cols]
        m = np.maximum(m, St.max(axis=1))
        seen = m > -np.inf
        Pt = np.where(seen[:, None], np.exp(St - np.where(seen, m, 0.0)[:, None]), 0.0) * 256.0  # kernel's P 2^8
        w = np.where(seen, np.exp(np.where(seen, m - m_fin, 0.0)), 0.0) / ell  # weight of this tile in O
        code = ofp8.e4m3_encode(np.clip(Pt, 0, 448))
        val = ofp8.e4m3_decode(code)
        lo = ofp8.e4m3_decode(np.maximum(code.astype(np.int64) - 1, 0).astype(np.uint8))
        hi = ofp8.e4m3_decode(np.minimum(code.astype(np.int64) + 1, 0x7E).astype(np.uint8))
        # distance to the nearer midpoint, relative to P
        near = np.minimum(np.abs(Pt - (val + lo) / 2), np.abs(Pt - (val + hi) / 2)) <= eps[:, None] * Pt
        step = np.maximum(val - lo, hi - val) / 256.0
        vabs = np.abs(vv[cols]).max(axis=1)
        flip += w * (near * step * vabs[None, :]).sum(axis=1)
        # window of the FP8 product: terms P code x V code, per channel
        terms = np.abs(val[:, :, None] * vdec[cols][None, :, :])  # [Nq, keys, d]
        tmax = terms.max(axis=1)
        E = np.floor(np.log2(np.where(tmax > 0, tmax, 1.0)))
        per_c = np.where(tmax > 0, terms.shape[1] * np.exp2(E - 12), 0.0)  # [Nq, d]
        win += w * per_c.max(axis=1) * vs[t] / 256.0
    return flip, win


PV_CASES = [
    # (B, Hq, Hkv, Nq, Nk, causal, with signs, outlier channels, scale, d)
    (1, 4, 2, 300, 300, True, True, 4, None, 128),
    (2, 2, 2, 130, 257, False, False, 0, None, 128),
    (1, 2, 1, 1, 1, True, True, 0, None, 128),
    (1, 2, 2, 200, 200, True, True, 2, -0.1, 128),
    (1, 2, 1, 64, 64, False, True, 0, 0.0, 128),
    (1, 1, 1, 1100, 1100, True, True, 0, None, 128),
    (1, 4, 2, 300, 300, True, True, 4, None, 64),
    (2, 2, 2, 130, 257, False, False, 0, None, 64),
    (1, 2, 1, 200, 1000, False, True, 0, None, 64),
]


@pytest.mark.parametrize("case", PV_CASES, ids=[_fwd_id(c) for c in PV_CASES])
def test_fwd_fp8_pv_parity(case):
    # against the oracle's tiled P-in-FP8 forward on the dequantized Q, K, V,
    # within the bf16 forward's bounds plus: the score window bound (as for
    # fa_fwd_fp8), the codes of P that a score that far off can round the
    # other way, and the window of the FP8 P V products
    import torch
    B, Hq, Hkv, Nq, Nk, causal, with_signs, outl, scale, d = case
    scale = float(np.float32(1 / np.sqrt(d))) if scale is None else scale
    announce(f"fa_fwd_fp8_pv {_fwd_id(case)}")
    inp = gen(61 + Nq + Nk, B, Hq, Hkv, Nq, Nk, d, outliers=outl)
    q, k, v, _ = upload(inp)
    signs = make_signs(7, d) if with_signs else None
    dq_c, dq_s = binding.quantize_fp8(q, _signs_dev(signs))
    dk_c, dk_s = binding.quantize_fp8(k, _signs_dev(signs))
    vt, vs = binding.quantize_vt_fp8(v)
    o32, lse = binding.forward_fp8_pv(dq_c, dq_s, dk_c, dk_s, vt, vs, scale, causal, out_dtype=torch.float32)
    o16, lse16 = binding.forward_fp8_pv(dq_c, dq_s, dk_c, dk_s, vt, vs, scale, causal, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    oqc, oqs = ofp8.quantize(inp.q, signs)
    okc, oks = ofp8.quantize(inp.k, signs)
    ovc, ovs = ofp8.quantize(inp.v)
    qd, kd, vd = ofp8.dequantize(oqc, oqs), ofp8.dequantize(okc, oks), ofp8.dequantize(ovc, ovs)
    O, L = ofp8.forward_probs_fp8_online(qd, kd, vd, scale, causal, tile=64)
    O32, L32, O16 = host(o32), host(lse), host(o16)
    worst = (0.0, 0.0, 0.0)
    for b in range(B):
        for h in range(Hq):
            g = h // (Hq // Hkv)
            delta = window_bound(oqc[b, h], oqs[b, h], okc[b, g], oks[b, g], scale, causal)
            flip, win = _pv_bounds(qd[b, h], kd[b, g], vd[b, g], ovc[b, g], ovs[b, g], scale, causal, delta)
            vmax = np.max(np.abs(vd[b, g]))
            dl = np.abs(L32[b, h] - L[b, h])
            do = np.max(np.abs(O32[b, h] - O[b, h]), axis=-1)
            assert np.all(dl <= 1e-3 + delta), f"L head {(b, h)}"
            bound_o = 1e-2 + np.expm1(2 * delta) * vmax + flip + win
            assert np.all(do <= bound_o), f"O head {(b, h)}: worst excess {np.max(do - bound_o):.3e}"
            assert np.all(np.abs(O16[b, h] - O[b, h]) <= bound_o[:, None] + bf16_half_ulp(O[b, h])), f"bf16 O {(b, h)}"
            worst = (max(worst[0], float(do.max())), max(worst[1], float(dl.max())), max(worst[2], float((flip + win).max())))
    print(f"max|dO|={worst[0]:.3e} max|dL|={worst[1]:.3e} flip+window bound <= {worst[2]:.3e}")
    if outl == 0:
        assert worst[0] <= 1e-2 and worst[1] <= 1e-3
    assert np.array_equal(host(lse16), L32), "L must not depend on the output dtype"


def test_fwd_fp8_pv_outlier_workload_full_size():
    # the GQA workload with outlier channels at full size through the FP8 P V
    # path; sampled heads and rows against the oracle's tiled P-in-FP8
    # forward, within the same bounds as the small cases
    import torch
    w = WORKLOADS["fwd_bf16_causal_gqa_b4_hq32_hkv8_n4096_d128_outliers"]
    announce(f"fa_fwd_fp8_pv full size {w.name}")
    inp = gen(w.seed, w.batch, w.n_q_heads, w.n_kv_heads, w.seqlen, w.seqlen, w.head_dim,
              outliers=w.n_outlier_channels)
    q, k, v, _ = upload(inp)
    signs = make_signs(w.seed, w.head_dim)
    sd = _signs_dev(signs)
    qc, qs = binding.quantize_fp8(q, sd)
    kc, ks = binding.quantize_fp8(k, sd)
    vt, vs = binding.quantize_vt_fp8(v)
    o, lse = binding.forward_fp8_pv(qc, qs, kc, ks, vt, vs, w.scale, w.causal, out_dtype=torch.float32)
    torch.cuda.synchronize()
    O, L = host(o), host(lse)
    assert np.all(np.isfinite(O)) and np.all(np.isfinite(L))
    rng = np.random.default_rng(98)
    worst_o = worst_l = 0.0
    for b, h in [(0, 0), (2, 17), (3, w.n_q_heads - 1)]:
        g = h // w.group
        oqc, oqs = ofp8.quantize(inp.q[b, h], signs)
        okc, oks = ofp8.quantize(inp.k[b, g], signs)
        ovc, ovs = ofp8.quantize(inp.v[b, g])
        codes, _ = _untranspose_vt(vt[b, g].cpu().numpy()[None, None], w.seqlen)
        np.testing.assert_array_equal(codes[0, 0], ovc)
        rows = _sample_rows(rng, w.seqlen, 48)
        qd, kd, vd = ofp8.dequantize(oqc, oqs), ofp8.dequantize(okc, oks), ofp8.dequantize(ovc, ovs)
        Or, Lr = ofp8.forward_probs_fp8_online(qd[None, None], kd[None, None], vd[None, None], w.scale, w.causal,
                                               rows=rows)
        delta = window_bound(oqc, oqs, okc, oks, w.scale, w.causal, rows)
        flip, win = _pv_bounds(qd, kd, vd, ovc, ovs, w.scale, w.causal, delta, rows=rows)
        dl = np.abs(L[b, h][rows] - Lr[0, 0])
        do = np.max(np.abs(O[b, h][rows] - Or[0, 0]), axis=-1)
        assert np.all(dl <= 1e-3 + delta), f"L head {(b, h)}"
        assert np.all(do <= 1e-2 + np.expm1(2 * delta) * np.max(np.abs(vd)) + flip + win), f"O head {(b, h)}"
        worst_o, worst_l = max(worst_o, float(do.max())), max(worst_l, float(dl.max()))
    print(f"{w.name} fp8 P V: max|dO|={worst_o:.3e} max|dL|={worst_l:.3e}")


# fa_fwd_fp8_quantize_q: Q in bf16, quantized inside the forward
QQ_CASES = [
    # (B, Hq, Hkv, Nq, Nk, causal, with signs, outlier channels, scale, d, P V in FP8)
    (1, 4, 2, 300, 300, True, True, 4, None, 128, False),
    (2, 2, 2, 130, 257, False, False, 0, None, 128, False),
    (1, 2, 1, 1, 1, True, True, 0, None, 128, True),
    (1, 2, 2, 200, 200, True, True, 2, -0.1, 128, True),
    (1, 3, 1, 70, 600, False, True, 0, None, 64, False),
    (1, 4, 2, 300, 300, True, True, 4, None, 64, True),
    (1, 1, 1, 1100, 1100, True, True, 0, None, 128, True),
    (2, 2, 2, 130, 257, False, False, 0, 0.0, 64, True),
]


def _qq_id(c):
    return _fwd_id(c[:10]) + ("pv8" if c[10] else "")


def _two_pass_and_fused(inp, q, k, v, signs, scale, causal, pv8, out_dtype):
    sd = _signs_dev(signs)
    qc, qs = binding.quantize_fp8(q, sd)
    kc, ks = binding.quantize_fp8(k, sd)
    if pv8:
        vt, vs = binding.quantize_vt_fp8(v)
        ref = binding.forward_fp8_pv(qc, qs, kc, ks, vt, vs, scale, causal, out_dtype=out_dtype)
        got = binding.forward_fp8_quantize_q(q, kc, ks, vt, scale, causal, signs=sd, v_scales=vs, out_dtype=out_dtype)
    else:
        ref = binding.forward_fp8(qc, qs, kc, ks, v, scale, causal, out_dtype=out_dtype)
        got = binding.forward_fp8_quantize_q(q, kc, ks, v, scale, causal, signs=sd, out_dtype=out_dtype)
    return ref, got


@pytest.mark.parametrize("case", QQ_CASES, ids=[_qq_id(c) for c in QQ_CASES])
def test_fwd_fp8_quantize_q_equals_two_passes(case):
    # the same codes, scales and products as fa_quantize_fp8(Q) followed by
    # fa_fwd_fp8 / fa_fwd_fp8_pv (whose parity with the oracle the tests
    # above establish), so O (fp32 and bf16) and L agree bit for bit
    import torch
    B, Hq, Hkv, Nq, Nk, causal, with_signs, outl, scale, d, pv8 = case
    scale = float(np.float32(1 / np.sqrt(d))) if scale is None else scale
    announce(f"fa_fwd_fp8_quantize_q {_qq_id(case)}")
    inp = gen(71 + Nq + Nk, B, Hq, Hkv, Nq, Nk, d, outliers=outl)
    q, k, v, _ = upload(inp)
    signs = make_signs(9, d) if with_signs else None
    for od in (torch.float32, torch.bfloat16):
        (o_ref, l_ref), (o, l) = _two_pass_and_fused(inp, q, k, v, signs, scale, causal, pv8, od)
        torch.cuda.synchronize()
        assert torch.equal(o, o_ref), f"O ({od}) differs from the two-pass path"
        assert torch.equal(l, l_ref), f"L ({od}) differs from the two-pass path"


def test_fwd_fp8_quantize_q_against_the_oracle():
    # one case straight against the oracle's FP8 forward (bf16 V), as
    # test_fwd_fp8_parity does for the two-pass path
    import torch
    B, Hq, Hkv, Nq, Nk, d, causal = 1, 4, 2, 300, 300, 128, True
    scale = float(np.float32(1 / np.sqrt(d)))
    announce("fa_fwd_fp8_quantize_q against the oracle")
    inp = gen(77, B, Hq, Hkv, Nq, Nk, d)
    q, k, v, _ = upload(inp)
    signs = make_signs(9, d)
    sd = _signs_dev(signs)
    kc, ks = binding.quantize_fp8(k, sd)
    o, l = binding.forward_fp8_quantize_q(q, kc, ks, v, scale, causal, signs=sd, out_dtype=torch.float32)
    torch.cuda.synchronize()
    O, L = ofp8.forward_fp8(inp.q, inp.k, inp.v, scale, causal, signs)
    oqc, oqs = ofp8.quantize(inp.q, signs)
    okc, oks = ofp8.quantize(inp.k, signs)
    O32, L32 = host(o), host(l)
    for b in range(B):
        for h in range(Hq):
            g = h // (Hq // Hkv)
            bound = window_bound(oqc[b, h], oqs[b, h], okc[b, g], oks[b, g], scale, causal)
            _assert_within(O32[b, h], L32[b, h], O[b, h], L[b, h], np.max(np.abs(inp.v[b, g])), bound, f"head {(b, h)}")
    assert np.max(np.abs(O32 - O)) <= 1e-2
    assert np.max(np.abs(L32 - L)) <= 1e-3


@pytest.mark.parametrize("pv8", [False, True])
def test_fwd_fp8_quantize_q_full_size(pv8):
    # the 2K-key causal workload at full size (B8 H16 d128), both V paths:
    # bit for bit equal to the two passes
    import torch
    w = WORKLOADS["fwd_bf16_causal_b8_h16_n2048_d128"]
    announce(f"fa_fwd_fp8_quantize_q full size {w.name} pv8={pv8}")
    inp = gen(w.seed, w.batch, w.n_q_heads, w.n_kv_heads, w.seqlen, w.seqlen, w.head_dim)
    q, k, v, _ = upload(inp)
    signs = make_signs(w.seed, w.head_dim)
    (o_ref, l_ref), (o, l) = _two_pass_and_fused(inp, q, k, v, signs, w.scale, w.causal, pv8, torch.bfloat16)
    torch.cuda.synchronize()
    assert torch.equal(o, o_ref) and torch.equal(l, l_ref)
