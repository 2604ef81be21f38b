"""FP8 (OCP E4M3) quantization with incoherent processing, for the oracle.

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py). Written from the FP8
section of the FlashAttention-3 news page ("Độ chính xác thấp FP8 và
incoherent processing"): Q and K are multiplied by the same random
orthogonal matrix, a Hadamard transform with random signs, before they are
quantized to FP8; since (Q M)(K M)^T = Q K^T, attention is unchanged up to
the quantization, while outlier channels are spread out. The page leaves the
number format, the scaling granularity and the normalisation open; the
readings used here are:

* format: OCP FP8 E4M3 ("E4M3FN"): 1 sign bit, 4 exponent bits with bias 7,
  3 mantissa bits, no infinities, code S.1111.111 is NaN, largest finite
  448, subnormals k * 2^-9;
* rounding: to nearest, ties to even;
* transform: y = FWHT(x o s) / sqrt(d) with the unnormalised Walsh-Hadamard
  transform (Sylvester order), s = +-1 per channel; the quantization decision
  depends on y, so it is taken in the kernel's precision: float32 butterflies
  (a + b, a - b) in stage order h = 1, 2, ..., d/2, then one float32 multiply
  by float32(1/sqrt d);
* scaling: one power-of-two scale 2^e per block of 64 rows of a (batch,
  head), the smallest with max|y| <= 448 * 2^e (so y / 2^e is exact and
  never saturates), kept a normal float32 number: e >= -126, and e = 0
  for an all-zero block; or, "per tensor", one such scale for the whole
  array (the page's baseline of standard FP8 attention, whose scaling the
  page does not state);
* V: quantized the same way but never transformed (the transform is only
  free for Q and K, whose product it leaves unchanged);
* P: the second product can take the probabilities in FP8 too. Reading:
  with the row maximum m, P~ = exp(S - m) lies in (0, 1], and P~ * 2^8 is
  quantized with the same rounding (a fixed power-of-two scale, so the
  largest probability is exactly 1 and values down to 2^-14 keep E4M3's
  3 mantissa bits); the row sum l = sum P~ stays exact (fp64 here), so
  O = (fp8(P~) V) / l and L = m + ln l.

The attention itself is then the plain fp64 definition (oracle.attention) on
the dequantized values decode(code) * 2^e, or, with P in FP8, the same steps
written out with the quantized P~ in the second product.
"""

from __future__ import annotations

import math

import numpy as np

from .attention import forward as _forward

E4M3_MAX = 448.0
BLOCK_ROWS = 64


def e4m3_decode(codes):
    """Value of each E4M3 code (NaN for the two NaN codes), float64."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    exp = (c >> 3) & 0xF
    man = c & 0x7
    val = np.where(exp == 0, man / 8.0 * 2.0 ** -6, (1.0 + man / 8.0) * np.exp2(exp - 7.0))
    val = np.where((exp == 15) & (man == 7), np.nan, val)
    return sign * val


def e4m3_encode(x):
    """E4M3 code of each value (|x| <= 448), round to nearest, ties to even."""
    x = np.asarray(x, dtype=np.float64)
    if np.any(np.abs(x) > E4M3_MAX) or np.any(~np.isfinite(x)):
        raise ValueError("values must be finite with |x| <= 448")
    a = np.abs(x)
    sign = np.signbit(x).astype(np.int64) << 7
    # exponent of the binade (normals) or the subnormal range
    with np.errstate(divide="ignore"):
        E = np.floor(np.log2(np.where(a > 0, a, 1.0))).astype(np.int64)
    E = np.maximum(E, -6)
    # a / 2^(E-3) lies in [8, 16) for normals and [0, 8) for subnormals; the
    # quotient is exact (a is an fp32 value, the divisor a power of two)
    q = np.rint(a / np.exp2(E - 3.0)).astype(np.int64)  # np.rint: half to even
    # q == 16 rounds up into the next binade
    up = q == 16
    E = np.where(up, E + 1, E)
    q = np.where(up, 8, q)
    normal = q >= 8
    mag = np.where(normal, ((E + 7) << 3) | (q - 8), q)
    return (sign | mag).astype(np.uint8)


def hadamard_rows(x, signs):
    """FWHT(x o s) / sqrt(d) along the last axis, in float32 (see module doc)."""
    y = np.array(x, dtype=np.float32, copy=True)
    d = y.shape[-1]
    if d & (d - 1):
        raise ValueError("head_dim must be a power of two")
    y = y * np.asarray(signs, dtype=np.float32)
    h = 1
    while h < d:
        v = y.reshape(y.shape[:-1] + (d // (2 * h), 2, h))
        a, b = v[..., 0, :], v[..., 1, :]
        y = np.stack([a + b, a - b], axis=-2).reshape(y.shape)
        h *= 2
    return y * np.float32(1.0 / math.sqrt(d))


E_MIN = -126  # 2^e stays a normal float32 number


def block_scale_exponent(amax):
    """Smallest e >= -126 with amax <= 448 * 2^e (0 for amax == 0)."""
    amax = float(amax)
    if amax == 0.0:
        return 0
    if amax <= E4M3_MAX * 2.0 ** E_MIN:
        return E_MIN
    e = math.ceil(math.log2(amax / E4M3_MAX))
    # guard the boundary against log2 rounding: step to the exact smallest e
    while amax > E4M3_MAX * 2.0 ** (e - 1):
        e += 1
    while amax <= E4M3_MAX * 2.0 ** (e - 1):
        e -= 1
    return e


def quantize(x, signs=None, per_tensor=False):
    """Codes [..., N, d] (uint8) and block scales [..., ceil(N/64)] (float64
    powers of two) of x [..., N, d] (values exactly representable in fp32).
    per_tensor: one scale for the whole array (repeated in every block)."""
    x = np.asarray(x, dtype=np.float32)
    y = hadamard_rows(x, signs) if signs is not None else x.copy()
    N = y.shape[-2]
    nb = -(-N // BLOCK_ROWS)
    codes = np.empty(y.shape, dtype=np.uint8)
    scales = np.empty(y.shape[:-2] + (nb,))
    e_all = block_scale_exponent(np.max(np.abs(y))) if per_tensor and y.size else None
    for idx in np.ndindex(*y.shape[:-2]):
        for j in range(nb):
            blk = y[idx][j * BLOCK_ROWS:(j + 1) * BLOCK_ROWS].astype(np.float64)
            e = e_all if per_tensor else block_scale_exponent(np.max(np.abs(blk)))
            scales[idx + (j,)] = 2.0 ** e
            codes[idx][j * BLOCK_ROWS:(j + 1) * BLOCK_ROWS] = e4m3_encode(blk / 2.0 ** e)
    return codes, scales


def dequantize(codes, scales):
    """decode(code) * 2^e, float64, [..., N, d]."""
    vals = e4m3_decode(codes)
    N = vals.shape[-2]
    rep = np.repeat(np.asarray(scales, dtype=np.float64), BLOCK_ROWS, axis=-1)[..., :N]
    return vals * rep[..., None]


P_SCALE = 2.0 ** 8  # fixed scale of the probabilities' FP8 codes


def quantize_probs(p):
    """fp8(P~): each probability in [0, 1] as the E4M3 value of P~ * 2^8,
    divided back by 2^8 (float64)."""
    p = np.asarray(p, dtype=np.float64)
    if np.any(p < 0) or np.any(p > 1):
        raise ValueError("probabilities must lie in [0, 1]")
    return e4m3_decode(e4m3_encode(p * P_SCALE)) / P_SCALE


def forward_probs_fp8(q, k, v, scale, causal):
    """Attention with the probabilities rounded to FP8 in the second
    product: per (batch, query head), S = s Q K^T (causal mask -inf),
    m = rowmax S, P~ = exp(S - m), l = sum P~, O = (fp8(P~) V) / l,
    L = m + ln l. q: [B,Hq,Nq,d]; k, v: [B,Hkv,Nk,d]; float64 results."""
    q, k, v = (np.asarray(t, dtype=np.float64) for t in (q, k, v))
    B, Hq, Nq, d = q.shape
    G = Hq // k.shape[1]
    Nk = k.shape[2]
    O = np.empty((B, Hq, Nq, v.shape[-1]))
    L = np.empty((B, Hq, Nq))
    cols = np.arange(Nk)
    for b in range(B):
        for h in range(Hq):
            g = h // G
            for a in range(0, Nq, 256):
                rows = np.arange(a, min(Nq, a + 256))
                S = float(scale) * (q[b, h, rows] @ k[b, g].T)
                if causal:
                    S = np.where(cols[None, :] > rows[:, None], -np.inf, S)
                m = S.max(axis=1)
                Pt = np.exp(S - m[:, None])
                ell = Pt.sum(axis=1)
                O[b, h, rows] = (quantize_probs(Pt) @ v[b, g]) / ell[:, None]
                L[b, h, rows] = m + np.log(ell)
    return O, L


def forward_probs_fp8_online(q, k, v, scale, causal, tile=64, quant=None, rows=None):
    """P in FP8 the way a tiled forward forms it: against the running row
    maximum of the key tiles seen so far (online softmax, page "6.2
    FlashAttention V2 chi tiết", section 6.1), so the rounding is applied to
    exp(S_j - m_j) of each tile j, not to exp(S - m) with the final maximum.
    Key tiles of `tile` keys in order; per query row, with m = -inf, l = 0,
    O = 0:
        S_j = s Q K_j^T (causal mask -inf), m' = max(m, rowmax S_j),
        a = exp(m - m'),  P~_j = exp(S_j - m'),
        O = a O + fp8(P~_j) V_j,  l = a l + rowsum P~_j,  m = m'
    then O / l and L = m + ln l. `quant` replaces fp8 (identity: plain
    attention); `rows` optionally selects query rows (their positions still
    decide the causal mask). q: [B,Hq,Nq,d]; k, v: [B,Hkv,Nk,d]; float64
    results [B, Hq, len(rows) or Nq, ...]."""
    quant = quantize_probs if quant is None else quant
    q, k, v = (np.asarray(t, dtype=np.float64) for t in (q, k, v))
    B, Hq, _, _ = q.shape
    G = Hq // k.shape[1]
    Nk = k.shape[2]
    rows = np.arange(q.shape[2]) if rows is None else np.asarray(rows, dtype=np.int64)
    q = q[:, :, rows]
    Nq = rows.size
    O = np.empty((B, Hq, Nq, v.shape[-1]))
    L = np.empty((B, Hq, Nq))
    for b in range(B):
        for h in range(Hq):
            g = h // G
            m = np.full(Nq, -np.inf)
            ell = np.zeros(Nq)
            acc = np.zeros((Nq, v.shape[-1]))
            for j0 in range(0, Nk, tile):
                cols = np.arange(j0, min(Nk, j0 + tile))
                S = float(scale) * (q[b, h] @ k[b, g, cols].T)
                if causal:
                    S = np.where(cols[None, :] > rows[:, None], -np.inf, S)
                m_new = np.maximum(m, S.max(axis=1))
                seen = m_new > -np.inf  # rows with no visible key yet keep O = 0, l = 0
                alpha = np.where(seen, np.exp(np.where(seen, m - m_new, 0.0)), 1.0)
                Pt = np.where(seen[:, None], np.exp(S - np.where(seen, m_new, 0.0)[:, None]), 0.0)
                acc = alpha[:, None] * acc + quant(Pt) @ v[b, g, cols]
                ell = alpha * ell + Pt.sum(axis=1)
                m = m_new
            O[b, h] = acc / ell[:, None]
            L[b, h] = m + np.log(ell)
    return O, L


def forward_fp8(q, k, v, scale, causal, signs=None, per_tensor=False, v_fp8=False, p_fp8=False):
    """The FP8 forward: quantize Q and K (same signs; 64-row block scales, or
    one scale per tensor), optionally V (never transformed) and P, then the
    fp64 attention of the dequantized values. Returns (O, L)."""
    qc, qs = quantize(q, signs, per_tensor)
    kc, ks = quantize(k, signs, per_tensor)
    vv = dequantize(*quantize(v, None, per_tensor)) if v_fp8 else v
    if p_fp8:
        return forward_probs_fp8(dequantize(qc, qs), dequantize(kc, ks), vv, scale, causal)
    return _forward(dequantize(qc, qs), dequantize(kc, ks), vv, scale, causal)
