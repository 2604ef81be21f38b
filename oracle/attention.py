"""Plain fp64 CPU oracle for exact scaled-dot-product attention.

TEST INFRASTRUCTURE ONLY. Nothing in the library imports this module; only the
tests, the smoke check and the CPU-baseline leg of the benchmark use it. It
shares no code with the HIP kernels.

The tiled FlashAttention-2 method reaches the plain definition exactly (up to
rounding order): the FlashAttention-3 news page ("Ôn lại cách FlashAttention
hoạt động") states that tiling with softmax rescaling gives the correct output
with no approximation. So this oracle is the plain definition, written out in
float64, with no tiling, no online rescaling and no fusion:

forward, per (batch, query head), with h_kv = h_q // (Hq / Hkv)
    S = s * Q K^T                                   (page "6.2 FlashAttention V2
                                                     chi tiết", section 6.1)
    S[i, j] = -inf for j > i when causal            (same page, section 5.1)
    m_i = max_j S_ij,  l_i = sum_j exp(S_ij - m_i)
    L_i = m_i + ln l_i                              (section 6.1 and 7.1; CSDN
                                                     FlashAttention-2 article,
                                                     "使用logsumexp简化存储")
    P = exp(S - L 1^T),  O = P V

backward (CSDN FlashAttention-2 article, "3.1.2 反向传播公式解析"):
    dP = dO V^T
    D_i = sum_c dO_ic O_ic                          (page 6.2, section 7.3)
    dS = P o (dP - D 1^T)
    dQ = s * dS K,  dK = s * dS^T Q,  dV = P^T dO
    and for grouped-query attention dK, dV are summed over the query heads
    sharing one K/V head (CSDN article, "多查询注意力和分组查询注意力").

Readings where the pages are silent or garbled:

* the backward formulas on the CSDN page write S = Q K^T without the scale;
  the forward scales by 1/sqrt(d), so by the chain rule the scale s multiplies
  dQ and dK (pinned by finite differences);
* masked scores are -inf (the page's mask value is lost in extraction; only
  "becomes 0 after softmax" survives);
* causal attention is defined only for equal query and key lengths here;
* the scale is whatever float32 value the caller passes, widened to float64.

Inputs may be any real dtype; they are converted to float64 first. Rows are
processed in blocks only to bound memory; every row is computed from the whole
row of scores, so blocking changes nothing.
"""

from __future__ import annotations

import numpy as np

_NEG_INF = -np.inf


def _as64(x):
    return np.asarray(x, dtype=np.float64)


def _check_shapes(q, k, v, causal):
    if q.ndim != 4 or k.ndim != 4 or v.ndim != 4:
        raise ValueError("q, k, v must be [B, H, N, d]")
    B, Hq, Nq, d = q.shape
    Bk, Hkv, Nk, dk = k.shape
    if (Bk, dk) != (B, d) or v.shape != k.shape:
        raise ValueError("k and v must be [B, Hkv, Nk, d] matching q")
    if Hq % Hkv:
        raise ValueError("n_q_heads must be a multiple of n_kv_heads")
    if causal and Nq != Nk:
        raise ValueError("causal attention needs seqlen_q == seqlen_k")
    return B, Hq, Hkv, Nq, Nk, d


def _scores(q_rows, row_idx, kh, s, causal):
    """s * q_rows kh^T with the causal mask applied (row_idx are the absolute
    query positions of q_rows)."""
    S = s * (q_rows @ kh.T)
    if causal:
        cols = np.arange(kh.shape[0])
        S = np.where(cols[None, :] > row_idx[:, None], _NEG_INF, S)
    return S


def forward_head(qh, kh, vh, scale, causal, rows=None, row_block=256):
    """O and L for one query head against its K/V head.

    qh: [Nq, d]; kh, vh: [Nk, d]. ``rows`` optionally selects query rows.
    Returns (O [n, d], L [n]) in float64.
    """
    qh, kh, vh = _as64(qh), _as64(kh), _as64(vh)
    s = float(scale)
    idx = np.arange(qh.shape[0]) if rows is None else np.asarray(rows, dtype=np.int64)
    O = np.empty((idx.size, vh.shape[1]))
    L = np.empty(idx.size)
    for a in range(0, idx.size, row_block):
        r = idx[a:a + row_block]
        S = _scores(qh[r], r, kh, s, causal)
        m = S.max(axis=1)
        ell = np.exp(S - m[:, None]).sum(axis=1)
        Lb = m + np.log(ell)
        P = np.exp(S - Lb[:, None])
        O[a:a + r.size] = P @ vh
        L[a:a + r.size] = Lb
    return O, L


def forward(q, k, v, scale, causal):
    """Exact attention forward. q: [B,Hq,Nq,d]; k, v: [B,Hkv,Nk,d].

    Returns (O [B,Hq,Nq,d], L [B,Hq,Nq]) in float64, L in natural log.
    """
    q, k, v = _as64(q), _as64(k), _as64(v)
    B, Hq, Hkv, Nq, Nk, d = _check_shapes(q, k, v, causal)
    G = Hq // Hkv
    O = np.empty((B, Hq, Nq, d))
    L = np.empty((B, Hq, Nq))
    for b in range(B):
        for h in range(Hq):
            g = h // G
            O[b, h], L[b, h] = forward_head(q[b, h], k[b, g], v[b, g], scale, causal)
    return O, L


def row_dot(do, o):
    """D = rowsum(dO o O), the backward preprocess vector (page 6.2,
    section 7.3). Works on any leading shape; sums the last axis."""
    return (_as64(do) * _as64(o)).sum(axis=-1)


def backward_head(qh, kh, vh, doh, scale, causal, row_block=256):
    """Gradients of one query head against its K/V head.

    Returns (dQ [Nq,d], dK [Nk,d], dV [Nk,d]) in float64. The forward O and L
    are computed here from the plain definition.
    """
    qh, kh, vh, doh = _as64(qh), _as64(kh), _as64(vh), _as64(doh)
    s = float(scale)
    Nq = qh.shape[0]
    dQ = np.empty_like(qh)
    dK = np.zeros_like(kh)
    dV = np.zeros_like(vh)
    for a in range(0, Nq, row_block):
        r = np.arange(a, min(Nq, a + row_block))
        S = _scores(qh[r], r, kh, s, causal)
        m = S.max(axis=1)
        Lb = m + np.log(np.exp(S - m[:, None]).sum(axis=1))
        P = np.exp(S - Lb[:, None])
        Ob = P @ vh
        dP = doh[r] @ vh.T
        D = row_dot(doh[r], Ob)
        dS = P * (dP - D[:, None])
        dQ[r] = s * (dS @ kh)
        dK += s * (dS.T @ qh[r])
        dV += P.T @ doh[r]
    return dQ, dK, dV


def backward(q, k, v, do, scale, causal):
    """Exact attention gradients for upstream gradient dO.

    Returns (dQ [B,Hq,Nq,d], dK [B,Hkv,Nk,d], dV [B,Hkv,Nk,d]) in float64;
    dK and dV are summed over the query heads that share each K/V head.
    """
    q, k, v, do = _as64(q), _as64(k), _as64(v), _as64(do)
    B, Hq, Hkv, Nq, Nk, d = _check_shapes(q, k, v, causal)
    G = Hq // Hkv
    dQ = np.empty_like(q)
    dK = np.zeros_like(k)
    dV = np.zeros_like(v)
    for b in range(B):
        for h in range(Hq):
            g = h // G
            dq, dk, dv = backward_head(q[b, h], k[b, g], v[b, g], do[b, h], scale, causal)
            dQ[b, h] = dq
            dK[b, g] += dk
            dV[b, g] += dv
    return dQ, dK, dV


def probabilities_head(qh, kh, scale, causal):
    """The full softmax matrix P = exp(S - L) of one head (small inputs only)."""
    qh, kh = _as64(qh), _as64(kh)
    r = np.arange(qh.shape[0])
    S = _scores(qh, r, kh, float(scale), causal)
    m = S.max(axis=1)
    L = m + np.log(np.exp(S - m[:, None]).sum(axis=1))
    return np.exp(S - L[:, None])
