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


def backward_dq_rows(qh, kh, vh, doh, scale, causal, rows, row_block=64):
    """dQ for the query rows ``rows`` of one head (page 6.2, section 7; CSDN
    article, 3.1.2): every quantity of row i is local to that row, so
    P_i = exp(S_i - L_i), O_i = P_i V, D_i = dO_i . O_i, dP_i = dO_i V^T,
    dS_i = P_i o (dP_i - D_i) and dQ_i = s dS_i K need only row i of Q and dO
    and all of K and V. Returns dQ [n, d] in float64 (for long sequences,
    where the full backward is out of reach)."""
    qh, kh, vh, doh = _as64(qh), _as64(kh), _as64(vh), _as64(doh)
    s = float(scale)
    idx = np.asarray(rows, dtype=np.int64)
    dQ = np.empty((idx.size, qh.shape[1]))
    for a in range(0, idx.size, row_block):
        r = idx[a:a + row_block]
        S = _scores(qh[r], r, kh, s, causal)
        m = S.max(axis=1)
        Lb = m + np.log(np.exp(S - m[:, None]).sum(axis=1))
        P = np.exp(S - Lb[:, None])
        D = row_dot(doh[r], P @ vh)
        dS = P * (doh[r] @ vh.T - D[:, None])
        dQ[a:a + r.size] = s * (dS @ kh)
    return dQ


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


# ---------------------------------------------------------------------------
# packed variable-length batches
# ---------------------------------------------------------------------------
#
# A batch of sequences of different lengths packed along the row axis (the
# variable-length batches of the FlashAttention-3 news page): sequence b owns
# query rows cu_q[b]..cu_q[b+1]-1 and key rows cu_k[b]..cu_k[b+1]-1, and
# each sequence is attended on its own with the definition above. Arrays are
# [H, total, d] (L: [H, total]). Reading where the pages are silent: a
# sequence with queries but no keys has no softmax at all; its rows get
# O = 0, L = -inf (the logsumexp of an empty set) and dQ = 0.

def _spans(cu):
    cu = np.asarray(cu, dtype=np.int64)
    if cu.ndim != 1 or cu.size < 2 or cu[0] != 0 or np.any(np.diff(cu) < 0):
        raise ValueError("cu_seqlens must be non-decreasing offsets starting at 0")
    return [(int(cu[b]), int(cu[b + 1])) for b in range(cu.size - 1)]


def forward_varlen(q, k, v, cu_q, cu_k, scale, causal):
    """q: [Hq, total_q, d]; k, v: [Hkv, total_k, d]. Returns (O, L) float64."""
    q, k, v = _as64(q), _as64(k), _as64(v)
    Hq, Hkv = q.shape[0], k.shape[0]
    if Hq % Hkv:
        raise ValueError("n_q_heads must be a multiple of n_kv_heads")
    G = Hq // Hkv
    sq, sk = _spans(cu_q), _spans(cu_k)
    if len(sq) != len(sk):
        raise ValueError("cu_seqlens_q and cu_seqlens_k must describe the same number of sequences")
    O = np.zeros(q.shape)
    L = np.full(q.shape[:2], _NEG_INF)
    for (q0, q1), (k0, k1) in zip(sq, sk):
        if q1 == q0 or k1 == k0:
            continue
        if causal and q1 - q0 != k1 - k0:
            raise ValueError("causal attention needs equal query and key lengths per sequence")
        for h in range(Hq):
            O[h, q0:q1], L[h, q0:q1] = forward_head(q[h, q0:q1], k[h // G, k0:k1], v[h // G, k0:k1], scale, causal)
    return O, L


def backward_varlen(q, k, v, do, cu_q, cu_k, scale, causal):
    """Gradients of forward_varlen. Returns (dQ, dK, dV) float64; dK, dV are
    summed over the query heads sharing each K/V head."""
    q, k, v, do = _as64(q), _as64(k), _as64(v), _as64(do)
    Hq, Hkv = q.shape[0], k.shape[0]
    G = Hq // Hkv
    sq, sk = _spans(cu_q), _spans(cu_k)
    dQ = np.zeros(q.shape)
    dK = np.zeros(k.shape)
    dV = np.zeros(v.shape)
    for (q0, q1), (k0, k1) in zip(sq, sk):
        if q1 == q0 or k1 == k0:
            continue
        if causal and q1 - q0 != k1 - k0:
            raise ValueError("causal attention needs equal query and key lengths per sequence")
        for h in range(Hq):
            g = h // G
            dq, dk, dv = backward_head(q[h, q0:q1], k[g, k0:k1], v[g, k0:k1], do[h, q0:q1], scale, causal)
            dQ[h, q0:q1] = dq
            dK[g, k0:k1] += dk
            dV[g, k0:k1] += dv
    return dQ, dK, dV
