"""Checks that pin the CPU oracle to facts fixed by the pages and by the
mathematics, independent of the oracle's own formulas.

Every pin takes the oracle module as an argument so that the same checks can
be run against deliberately broken copies of the oracle (see
test_oracle_mutants.py): each plausible mistake must fail at least one pin.

Pins (the passage or fact each one follows):

* brute force: pure-Python scalar loops with math.fsum on tiny shapes;
* softmax rows sum to 1 (page "6.2 FlashAttention V2 chi tiết", 6.1: O is the
  accumulated sum divided by l);
* the CSDN FlashAttention-2 article's two-block online-softmax derivation
  ("具体计算过程"), and the page-6.2 tiled forward loop (section 6.1) with its
  causal loop bound and diagonal-crossing test, both equal the direct result;
* the page-6.2 section 5.3 drawing of the three causal block cases
  (tests/golden/causal_block_cases.txt);
* closed forms: identical key rows, scale 0, causal row 0, a single key;
* invariants: key shift, key permutation, bounds on L;
* grouped-query attention equals multi-head attention with repeated K/V, and
  dK, dV are group sums (CSDN article, "多查询注意力和分组查询注意力");
* D = rowsum(dO o O) = rowsum(P o dP) (page 6.2, section 7.3);
* central finite differences of <dO, O> for the backward;
* backward sum rules: sum_j dK_j = 0 and sum_j dV_j = sum_i dO_i.
"""

from __future__ import annotations

import math
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rng_inputs(seed, B, Hq, Hkv, Nq, Nk, d, scale_std=1.0):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, Hq, Nq, d)) * scale_std
    k = rng.standard_normal((B, Hkv, Nk, d)) * scale_std
    v = rng.standard_normal((B, Hkv, Nk, d))
    do = rng.standard_normal((B, Hq, Nq, d))
    return q, k, v, do


# ----------------------------------------------------------------------------
# brute force
# ----------------------------------------------------------------------------

def brute_forward(q, k, v, s, causal):
    """Scalar pure-Python attention: loops, math.exp, math.fsum; no NumPy
    arithmetic. Contiguous query-head groups share one K/V head."""
    B, Hq, Nq, d = len(q), len(q[0]), len(q[0][0]), len(q[0][0][0])
    Hkv, Nk = len(k[0]), len(k[0][0])
    G = Hq // Hkv
    O = [[[[0.0] * d for _ in range(Nq)] for _ in range(Hq)] for _ in range(B)]
    L = [[[0.0] * Nq for _ in range(Hq)] for _ in range(B)]
    for b in range(B):
        for h in range(Hq):
            kk, vv = k[b][h // G], v[b][h // G]
            for i in range(Nq):
                qi = q[b][h][i]
                cols = [j for j in range(Nk) if not (causal and j > i)]
                sc = [s * math.fsum(qi[c] * kk[j][c] for c in range(d)) for j in cols]
                mx = max(sc)
                e = [math.exp(x - mx) for x in sc]
                den = math.fsum(e)
                L[b][h][i] = mx + math.log(den)
                for c in range(d):
                    O[b][h][i][c] = math.fsum(e[t] * vv[cols[t]][c] for t in range(len(cols))) / den
    return np.array(O), np.array(L)


def pin_brute_force(ora):
    for causal, (B, Hq, Hkv, Nq, Nk, d) in [
        (False, (1, 2, 1, 5, 7, 3)),
        (True, (2, 4, 2, 6, 6, 4)),
        (False, (1, 3, 3, 4, 1, 2)),
    ]:
        q, k, v, _ = _rng_inputs(11 + Nq, B, Hq, Hkv, Nq, Nk, d)
        s = 0.37
        Ob, Lb = brute_forward(q.tolist(), k.tolist(), v.tolist(), s, causal)
        O, L = ora.forward(q, k, v, s, causal)
        assert np.max(np.abs(O - Ob)) <= 1e-12, "O differs from scalar brute force"
        assert np.max(np.abs(L - Lb)) <= 1e-12, "L differs from scalar brute force"


# ----------------------------------------------------------------------------
# softmax normalisation
# ----------------------------------------------------------------------------

def pin_rows_sum_to_one(ora):
    q, k, _, _ = _rng_inputs(3, 1, 1, 1, 9, 9, 5)
    for causal in (False, True):
        P = ora.probabilities_head(q[0, 0], k[0, 0], 0.8, causal)
        assert np.all(P >= 0)
        assert np.max(np.abs(P.sum(axis=1) - 1.0)) <= 1e-14, "softmax rows must sum to 1"
    # O of constant V rows is that constant: the normaliser is applied.
    q, k, v, _ = _rng_inputs(4, 1, 2, 2, 6, 6, 3)
    v[:] = 2.5
    O, _ = ora.forward(q, k, v, 1.1, True)
    assert np.max(np.abs(O - 2.5)) <= 1e-13


# ----------------------------------------------------------------------------
# the pages' online-softmax recurrences
# ----------------------------------------------------------------------------

def two_block_combine(q, k1, v1, k2, v2, s):
    """The CSDN article's two-block derivation, step by step (no masking):
    block 1: m1 = rowmax(S1), l1 = rowsum(e^{S1-m1}), O~1 = e^{S1-m1} V1;
    block 2: m2 = max(m1, rowmax(S2)), l2 = e^{m1-m2} l1 + rowsum(e^{S2-m2}),
             O~2 = diag(e^{m1-m2}) O~1 + e^{S2-m2} V2;
    then O = diag(l2)^-1 O~2 and L = m2 + log l2."""
    S1 = s * (q @ k1.T)
    S2 = s * (q @ k2.T)
    m1 = S1.max(axis=1)
    l1 = np.exp(S1 - m1[:, None]).sum(axis=1)
    Ot1 = np.exp(S1 - m1[:, None]) @ v1
    m2 = np.maximum(m1, S2.max(axis=1))
    l2 = np.exp(m1 - m2) * l1 + np.exp(S2 - m2[:, None]).sum(axis=1)
    Ot2 = np.exp(m1 - m2)[:, None] * Ot1 + np.exp(S2 - m2[:, None]) @ v2
    return Ot2 / l2[:, None], m2 + np.log(l2)


def pin_two_block_identity(ora):
    q, k, v, _ = _rng_inputs(5, 1, 1, 1, 7, 12, 4, scale_std=2.0)
    qh, kh, vh = q[0, 0], k[0, 0], v[0, 0]
    O, L = ora.forward_head(qh, kh, vh, 0.9, False)
    for c in (1, 5, 11):
        Oc, Lc = two_block_combine(qh, kh[:c], vh[:c], kh[c:], vh[c:], 0.9)
        assert np.max(np.abs(Oc - O)) <= 1e-12, "two-block recurrence differs from direct O"
        assert np.max(np.abs(Lc - L)) <= 1e-12, "two-block recurrence differs from direct L"


def _tile_partial(Qi, Kj, Vj, s, rows, cols, causal):
    """Softmax statistics of one (Q tile, K/V tile) pair on its own: the
    tile's row max m, its row sum l = sum exp(S - m) and the unnormalised
    output O~ = exp(S - m) V_j. Rows that see no key of the tile get m = -inf,
    l = 0, O~ = 0."""
    S = s * (Qi @ Kj.T)
    if causal:
        S = np.where(cols[None, :] > rows[:, None], -np.inf, S)
    m = S.max(axis=1)
    base = np.where(np.isfinite(m), m, 0.0)
    E = np.exp(S - base[:, None])
    return m, E.sum(axis=1), E @ Vj


def _merge(a, b):
    """Combine the statistics of two disjoint key sets (the rescaling of the
    CSDN article's two-block derivation, in either order): m = max(m1, m2),
    l = e^{m1-m} l1 + e^{m2-m} l2, O~ = e^{m1-m} O~1 + e^{m2-m} O~2."""
    (m1, l1, o1), (m2, l2, o2) = a, b
    m = np.maximum(m1, m2)
    base = np.where(np.isfinite(m), m, 0.0)
    w1, w2 = np.exp(m1 - base), np.exp(m2 - base)
    return m, w1 * l1 + w2 * l2, w1[:, None] * o1 + w2[:, None] * o2


def tiled_forward(Q, K, V, s, Br, Bc, causal, rng=None):
    """Forward by tiles: for each Q tile of Br rows, the statistics of every
    K/V tile of Bc keys it must visit, merged in a random order (tree-like,
    not left to right), then O = O~ / l and L = m + log l. Under the causal
    mask, K/V tiles whose first key lies after the Q tile's last row are not
    visited at all (page 6.2, section 5.3: the block-skip rule); tiles that
    cross the diagonal are masked element by element. Equal to the plain
    definition for any Br, Bc and merge order, which is what the pin checks."""
    rng = rng or np.random.default_rng(0)
    N, d = Q.shape
    O = np.zeros((N, d))
    L = np.zeros(N)
    for i in range(0, N, Br):
        rows = np.arange(i, min(N, i + Br))
        parts = []
        for j in range(0, K.shape[0], Bc):
            cols = np.arange(j, min(K.shape[0], j + Bc))
            if causal and cols[0] > rows[-1]:
                continue  # the whole tile lies above the diagonal
            parts.append(_tile_partial(Q[rows], K[cols], V[cols], s, rows, cols, causal))
        while len(parts) > 1:
            a, b = sorted(rng.choice(len(parts), size=2, replace=False))
            merged = _merge(parts[a], parts[b])
            parts = [p for t, p in enumerate(parts) if t not in (a, b)] + [merged]
        m, ell, Ot = parts[0]
        O[rows] = Ot / ell[:, None]
        L[rows] = m + np.log(ell)
    return O, L


def pin_tiled_loop(ora):
    q, k, v, _ = _rng_inputs(6, 1, 1, 1, 37, 37, 5)
    qh, kh, vh = q[0, 0], k[0, 0], v[0, 0]
    rng = np.random.default_rng(6)
    for causal in (False, True):
        O, L = ora.forward_head(qh, kh, vh, 0.6, causal)
        for Br, Bc in [(8, 8), (16, 4), (4, 16), (37, 37), (5, 7), (1, 1)]:
            Ot, Lt = tiled_forward(qh, kh, vh, 0.6, Br, Bc, causal, rng)
            assert np.max(np.abs(Ot - O)) <= 1e-12, f"tiled forward differs (Br={Br}, Bc={Bc})"
            assert np.max(np.abs(Lt - L)) <= 1e-12


def load_causal_golden():
    cases = []
    with open(os.path.join(GOLDEN, "causal_block_cases.txt"), encoding="utf-8") as f:
        lines = [ln.rstrip("\n") for ln in f if ln.strip() and not ln.startswith("#")]
    a = 0
    while a < len(lines):
        _, name, off = lines[a].split()
        grid = np.array([[ch == "■" for ch in row] for row in lines[a + 1:a + 4]])
        cases.append((name, int(off), grid))
        a += 4
    return cases


def pin_causal_drawing(ora):
    """Visibility seen through the oracle (zero scores give P = 1/n on the
    visible keys and 0 on masked ones) matches the page's drawing."""
    N = 24
    q = np.zeros((N, 2))
    k = np.zeros((N, 2))
    P = ora.probabilities_head(q, k, 1.0, True)
    cases = load_causal_golden()
    assert [c[0] for c in cases] == ["below_diagonal", "diagonal", "above_diagonal"]
    for name, off, grid in cases:
        k0 = 8
        q0 = k0 + off
        block = P[q0:q0 + 3, k0:k0 + 6] > 0
        assert np.array_equal(block, grid), f"causal case {name} does not match the drawing"


# ----------------------------------------------------------------------------
# closed forms and special cases
# ----------------------------------------------------------------------------

def pin_identical_keys(ora):
    q, k, v, _ = _rng_inputs(7, 1, 1, 1, 10, 10, 4)
    kh = np.tile(k[0, 0, :1], (10, 1))
    qh, vh = q[0, 0], v[0, 0]
    s = 0.7
    for causal in (False, True):
        O, L = ora.forward_head(qh, kh, vh, s, causal)
        n = np.arange(1, 11) if causal else np.full(10, 10)
        mean = np.cumsum(vh, axis=0) / n[:, None] if causal else np.tile(vh.mean(axis=0), (10, 1))
        assert np.max(np.abs(O - mean)) <= 1e-13, "identical keys must give the mean of visible V"
        Lref = s * (qh @ kh[0]) + np.log(n)
        assert np.max(np.abs(L - Lref)) <= 1e-13


def pin_zero_scale(ora):
    q, k, v, do = _rng_inputs(8, 1, 2, 1, 9, 9, 3)
    for causal in (False, True):
        O, L = ora.forward(q, k, v, 0.0, causal)
        n = np.arange(1, 10) if causal else np.full(9, 9)
        assert np.max(np.abs(L[0, 0] - np.log(n))) <= 1e-14
        vh = v[0, 0]
        mean = np.cumsum(vh, axis=0) / n[:, None] if causal else np.tile(vh.mean(axis=0), (9, 1))
        assert np.max(np.abs(O[0, 1] - mean)) <= 1e-13
        dQ, dK, dV = ora.backward(q, k, v, do, 0.0, causal)
        assert np.all(dQ == 0.0) and np.all(dK == 0.0), "scale 0 must give dQ = dK = 0 exactly"
        ref = np.zeros((9, 3))
        for h in range(2):
            for i in range(9):
                vis = range(i + 1) if causal else range(9)
                for j in vis:
                    ref[j] += do[0, h, i] / n[i]
        assert np.max(np.abs(dV[0, 0] - ref)) <= 1e-13


def pin_causal_row0_and_single_key(ora):
    q, k, v, _ = _rng_inputs(9, 2, 2, 2, 6, 6, 5)
    s = 0.45
    O, L = ora.forward(q, k, v, s, True)
    assert np.max(np.abs(O[:, :, 0] - v[:, :, 0])) <= 1e-15, "causal row 0 must equal V[0]"
    ref = s * np.einsum("bhd,bhd->bh", q[:, :, 0], k[:, :, 0])
    assert np.max(np.abs(L[:, :, 0] - ref)) <= 1e-14
    q1, k1, v1, _ = _rng_inputs(10, 1, 1, 1, 4, 1, 3)
    O, L = ora.forward(q1, k1, v1, s, False)
    assert np.max(np.abs(O[0, 0] - v1[0, 0, 0])) <= 1e-15, "a single key gives O = V[0]"
    assert np.max(np.abs(L[0, 0] - s * (q1[0, 0] @ k1[0, 0, 0]))) <= 1e-14


# ----------------------------------------------------------------------------
# invariants
# ----------------------------------------------------------------------------

def pin_key_shift(ora):
    q, k, v, _ = _rng_inputs(12, 1, 1, 1, 8, 8, 4)
    c = np.array([0.3, -1.2, 2.0, 0.5])
    s = 0.5
    for causal in (False, True):
        O, L = ora.forward(q, k, v, s, causal)
        O2, L2 = ora.forward(q, k + c, v, s, causal)
        assert np.max(np.abs(O2 - O)) <= 1e-12, "a common key shift must leave O unchanged"
        assert np.max(np.abs(L2 - L - s * (q @ c))) <= 1e-12


def pin_key_permutation(ora):
    q, k, v, _ = _rng_inputs(13, 1, 1, 1, 6, 11, 4)
    perm = np.random.default_rng(0).permutation(11)
    O, L = ora.forward(q, k, v, 0.9, False)
    O2, L2 = ora.forward(q, k[:, :, perm], v[:, :, perm], 0.9, False)
    assert np.max(np.abs(O2 - O)) <= 1e-12 and np.max(np.abs(L2 - L)) <= 1e-12


def pin_lse_bounds(ora):
    q, k, v, _ = _rng_inputs(14, 1, 1, 1, 16, 16, 8, scale_std=3.0)
    s = 0.35
    for causal in (False, True):
        _, L = ora.forward(q, k, v, s, causal)
        S = s * (q[0, 0] @ k[0, 0].T)
        if causal:
            S = np.where(np.triu(np.ones((16, 16), bool), 1), -np.inf, S)
        mx = S.max(axis=1)
        n = np.arange(1, 17) if causal else np.full(16, 16)
        assert np.all(L[0, 0] >= mx - 1e-12) and np.all(L[0, 0] <= mx + np.log(n) + 1e-12)


def pin_gqa_reduction(ora):
    B, Hq, Hkv, N, d = 2, 6, 2, 7, 3
    q, k, v, do = _rng_inputs(15, B, Hq, Hkv, N, N, d)
    G = Hq // Hkv
    kr = np.repeat(k, G, axis=1)
    vr = np.repeat(v, G, axis=1)
    for causal in (False, True):
        O, L = ora.forward(q, k, v, 0.7, causal)
        Om, Lm = ora.forward(q, kr, vr, 0.7, causal)
        assert np.max(np.abs(O - Om)) <= 1e-14 and np.max(np.abs(L - Lm)) <= 1e-14
        dQ, dK, dV = ora.backward(q, k, v, do, 0.7, causal)
        dQm, dKm, dVm = ora.backward(q, kr, vr, do, 0.7, causal)
        assert np.max(np.abs(dQ - dQm)) <= 1e-13
        assert np.max(np.abs(dK - dKm.reshape(B, Hkv, G, N, d).sum(axis=2))) <= 1e-13
        assert np.max(np.abs(dV - dVm.reshape(B, Hkv, G, N, d).sum(axis=2))) <= 1e-13


def pin_d_identity(ora):
    q, k, v, do = _rng_inputs(16, 1, 1, 1, 12, 12, 6)
    for causal in (False, True):
        O, _ = ora.forward(q, k, v, 0.4, causal)
        D = ora.row_dot(do, O)[0, 0]
        P = ora.probabilities_head(q[0, 0], k[0, 0], 0.4, causal)
        dP = do[0, 0] @ v[0, 0].T
        assert np.max(np.abs(D - (P * dP).sum(axis=1))) <= 1e-13


# ----------------------------------------------------------------------------
# backward
# ----------------------------------------------------------------------------

def pin_finite_differences(ora):
    B, Hq, Hkv, N, d = 1, 4, 2, 6, 3
    q, k, v, do = _rng_inputs(17, B, Hq, Hkv, N, N, d)
    s = 0.8
    h = 1e-6
    for causal in (False, True):
        dQ, dK, dV = ora.backward(q, k, v, do, s, causal)

        def f(qq, kk, vv):
            O, _ = ora.forward(qq, kk, vv, s, causal)
            return float((O * do).sum())

        for name, x, g in (("q", q, dQ), ("k", k, dK), ("v", v, dV)):
            num = np.zeros_like(x)
            it = np.nditer(x, flags=["multi_index"])
            for _ in it:
                idx = it.multi_index
                xp = x.copy()
                xm = x.copy()
                xp[idx] += h
                xm[idx] -= h
                args_p = {"q": (xp, k, v), "k": (q, xp, v), "v": (q, k, xp)}[name]
                args_m = {"q": (xm, k, v), "k": (q, xm, v), "v": (q, k, xm)}[name]
                num[idx] = (f(*args_p) - f(*args_m)) / (2 * h)
            rel = np.max(np.abs(num - g)) / max(1.0, np.max(np.abs(g)))
            assert rel <= 1e-6, f"d{name} disagrees with finite differences (rel {rel:.2e})"


def pin_backward_sum_rules(ora):
    q, k, v, do = _rng_inputs(18, 2, 4, 2, 10, 10, 4)
    for causal in (False, True):
        dQ, dK, dV = ora.backward(q, k, v, do, 0.6, causal)
        assert np.max(np.abs(dK.sum(axis=2))) <= 1e-12, "sum over keys of dK must vanish"
        ref = do.reshape(2, 2, 2, 10, 4).sum(axis=(2, 3))
        assert np.max(np.abs(dV.sum(axis=2) - ref)) <= 1e-12, "sum of dV must equal sum of dO"


ALL_PINS = [
    pin_brute_force,
    pin_rows_sum_to_one,
    pin_two_block_identity,
    pin_tiled_loop,
    pin_causal_drawing,
    pin_identical_keys,
    pin_zero_scale,
    pin_causal_row0_and_single_key,
    pin_key_shift,
    pin_key_permutation,
    pin_lse_bounds,
    pin_gqa_reduction,
    pin_d_identity,
    pin_finite_differences,
    pin_backward_sum_rules,
]
