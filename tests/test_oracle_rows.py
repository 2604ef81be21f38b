"""Pin of oracle.backward_dq_rows (the row-local dQ used for sampled rows of
long sequences): it must equal the dQ rows of the full oracle backward,
which the finite-difference pins check, on small inputs."""

import numpy as np
import pytest

import oracle


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("n,d", [(1, 8), (37, 16), (130, 32)])
def test_backward_dq_rows_equals_full_backward(causal, n, d):
    rng = np.random.default_rng(n + d)
    q, k, v, do = (rng.standard_normal((n, d)) for _ in range(4))
    full, _, _ = oracle.backward_head(q, k, v, do, 0.3, causal)
    rows = np.unique(np.concatenate([[0, n - 1], rng.integers(0, n, size=min(n, 20))]))
    got = oracle.backward_dq_rows(q, k, v, do, 0.3, causal, rows, row_block=7)
    np.testing.assert_allclose(got, full[rows], rtol=0, atol=1e-12)


def test_backward_dq_rows_is_independent_of_the_other_rows():
    # a row's dQ does not depend on which other rows are asked for (up to the
    # rounding order of the matrix products)
    rng = np.random.default_rng(5)
    q, k, v, do = (rng.standard_normal((50, 8)) for _ in range(4))
    a = oracle.backward_dq_rows(q, k, v, do, 0.5, True, [3, 40])
    b = oracle.backward_dq_rows(q, k, v, do, 0.5, True, [40])
    np.testing.assert_allclose(a[1], b[0], rtol=0, atol=1e-12)
