"""CPU oracle for exact attention (float64, NumPy).

TEST INFRASTRUCTURE ONLY: imported by the tests, the smoke check and the
CPU-baseline leg of the benchmark, never by the library itself.
"""

from .attention import (  # noqa: F401
    backward,
    backward_dq_rows,
    backward_head,
    backward_varlen,
    forward,
    forward_head,
    forward_varlen,
    probabilities_head,
    row_dot,
)
from . import fp8  # noqa: F401,E402
