"""The machine-limit microbenchmarks (tests/hw/machine_limits.hip) run and
give physically possible figures: the matrix core at most its rate at the
measured clock, the LDS at most 64 banks x 4 bytes per clock, a shader clock
between idle and the 2.4 GHz maximum. The figures themselves are recorded by
`bench.py --machine-limits`."""

import pytest

pytestmark = pytest.mark.gpu


def test_machine_limit_probes_give_possible_figures():
    from tests.hw import machine_limits
    rows = machine_limits.run(iters_mfma=4000, iters_exp=4000, iters_lds=1024)
    assert len(rows) == 10
    for r in rows:
        print(r)
        assert 0.3 < r["clock_ghz"] < 2.6, r
        if r["unit"] == "TFLOP/s":
            assert 0.0 < r["pct_at_clock"] < 105.0, r
        elif r["unit"] == "bytes / clock / CU":
            assert 16.0 < r["value"] <= 64 * 4 * 1.05, r
        else:
            assert 1.0 < r["value"] <= 64.0 * 1.05, r  # at most one lane-op per lane of a CU's 4 SIMDs per clock
    mfma2 = rows[1]
    assert mfma2["pct_at_clock"] > 60.0, mfma2
