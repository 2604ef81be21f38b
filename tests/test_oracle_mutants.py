"""Each plausible mistake planted in a copy of the oracle (on the CPU) must
fail at least one pin: this shows the pins are strong enough to trust the
oracle."""

import importlib.util
import os
import sys
import types

import pytest

from tests.oracle_pins import ALL_PINS

SRC = os.path.join(os.path.dirname(os.path.dirname(__file__)), "oracle", "attention.py")

MUTANTS = {
    "mask_excludes_diagonal": ("cols[None, :] > row_idx[:, None]", "cols[None, :] >= row_idx[:, None]"),
    "mask_transposed": ("cols[None, :] > row_idx[:, None]", "cols[None, :] < row_idx[:, None]"),
    "forward_unscaled": ("S = s * (q_rows @ kh.T)", "S = (q_rows @ kh.T)"),
    "lse_without_log": ("Lb = m + np.log(ell)", "Lb = m + ell"),
    "output_unnormalised": ("P = np.exp(S - Lb[:, None])\n        O[a", "P = np.exp(S - m[:, None])\n        O[a"),
    "dq_unscaled": ("dQ[r] = s * (dS @ kh)", "dQ[r] = (dS @ kh)"),
    "dk_unscaled": ("dK += s * (dS.T @ qh[r])", "dK += (dS.T @ qh[r])"),
    "ds_wrong_sign": ("dS = P * (dP - D[:, None])", "dS = P * (dP + D[:, None])"),
    "dv_untransposed": ("dV += P.T @ doh[r]", "dV += P @ doh[r]"),
    "d_from_dO_only": ("(_as64(do) * _as64(o)).sum(axis=-1)", "(_as64(do) * _as64(do)).sum(axis=-1)"),
    "dk_operand_swapped": ("dK += s * (dS.T @ qh[r])", "dK += s * (dS.T @ doh[r])"),
    "gqa_interleaved_groups": ("g = h // G\n            O[b, h]", "g = h % Hkv\n            O[b, h]"),
    "gqa_backward_not_summed": ("dK[b, g] += dk", "dK[b, g] = dk"),
    # the full backward's recompute (the row-local dQ has its own pin against it)
    "p_recompute_unmasked_in_backward": ("S = _scores(qh[r], r, kh, s, causal)\n        m = S.max(axis=1)\n"
                                         "        Lb = m + np.log(np.exp(S - m[:, None]).sum(axis=1))\n"
                                         "        P = np.exp(S - Lb[:, None])\n        Ob = P @ vh",
                                         "S = _scores(qh[r], r, kh, s, False)\n        m = S.max(axis=1)\n"
                                         "        Lb = m + np.log(np.exp(S - m[:, None]).sum(axis=1))\n"
                                         "        P = np.exp(S - Lb[:, None])\n        Ob = P @ vh"),
}


def _load_mutant(name, old, new):
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation site for {name} not unique"
    mod = types.ModuleType(f"oracle_mutant_{name}")
    exec(compile(src.replace(old, new), f"<mutant {name}>", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name):
    mod = _load_mutant(name, *MUTANTS[name])
    failed = []
    for pin in ALL_PINS:
        try:
            pin(mod)
        except (AssertionError, ValueError, IndexError, FloatingPointError):
            failed.append(pin.__name__)
    assert failed, f"no pin catches the planted mistake {name}"
