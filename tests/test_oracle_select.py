"""Pins of the beam-selection oracle (no GPU), and planted mistakes that the pins must catch."""

import inspect
import types

import numpy as np
import pytest

import oracle
import oracle.beam_selection as bsel
from tests import select_checks as sc


@pytest.mark.parametrize("check", sc.ALL_CHECKS, ids=lambda c: c.__name__)
def test_pin(check):
    check(oracle)


def test_rejects_bad_arguments():
    with pytest.raises(ValueError):
        oracle.beam_select(np.zeros((1, 2), np.float32), np.zeros((1, 2, 3), np.float32), 7)
    with pytest.raises(ValueError):
        oracle.beam_select(np.zeros((1, 2), np.float32), np.full((1, 2, 3), np.nan, np.float32), 1)


MUTANTS = [
    ("ascending instead of descending", "np.lexsort((idx, -flat[r].astype(np.float64)))",
     "np.lexsort((idx, flat[r].astype(np.float64)))"),
    ("ties to the larger index", "np.lexsort((idx, -flat[r].astype(np.float64)))",
     "np.lexsort((-idx, -flat[r].astype(np.float64)))"),
    ("parent and token from the wrong divisor", "parent[r] = order // n_cand", "parent[r] = order // n_prev"),
    ("score without the beam score", "return (bs[:, :, None] + lp).astype(np.float32)",
     "return (0 * bs[:, :, None] + lp).astype(np.float32)"),
    ("one survivor dropped", "[:n_beams]", "[1:n_beams + 1]"),
]


@pytest.mark.parametrize("desc,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_planted_mistake_is_caught(desc, old, new):
    src = inspect.getsource(bsel)
    assert src.count(old) >= 1, f"mutation anchor not found: {old!r}"
    mod = types.ModuleType("select_mutant")
    exec(compile(src.replace(old, new, 1), "select_mutant", "exec"), mod.__dict__)
    caught = []
    for check in sc.ALL_CHECKS:
        try:
            check(mod)
        except Exception as e:  # noqa: BLE001 - any failure of a pin counts as a catch
            caught.append((check.__name__, type(e).__name__))
    assert caught, f"no pin catches: {desc}"
