"""Sensitivity of the oracle pins: plant one mistake at a time in a copy of the oracle (on the CPU)
and check that at least one pin fails for every planted mistake."""

import inspect
import types

import pytest

import oracle.gdn_beam as gb
from tests import oracle_checks as oc

# (description, text in oracle/gdn_beam.py, replacement)
MUTANTS = [
    ("sign of the key-damping term", "S_damped = S - beta", "S_damped = S + beta"),
    ("dropped write term", "+ beta[..., None, None] * (v[..., :, None] * k[..., None, :])", ""),
    ("transposed rank-one factor", "(Sk[..., :, None] * k[..., None, :])", "(k[..., :, None] * Sk[..., None, :])"),
    ("decay includes the record's own alpha", "for i in range(j + 1, n):", "for i in range(j, n):"),
    ("S_ctx decay dropped", "A *= chain_alpha[:, i]", "A *= 1.0"),
    ("alpha dropped from u", "u = bt[:, None] * (vt - at[:, None] * p)", "u = bt[:, None] * (vt - p)"),
    ("beta dropped from u", "u = bt[:, None] * (vt - at[:, None] * p)", "u = (vt - at[:, None] * p)"),
    ("output from the pre-update state", "o = at[:, None] * Sq_prev + np.sum(kt * qt, axis=1)[:, None] * u",
     "o = Sq_prev"),
    ("own record missing from the output", "np.sum(kt * qt, axis=1)[:, None] * u", "0.0 * u"),
    ("query replay uses key projections", "c * proj_q", "c * proj_k"),
    ("S_ctx projection transposed", "(kt @ S_ctx.T)", "(kt @ S_ctx)"),
    ("chain copied from the wrong beam", "out[b, : t - 1] = chain_prev[p, : t - 1]",
     "out[b, : t - 1] = chain_prev[min(b, chain_prev.shape[0] - 1), : t - 1]"),
    ("chain loses its oldest record", "out[b, : t - 1] = chain_prev[p, : t - 1]",
     "out[b, 1 : t - 1] = chain_prev[p, 1 : t - 1]"),
    ("slots shifted within a step", "return (t - 1) * max_beams + b", "return (t - 1) * max_beams + (b + 1) % max_beams"),
    ("FullState never advances", "        states = S\n", "        pass\n"),
    ("FullState ignores parents", "S = gdn_step(states[par]", "S = gdn_step(states[np.minimum(np.arange(len(par)), len(states) - 1)]"),
    ("prefill skips the first token", "for n in range(N):", "for n in range(1, N):"),
]


def _mutant_module(old, new):
    src = inspect.getsource(gb)
    assert src.count(old) >= 1, f"mutation anchor not found: {old!r}"
    mod = types.ModuleType("oracle_mutant")
    exec(compile(src.replace(old, new, 1), "oracle_mutant", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("desc,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_planted_mistake_is_caught(desc, old, new):
    mod = _mutant_module(old, new)
    caught = []
    for check in oc.ALL_CHECKS:
        try:
            check(mod)
        except Exception as e:  # noqa: BLE001 - any failure of a pin counts as a catch
            caught.append((check.__name__, type(e).__name__))
    assert caught, f"no pin catches: {desc}"
