"""Pins of the CPU oracle (no GPU): every check in oracle_checks on the real oracle, plus the seeded
tiny configuration end to end."""

import numpy as np
import pytest

import oracle
from linear_attention_beam_amd import inputs
from tests import oracle_checks as oc


@pytest.mark.parametrize("check", oc.ALL_CHECKS, ids=lambda c: c.__name__)
def test_pin(check):
    check(oracle)


def test_tiny_config_forms_agree():
    """The seeded tiny configuration (1 request, 1 head, d=16, 8 beams, 3 steps, fp32)."""
    cfg = inputs.config(0)
    S_ctx = inputs.direct_sctx(cfg)
    steps = [dict(q=s.q, k=s.k, v=s.v, alpha=s.alpha, beta=s.beta, parent=s.parent)
             for s in inputs.decode_inputs(cfg)]
    assert steps[0]["parent"].max() == 0
    fs = oracle.decode_fullstate(S_ctx, steps)
    rp = oracle.decode_replay(S_ctx, steps, cfg.B, cfg.L)
    for t in range(cfg.L):
        assert np.max(np.abs(fs["o"][(0, 0)][t] - rp["heads"][(0, 0)]["o"][t])) < 1e-12
    # every written record slot lies inside the arena and chains only point at earlier steps
    for t, table in enumerate(rp["chains"][0], start=1):
        assert table.shape == (cfg.B, cfg.L)
        assert np.all(table[:, t - 1] == (t - 1) * cfg.B + np.arange(cfg.B))
        assert np.all(table[:, t:] == -1)
        if t > 1:
            prev = rp["chains"][0][t - 2]
            assert np.array_equal(table[:, : t - 1], prev[steps[t - 1]["parent"][0], : t - 1])
