"""The multi-layer beam-search decode (random weights) against the oracle.

Every layer's decode steps are recomputed by the oracle from the inputs the layer received (recorded q, k,
v, alpha, beta and the shared parents) and that layer's own prompt prefill; every beam selection is
recomputed from the recorded candidate scores.  Outputs within max-abs 1e-3, selections bit for bit.
"""

import numpy as np
import pytest
import torch

import oracle
from linear_attention_beam_amd import harness, inputs
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu


def check_stack(cfg: harness.StackConfig, heads=None):
    gu.log(f"harness {cfg}")
    stack = harness.GDNStack(cfg)
    try:
        tokens, final = stack.decode(record=True)
        torch.cuda.synchronize()
        rec = stack.record
    finally:
        stack.close()
    assert len(rec) == cfg.L and len(tokens) == cfg.L

    for t0, st in enumerate(rec):
        n_beams = st["parent"].shape[1]
        ref = oracle.beam_select(st["beam_scores"].numpy(), st["logp"].numpy(), n_beams)
        assert np.array_equal(st["parent"].numpy(), ref[0]), f"parents t={t0 + 1}"
        assert np.array_equal(st["token"].numpy(), ref[1]), f"tokens t={t0 + 1}"
        assert np.array_equal(st["scores"].numpy().view(np.uint32), ref[2].view(np.uint32)), f"scores t={t0 + 1}"
    assert rec[0]["parent"].shape[1] == min(cfg.B, cfg.n_cand)
    assert np.all(rec[0]["parent"].numpy() == 0)

    heads = [(r, h) for r in range(cfg.R) for h in range(cfg.H)] if heads is None else heads
    worst = 0.0
    for layer in range(cfg.layers):
        pcfg = inputs.config(2, R=cfg.R, H=cfg.H, d_k=cfg.d_k, d_v=cfg.d_v, prefill_steps=cfg.prefill_tokens,
                             alpha_lo=cfg.alpha_lo)
        pf = inputs.prefill_inputs(pcfg, seed=100 + layer)
        steps = []
        for st in rec:
            x = st["layers"][layer]
            steps.append(dict(q=x["q"].double().numpy(), k=x["k"].double().numpy(), v=x["v"].double().numpy(),
                              alpha=x["alpha"].double().numpy(), beta=x["beta"].double().numpy(),
                              parent=st["parent"].numpy()))
        for r, h in heads:
            sctx = gu.oracle_prefill_head(pf, r, h)
            res = oracle.decode_replay(sctx[None, None], [dict(q=s["q"][r:r + 1, :, h:h + 1],
                                                               k=s["k"][r:r + 1, :, h:h + 1],
                                                               v=s["v"][r:r + 1, :, h:h + 1],
                                                               alpha=s["alpha"][r:r + 1, :, h:h + 1],
                                                               beta=s["beta"][r:r + 1, :, h:h + 1],
                                                               parent=s["parent"][r:r + 1]) for s in steps],
                                       cfg.B, cfg.L)
            ref = res["heads"][(0, 0)]
            for t0, st in enumerate(rec):
                got = st["layers"][layer]["o"][r, :, h].double().numpy()
                assert np.all(np.isfinite(got))
                e = float(np.max(np.abs(got - ref["o"][t0])))
                worst = max(worst, e)
                assert e <= gu.TOL, f"layer {layer} r={r} h={h} t={t0 + 1}: max|o err| {e:.3g}"
    gu.log(f"  max|o err| {worst:.3g}")
    return rec


def test_stack_small():
    """Two layers, 2 requests x 2 heads, 48 candidates: 48 beams after the first step, then 64."""
    cfg = harness.StackConfig(R=2, B=64, L=4, layers=2, H=2, d_k=128, d_v=128, D=256, n_cand=48,
                              prefill_tokens=16, seed=1)
    rec = check_stack(cfg)
    assert [st["parent"].shape[1] for st in rec] == [48, 64, 64, 64]


def test_stack_small_odd_dims():
    """Small head sizes (d_k = 64, d_v = 32, on the fused kernel's smaller row size); 7 candidates, then 40
    beams."""
    cfg = harness.StackConfig(R=3, B=40, L=3, layers=3, H=3, d_k=64, d_v=32, D=96, n_cand=7,
                              prefill_tokens=8, seed=2)
    rec = check_stack(cfg)
    assert [st["parent"].shape[1] for st in rec] == [7, 40, 40]


def test_stack_wide_sampled():
    """Three layers, 4 requests x 16 heads, 256 beams x 256 candidates; sampled heads against the oracle."""
    cfg = harness.StackConfig(R=4, B=256, L=4, layers=3, H=16, d_k=128, d_v=128, D=1024, n_cand=256,
                              prefill_tokens=32, seed=3)
    check_stack(cfg, heads=[(0, 0), (1, 7), (2, 15), (3, 9)])
