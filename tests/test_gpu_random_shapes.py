"""A seeded sweep of decode shapes against the oracle, every request and head: request and head counts, head
sizes (multiples of 32 for the fused kernel, others for the fp32 kernel), record capacity, decode length,
per-step beam counts (growing, shrinking, one), tile sizes and kernels drawn at random from a fixed seed, so
that combinations the hand-picked edge cases do not name are covered too.  Decays are drawn from U(0, 1) in
a third of the cases, so that chain products also get small."""

import numpy as np
import pytest

from linear_attention_beam_amd import inputs, onela
from tests import gpu_util as gu
from tests.test_gpu_edges import check_all_heads, ragged_steps, short_prefill_sctx

pytestmark = pytest.mark.gpu

N_CASES = 24


def draw_case(i):
    rng = np.random.default_rng([0x5A3E, i])
    R = int(rng.integers(1, 4))
    H = int(rng.integers(1, 6))
    d_v = int(rng.choice([32, 64, 96, 128, 160, 192, 224, 256, 48, 80]))
    L = int(rng.integers(1, 10))
    B_max = int(rng.choice([1, 7, 16, 37, 64, 100, 130, 200]))
    beams = [int(rng.integers(1, B_max + 1)) for _ in range(L)]
    tile = int(rng.choice([0, 16, 32]))
    kernel = str(rng.choice(["fused", "fused", "fused", "generic", "materialize"]))
    small_alpha = bool(rng.random() < 1 / 3)
    d_k = int(rng.choice([128, 64, 256]))
    return dict(R=R, H=H, d_k=d_k, d_v=d_v, L=L, B_max=B_max, beams=beams, tile=tile, kernel=kernel,
                small_alpha=small_alpha)


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_shape(i):
    c = draw_case(i)
    gu.log(f"random shape {i}: {c}")
    cfg = inputs.config(2, R=c["R"], H=c["H"], d_k=c["d_k"], d_v=c["d_v"], B=c["B_max"], L=c["L"])
    steps = ragged_steps(inputs.decode_inputs(cfg, seed=100 + i), c["beams"])
    if c["small_alpha"]:
        rng = np.random.default_rng([0x5A3F, i])
        for s in steps:
            s.alpha[...] = rng.uniform(0.0, 1.0, size=s.alpha.shape).astype(np.float32)
    sctx = short_prefill_sctx(cfg)
    tile = c["tile"] if c["kernel"] == "fused" else 0

    def go(tile_beams):
        return gu.GpuRun(cfg, steps, sctx=sctx, tile_beams=tile_beams, force_generic=c["kernel"] == "generic",
                         materialize=c["kernel"] == "materialize")

    try:
        run = go(tile)
    except onela.OnelaError as e:
        # a requested tile too large for the device's LDS is refused on the host; the automatic tile fits
        if e.status != onela.ONELA_ERR_UNSUPPORTED or tile == 0:
            raise
        gu.log(f"  tile {tile} refused ({e}); automatic tile")
        run = go(0)
    assert run.status == onela.ONELA_OK
    assert run.view["fused"] == (c["kernel"] == "fused" and c["d_v"] % 32 == 0)
    gu.log(f"  max|o err|={check_all_heads(run, cfg, steps, sctx, c['B_max'], c['L']):.3g}")
