"""GPU beam selection against the oracle, through the C ABI: survivors, their order, parents, tokens and
scores bit for bit; host-side errors; and the selection feeding decode steps on the device."""

import numpy as np
import pytest
import torch

import oracle
from linear_attention_beam_amd import inputs, onela
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu


def run_select(si: inputs.SelectInputs, n_beams: int):
    dev = gu.device()
    p, t, s = onela.beam_select(torch.from_numpy(si.beam_scores).to(dev), torch.from_numpy(si.logp).to(dev), n_beams)
    torch.cuda.synchronize()
    return p.cpu().numpy(), t.cpu().numpy(), s.cpu().numpy()


def assert_same(si, n_beams, got):
    ref = oracle.beam_select(si.beam_scores, si.logp, n_beams)
    for name, a, b in zip(("parent", "token", "score"), got, ref):
        if name == "score":
            assert np.array_equal(a.view(np.uint32), b.view(np.uint32)), name
        else:
            assert np.array_equal(a, b), name


@pytest.mark.parametrize("R,n_prev,n_cand,n_beams,ties", [
    (1, 1, 5, 3, False),        # one parent: the first decode step
    (3, 7, 33, 50, False),
    (2, 32, 64, 2048, False),   # every candidate survives
    (2, 64, 64, 2048, False),   # one full chunk, half survive
    (2, 100, 300, 512, False),  # two passes
    (4, 512, 256, 2048, False),  # the largest n_beams
    (3, 300, 50, 700, True),    # many exact ties: the flat-index order decides
    (1, 1, 9000, 1, True),
    (2, 8193, 1, 7, False),     # one candidate per beam, just over one chunk
    # 512 chunks of 8192 in the first pass (512-thread chunk workgroups on a 256-CU GPU), then a second chunk
    # pass over 128 chunks of survivors (1024-thread workgroups), with ties
    (8, 1024, 512, 2048, True),
    (32, 512, 256, 64, False),  # 512-thread chunk workgroups, few survivors
])
def test_select_matches_oracle(R, n_prev, n_cand, n_beams, ties):
    gu.log(f"select R={R} n_prev={n_prev} n_cand={n_cand} n_beams={n_beams} ties={ties}")
    si = inputs.select_inputs(R, n_prev, n_cand, seed=1, ties=ties)
    assert_same(si, n_beams, run_select(si, n_beams))


def test_select_full_size():
    """32 requests x 512 beams x 256 candidates -> 512 survivors, as bench.py times it (one chunk pass, then the finish)."""
    gu.log("select full size 32 x 512 x 256 -> 512")
    si = inputs.select_inputs(32, 512, 256, seed=0)
    assert_same(si, 512, run_select(si, 512))


def test_select_neg_inf():
    si = inputs.select_inputs(2, 40, 130, seed=2)
    si.logp[:, ::3, :] = -np.inf
    si.logp[1, :, ::2] = -np.inf
    gu.log("select with -inf candidates")
    assert_same(si, 1000, run_select(si, 1000))
    all_inf = inputs.SelectInputs(si.beam_scores, np.full_like(si.logp, -np.inf))
    assert_same(all_inf, 300, run_select(all_inf, 300))


def test_select_host_errors():
    dev = gu.device()
    bs = torch.zeros((1, 4), device=dev)
    lp = torch.zeros((1, 4, 8), device=dev)
    for n_beams, status in ((33, onela.ONELA_ERR_INVALID_ARG), (0, onela.ONELA_ERR_INVALID_ARG)):
        with pytest.raises(onela.OnelaError) as e:
            onela.beam_select(bs, lp, n_beams)
        assert e.value.status == status
    with pytest.raises(onela.OnelaError) as e:
        onela.beam_select(torch.zeros((1, 64), device=dev), torch.zeros((1, 64, 64), device=dev), 2049)
    assert e.value.status == onela.ONELA_ERR_UNSUPPORTED
    need = onela.onela_beam_select_scratch(1, 256, 128, 100)  # 32768 candidates: one reduce pass
    assert need > 0
    small = torch.empty(need - 8, dtype=torch.uint8, device=dev)
    with pytest.raises(onela.OnelaError) as e:
        onela.beam_select(torch.zeros((1, 256), device=dev), torch.zeros((1, 256, 128), device=dev), 100, scratch=small)
    assert e.value.status == onela.ONELA_ERR_INVALID_ARG


def test_select_feeds_decode():
    """Beam search on the device: each step's survivors (selected on the GPU from synthetic candidate scores)
    are the next step's parents; outputs and chains match the oracle given the oracle's own selection."""
    cfg = inputs.config(2, R=2, H=3, B=64, L=4, prefill_steps=0, sctx_std=0.1)
    steps = inputs.decode_inputs(cfg)
    sctx = inputs.direct_sctx(cfg)
    n_cand = 24
    dev = gu.device()
    ctx = onela.OneLA(cfg.R, cfg.H, cfg.d_k, cfg.d_v, cfg.B, cfg.L, device=dev)
    ctx.set_context(torch.from_numpy(sctx).to(dev))
    beam_scores = torch.zeros((cfg.R, 1), device=dev)
    ref_scores = np.zeros((cfg.R, 1), np.float32)
    parent_gpu = torch.zeros((cfg.R, cfg.B), dtype=torch.int32, device=dev)  # step 1: the shared state
    outs = []
    for t, s in enumerate(steps, start=1):
        if t > 1:
            si = inputs.select_inputs(cfg.R, cfg.B, n_cand, seed=t, tag=7)
            si.beam_scores[:] = ref_scores
            parent_gpu, _, scores_gpu = onela.beam_select(beam_scores, torch.from_numpy(si.logp).to(dev), cfg.B)
            ref_parent, _, ref_scores = oracle.beam_select(ref_scores, si.logp, cfg.B)
            assert np.array_equal(parent_gpu.cpu().numpy(), ref_parent), f"parents of step {t}"
            beam_scores = scores_gpu
            s.parent = ref_parent.astype(np.int32)
        else:
            ref_scores = np.zeros((cfg.R, cfg.B), np.float32)
            beam_scores = torch.zeros((cfg.R, cfg.B), device=dev)
        up = gu.upload_step(s, dev)
        up["parent"] = parent_gpu
        outs.append(ctx.step(**up))
    torch.cuda.synchronize()
    assert ctx.status() == onela.ONELA_OK
    view = ctx.view()
    for r in range(cfg.R):
        for h in range(cfg.H):
            ref, chains = gu.oracle_head(sctx[r, h], steps, r, h, cfg.B, cfg.L)
            for t0 in range(cfg.L):
                got = outs[t0][r, :, h].double().cpu().numpy()
                assert np.max(np.abs(got - ref["o"][t0])) <= gu.TOL, (r, h, t0)
            for t0 in range(cfg.L):
                assert np.array_equal(view["chains"][t0, r].cpu().numpy(), chains[t0]), (r, t0)
    ctx.close()


def test_select_all_equal_scores():
    """Every candidate of a request scores the same: the flat index alone orders them, so the first flat
    indices survive; then one candidate above a 20000-way tie."""
    gu.log("select with every score equal")
    si = inputs.SelectInputs(np.zeros((2, 40), np.float32), np.zeros((2, 40, 500), np.float32))
    got = run_select(si, 300)
    assert_same(si, 300, got)
    assert np.array_equal(got[0][0], np.arange(300) // 500) and np.array_equal(got[1][0], np.arange(300) % 500)
    si = inputs.SelectInputs(np.zeros((1, 40), np.float32), np.full((1, 40, 500), -1.5, np.float32))
    si.logp[0, 39, 499] = -1.0
    got = run_select(si, 2048)
    assert_same(si, 2048, got)
    assert got[0][0, 0] == 39 and got[1][0, 0] == 499


@pytest.mark.parametrize("i", range(16))
def test_select_random_shapes(i):
    """A seeded sweep: request count, beams, candidates per beam and survivors drawn at random (survivors up to
    min(2048, candidates)), half with many exact ties; bit for bit against the oracle."""
    rng = np.random.default_rng([0x5E1E, i])
    R = int(rng.integers(1, 6))
    n_prev = int(rng.choice([1, 2, 3, 17, 64, 128, 255, 512, 1000]))
    n_cand = int(rng.choice([1, 2, 7, 31, 64, 100, 256, 1024, 3000]))
    n_beams = int(rng.integers(1, min(2048, n_prev * n_cand) + 1))
    ties = bool(i % 2)
    gu.log(f"select random {i}: R={R} n_prev={n_prev} n_cand={n_cand} n_beams={n_beams} ties={ties}")
    si = inputs.select_inputs(R, n_prev, n_cand, seed=20 + i, ties=ties)
    assert_same(si, n_beams, run_select(si, n_beams))


def test_select_reused_garbage_scratch():
    """The scratch's contents are arbitrary on entry: one buffer full of random bytes, reused by several calls
    (each finding the previous call's survivors), gives the oracle's survivors every time."""
    dev = gu.device()
    R, n_prev, n_cand, n_beams = 5, 300, 100, 256
    need = onela.onela_beam_select_scratch(R, n_prev, n_cand, n_beams)
    scratch = torch.randint(0, 256, (need,), dtype=torch.uint8, device=dev)
    for seed in range(3):
        gu.log(f"select with reused scratch, call {seed}")
        si = inputs.select_inputs(R, n_prev, n_cand, seed=40 + seed)
        got = onela.beam_select(torch.from_numpy(si.beam_scores).to(dev), torch.from_numpy(si.logp).to(dev), n_beams,
                                scratch=scratch)
        torch.cuda.synchronize()
        assert_same(si, n_beams, [x.cpu().numpy() for x in got])


def test_select_signed_zeros():
    """Scores of -0 (both addends -0) and +0 (other zero sums) rank alike, by flat index, and each keeps the sign
    of its float32 addition: the keys map both zeros to one value, so the output recomputes zero scores."""
    gu.log("select with signed zero scores")
    bs = np.zeros((2, 24), np.float32)
    lp = np.full((2, 24, 40), -3.0, np.float32)
    bs[:, ::2] = -0.0
    lp[:, :, ::3] = -0.0   # beams with bs = -0 give -0 here, beams with bs = +0 give +0
    lp[:, :, 1::3] = 0.0   # +0 for every beam
    lp[1, 5, 7] = 2.0 ** -140  # one subnormal score above the zeros
    si = inputs.SelectInputs(bs, lp)
    for n_beams in (100, 600):
        got = run_select(si, n_beams)
        assert_same(si, n_beams, got)
        assert np.any(np.signbit(got[2]) & (got[2] == 0)) and np.any(~np.signbit(got[2]) & (got[2] == 0))
