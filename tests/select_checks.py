"""Pins of the beam-selection oracle: each check takes a module exposing ``beam_select`` and raises on a
mismatch, so the same checks run on the oracle and on planted mutants of it."""

import numpy as np


def _brute(bs, lp, n_beams):
    """Pure-Python reading of the rule: rank by (score descending, flat index ascending)."""
    R, n_prev, n_cand = lp.shape
    out = []
    for r in range(R):
        cands = []
        for b in range(n_prev):
            for c in range(n_cand):
                s = float(np.float32(bs[r, b]) + np.float32(lp[r, b, c]))
                cands.append((-s, b * n_cand + c, b, c, s))
        cands.sort()
        out.append(cands[:n_beams])
    return out


def check_brute_force(mod):
    """Random tiny cases, with many exact ties (values on a coarse grid), against the Python brute force."""
    rng = np.random.default_rng(11)
    for R, n_prev, n_cand, n_beams in [(1, 1, 5, 3), (2, 3, 4, 7), (3, 5, 6, 30), (1, 4, 4, 16), (2, 7, 3, 1)]:
        bs = rng.integers(-4, 1, size=(R, n_prev)).astype(np.float32) * np.float32(0.5)
        lp = rng.integers(-6, 1, size=(R, n_prev, n_cand)).astype(np.float32) * np.float32(0.25)
        par, tok, sc = mod.beam_select(bs, lp, n_beams)
        ref = _brute(bs, lp, n_beams)
        for r in range(R):
            assert [x[2] for x in ref[r]] == list(par[r]), (R, n_prev, n_cand, n_beams, r)
            assert [x[3] for x in ref[r]] == list(tok[r])
            assert np.array_equal(np.array([x[4] for x in ref[r]], np.float32), sc[r])


def check_single_parent(mod):
    """One current beam (the first decode step): the survivors are that beam's best tokens."""
    rng = np.random.default_rng(12)
    lp = rng.standard_normal((2, 1, 50)).astype(np.float32)
    bs = np.array([[0.0], [-3.0]], np.float32)
    par, tok, sc = mod.beam_select(bs, lp, 10)
    assert np.all(par == 0)
    for r in range(2):
        assert list(tok[r]) == list(np.argsort(-lp[r, 0], kind="stable")[:10])
        assert np.array_equal(sc[r], (bs[r, 0] + lp[r, 0][tok[r]]).astype(np.float32))


def check_all_equal(mod):
    """All scores equal: the survivors are the first flat indices, in order."""
    par, tok, sc = mod.beam_select(np.zeros((1, 4), np.float32), np.full((1, 4, 3), -1.0, np.float32), 7)
    assert list(par[0]) == [0, 0, 0, 1, 1, 1, 2] and list(tok[0]) == [0, 1, 2, 0, 1, 2, 0]
    assert np.all(sc == -1.0)


def check_separated_parents(mod):
    """Parents whose scores are far apart: the best parent's tokens come first, then the next parent's."""
    rng = np.random.default_rng(13)
    lp = np.log(rng.dirichlet(np.ones(6), size=(1, 3))).astype(np.float32)
    bs = np.array([[-1000.0, 0.0, -500.0]], np.float32)
    par, tok, sc = mod.beam_select(bs, lp, 12)
    assert list(par[0]) == [1] * 6 + [2] * 6
    assert list(tok[0, :6]) == list(np.argsort(-lp[0, 1], kind="stable"))
    assert list(tok[0, 6:]) == list(np.argsort(-lp[0, 2], kind="stable"))


def check_top_set(mod):
    """Invariants on a larger random case: scores non-increasing, survivors distinct, and no candidate left
    out scores above the last survivor (nor ties it with a smaller flat index)."""
    rng = np.random.default_rng(14)
    R, n_prev, n_cand, n_beams = 3, 40, 64, 100
    bs = rng.standard_normal((R, n_prev)).astype(np.float32)
    lp = rng.standard_normal((R, n_prev, n_cand)).astype(np.float32)
    lp[:, ::7, ::5] = -np.inf
    par, tok, sc = mod.beam_select(bs, lp, n_beams)
    s = (bs[:, :, None] + lp).astype(np.float32).reshape(R, -1)
    for r in range(R):
        f = par[r].astype(np.int64) * n_cand + tok[r]
        assert len(set(f.tolist())) == n_beams
        assert np.all(sc[r][1:] <= sc[r][:-1])
        assert np.array_equal(s[r, f], sc[r])
        left = np.ones(n_prev * n_cand, bool)
        left[f] = False
        last, f_last = sc[r, -1], f[-1]
        assert not np.any(s[r, left] > last)
        assert not np.any((s[r, left] == last) & (np.nonzero(left)[0] < f_last))


def check_neg_inf_fill(mod):
    """When fewer candidates are finite than survivors are asked for, -inf candidates fill in by index."""
    lp = np.full((1, 2, 3), -np.inf, np.float32)
    lp[0, 1, 2] = -0.5
    par, tok, sc = mod.beam_select(np.zeros((1, 2), np.float32), lp, 4)
    assert list(zip(par[0], tok[0])) == [(1, 2), (0, 0), (0, 1), (0, 2)]
    assert sc[0, 0] == -0.5 and np.all(np.isneginf(sc[0, 1:]))


ALL_CHECKS = [check_brute_force, check_single_parent, check_all_equal, check_separated_parents, check_top_set,
              check_neg_inf_fill]
