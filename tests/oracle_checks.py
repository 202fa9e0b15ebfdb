"""Pins of the CPU oracle, written as plain functions of the oracle module.

Each ``check_*`` takes the oracle module and raises AssertionError (or any exception) when the module
is wrong.  ``test_oracle_pins.py`` runs them on the real oracle; ``test_oracle_mutants.py`` runs them on
copies of the oracle with planted mistakes and asserts that some check catches each mistake.

None of these checks re-types the oracle's formulas: they compare its two independent forms with each
other, with exact rational arithmetic of the gated delta rule's matrix form, with closed forms that the
recurrence implies, with invariants, and with a hand-derived ancestry table.
"""

from fractions import Fraction

import numpy as np


# ----------------------------------------------------------------------------------------------
# Problem builders
# ----------------------------------------------------------------------------------------------

def _unit(x):
    return x / np.linalg.norm(x, axis=-1, keepdims=True)


def random_problem(seed, R=2, H=2, d_k=5, d_v=4, beams=(4, 4, 4, 4), alpha_lo=0.5, sctx_scale=1.0):
    """Random fp64 problem; ``beams`` gives the beam count of each step (so its length is L)."""
    rng = np.random.default_rng(seed)
    S_ctx = rng.standard_normal((R, H, d_v, d_k)) * sctx_scale
    steps = []
    b_prev = 1
    for B in beams:
        steps.append(dict(
            q=_unit(rng.standard_normal((R, B, H, d_k))),
            k=_unit(rng.standard_normal((R, B, H, d_k))),
            v=rng.standard_normal((R, B, H, d_v)),
            alpha=rng.uniform(alpha_lo, 1.0, (R, B, H)),
            beta=rng.uniform(0.0, 1.0, (R, B, H)),
            parent=rng.integers(0, b_prev, (R, B)).astype(np.int32),
        ))
        b_prev = B
    return S_ctx, steps


def run_both(orc, S_ctx, steps, max_beams=None, max_steps=None):
    max_beams = max(len(s["parent"][0]) for s in steps) if max_beams is None else max_beams
    max_steps = len(steps) if max_steps is None else max_steps
    fs = orc.decode_fullstate(S_ctx, steps)
    rp = orc.decode_replay(S_ctx, steps, max_beams, max_steps)
    return fs, rp


def ancestor(steps, r, t, b, j):
    """Index of the beam at step j (1-based) on the history of beam b at step t, by walking parents."""
    while t > j:
        b = int(steps[t - 1]["parent"][r, b])
        t -= 1
    return b


# ----------------------------------------------------------------------------------------------
# Checks
# ----------------------------------------------------------------------------------------------

def check_forms_agree(orc):
    """FullState (dense, brute force) and record replay give the same outputs on tiny inputs."""
    cases = [
        dict(seed=1),
        dict(seed=2, R=1, H=3, d_k=3, d_v=7, beams=(5, 5, 5, 5, 5)),
        dict(seed=3, R=3, H=1, d_k=8, d_v=8, beams=(2, 6, 3, 8, 8, 1, 4, 8), alpha_lo=0.2),
        dict(seed=4, R=1, H=1, d_k=16, d_v=16, beams=(8, 8, 8)),
        dict(seed=5, R=2, H=2, d_k=4, d_v=6, beams=(3, 3), sctx_scale=0.0),
    ]
    for c in cases:
        S_ctx, steps = random_problem(**c)
        fs, rp = run_both(orc, S_ctx, steps)
        for key, o_fs in fs["o"].items():
            o_rp = rp["heads"][key]["o"]
            for t, (a, b) in enumerate(zip(o_fs, o_rp)):
                assert a.shape == b.shape, (c, key, t)
                err = np.max(np.abs(a - b)) if a.size else 0.0
                assert err < 1e-12, (c, key, t, err)


def check_records(orc):
    """Each beam's record holds its own alpha and k, in the slot of the placement rule; u is zero iff beta is."""
    S_ctx, steps = random_problem(11, beams=(4, 4, 4))
    for s in steps:
        s["beta"][..., 0] = 0.0            # head 0: beta = 0 everywhere
    rp = orc.decode_replay(S_ctx, steps, 4, 3)
    for (r, h), res in rp["heads"].items():
        for t, s in enumerate(steps, start=1):
            for b in range(4):
                slot = (t - 1) * 4 + b
                assert np.array_equal(res["K"][slot], s["k"][r, b, h])
                assert res["alpha"][slot] == s["alpha"][r, b, h]
                if h == 0:
                    assert np.all(res["U"][slot] == 0.0)
                else:
                    assert np.all(np.isfinite(res["U"][slot])) and np.any(res["U"][slot] != 0.0)


def _exact_gdn(S, k, v, a, b):
    """Gated delta rule in exact rationals, in its matrix form a*S(I - b k k^T) + b v k^T."""
    dv, dk = len(S), len(S[0])
    M = [[(Fraction(1) if i == j else Fraction(0)) - b * k[i] * k[j] for j in range(dk)] for i in range(dk)]
    SM = [[sum(S[i][l] * M[l][j] for l in range(dk)) for j in range(dk)] for i in range(dv)]
    return [[a * SM[i][j] + b * v[i] * k[j] for j in range(dk)] for i in range(dv)]


def _exact_matvec(S, x):
    return [sum(S[i][j] * x[j] for j in range(len(x))) for i in range(len(S))]


def check_exact_rational(orc):
    """Brute force in exact rationals on a 2x3 state, 3 beams, 3 steps, hand-picked rational inputs."""
    F = Fraction
    S_ctx = [[F(1, 2), F(-1), F(3, 4)], [F(2), F(1, 3), F(-5, 4)]]                # d_v=2, d_k=3
    keys = [(F(3, 5), F(4, 5), F(0)), (F(0), F(3, 5), F(-4, 5)), (F(2, 3), F(1, 3), F(2, 3)),
            (F(-1), F(0), F(0)), (F(0), F(0), F(1)), (F(6, 7), F(2, 7), F(-3, 7))]
    qs = [(F(1), F(-1, 2), F(1, 4)), (F(1, 3), F(2), F(-1)), (F(-3, 2), F(0), F(1, 2))]
    parents = [[0, 0, 0], [2, 0, 2], [1, 1, 0]]
    L, B = 3, 3
    # per step, per beam rational inputs
    kk = [[keys[(t * 2 + b) % 6] for b in range(B)] for t in range(L)]
    qq = [[qs[(t + b) % 3] for b in range(B)] for t in range(L)]
    vv = [[(F(t + 1, 2) - b, F(b + 1, 3) - t) for b in range(B)] for t in range(L)]
    aa = [[F(1, 2) + F(b + t, 8) for b in range(B)] for t in range(L)]
    bb = [[F(1, 3) + F(t * B + b, 12) for b in range(B)] for t in range(L)]
    expect = []
    states = [S_ctx]
    for t in range(L):
        new, o = [], []
        for b in range(B):
            S = _exact_gdn(states[parents[t][b]], kk[t][b], vv[t][b], aa[t][b], bb[t][b])
            new.append(S)
            o.append(_exact_matvec(S, qq[t][b]))
        states = new
        expect.append(o)
    f = lambda x: np.array(x, dtype=np.float64)  # noqa: E731
    steps = [dict(q=f(qq[t])[None, :, None], k=f(kk[t])[None, :, None], v=f(vv[t])[None, :, None],
                  alpha=f(aa[t])[None, :, None], beta=f(bb[t])[None, :, None],
                  parent=np.array([parents[t]], dtype=np.int32)) for t in range(L)]
    S_np = f(S_ctx)[None, None]
    fs, rp = run_both(orc, S_np, steps)
    for t in range(L):
        ex = np.array([[float(x) for x in row] for row in expect[t]])
        assert np.max(np.abs(fs["o"][(0, 0)][t] - ex)) < 1e-14, ("fullstate", t)
        assert np.max(np.abs(rp["heads"][(0, 0)]["o"][t] - ex)) < 1e-14, ("replay", t)


def check_beta_zero(orc):
    """beta = 0: no record carries anything (u = 0) and S_t = (product of alphas along the history,
    this step's included) S_ctx, so o_t = that product times S_ctx q_t."""
    S_ctx, steps = random_problem(21, R=2, H=2, d_k=6, d_v=5, beams=(5, 5, 5, 5))
    for s in steps:
        s["beta"][:] = 0.0
    fs, rp = run_both(orc, S_ctx, steps)
    for (r, h), o_fs in fs["o"].items():
        for t in range(1, len(steps) + 1):
            for b in range(5):
                prod, bb = 1.0, b
                for j in range(t, 0, -1):
                    prod *= steps[j - 1]["alpha"][r, bb, h]
                    bb = int(steps[j - 1]["parent"][r, bb])
                ex = prod * (S_ctx[r, h] @ steps[t - 1]["q"][r, b, h])
                assert np.max(np.abs(o_fs[t - 1][b] - ex)) < 1e-12
                assert np.max(np.abs(rp["heads"][(r, h)]["o"][t - 1][b] - ex)) < 1e-12
        U = rp["heads"][(r, h)]["U"]
        assert np.all(U[np.isfinite(U)] == 0.0)


def check_orthonormal_recall(orc):
    """alpha = beta = 1 with keys orthonormal along every history: S_t k_j = v_j for each record j on
    the history (the delta rule overwrites the value stored under a key) and S_t x = S_ctx x for x
    orthogonal to every key used."""
    rng = np.random.default_rng(31)
    R, H, d_k, d_v, B, L = 2, 2, 7, 4, 4, 5
    Q, _ = np.linalg.qr(rng.standard_normal((d_k, d_k)))
    S_ctx = rng.standard_normal((R, H, d_v, d_k))
    steps = []
    b_prev = 1
    for t in range(1, L + 1):
        k = np.broadcast_to(Q[:, t - 1], (R, B, H, d_k)).copy()
        j = rng.integers(1, t + 2, (R, B, H))          # j == t+1 means "a direction no key used"
        q = np.where((j <= t)[..., None], Q[:, np.minimum(j, t) - 1].transpose(1, 2, 3, 0), Q[:, L])
        steps.append(dict(q=q, k=k, v=rng.standard_normal((R, B, H, d_v)), alpha=np.ones((R, B, H)),
                          beta=np.ones((R, B, H)),
                          parent=rng.integers(0, b_prev, (R, B)).astype(np.int32), j=j))
        b_prev = B
    fs, rp = run_both(orc, S_ctx, steps)
    for (r, h), o_fs in fs["o"].items():
        for t in range(1, L + 1):
            for b in range(B):
                jj = int(steps[t - 1]["j"][r, b, h])
                if jj <= t:
                    anc = ancestor(steps, r, t, b, jj)
                    ex = steps[jj - 1]["v"][r, anc, h]
                else:
                    ex = S_ctx[r, h] @ Q[:, L]
                assert np.max(np.abs(o_fs[t - 1][b] - ex)) < 1e-12, (r, h, t, b, jj)
                assert np.max(np.abs(rp["heads"][(r, h)]["o"][t - 1][b] - ex)) < 1e-12, (r, h, t, b, jj)


def check_superposition(orc):
    """The recurrence is linear in (S_ctx, v) jointly for fixed keys, alphas and betas, so
    o(S_ctx, v) = o(S_ctx, 0) + o(0, v), and o(2 S_ctx, 0) = 2 o(S_ctx, 0)."""
    S_ctx, steps = random_problem(41, R=1, H=2, d_k=5, d_v=3, beams=(3, 4, 4, 2))
    zero_v = [dict(s, v=np.zeros_like(s["v"])) for s in steps]
    for form in ("fullstate", "replay"):
        def outs(S, st):
            if form == "fullstate":
                return orc.decode_fullstate(S, st)["o"]
            return {key: v["o"] for key, v in orc.decode_replay(S, st, 4, 4)["heads"].items()}
        full = outs(S_ctx, steps)
        a = outs(S_ctx, zero_v)
        b = outs(np.zeros_like(S_ctx), steps)
        dbl = outs(2 * S_ctx, zero_v)
        for key in full:
            for t in range(len(steps)):
                assert np.max(np.abs(full[key][t] - a[key][t] - b[key][t])) < 1e-12, (form, key, t)
                assert np.max(np.abs(dbl[key][t] - 2 * a[key][t])) < 1e-12, (form, key, t)


def check_single_beam_is_sequential(orc):
    """One beam (every parent 0) is plain sequential GDN continued from S_ctx."""
    S_ctx, steps = random_problem(51, R=1, H=1, d_k=6, d_v=6, beams=(1,) * 7)
    rp = orc.decode_replay(S_ctx, steps, 1, 7)
    g = lambda name: np.stack([s[name][0, 0, 0] for s in steps])  # noqa: E731
    seq = orc.sequential_outputs(S_ctx[0, 0], g("q"), g("k"), g("v"), g("alpha"), g("beta"))
    got = np.stack([o[0] for o in rp["heads"][(0, 0)]["o"]])
    assert np.max(np.abs(seq - got)) < 1e-12


def check_prefill(orc):
    """Prefill: beta = 0 decays S0 by the product of alphas; alpha = beta = 1 with orthonormal keys
    stores v_n under k_n; exact rationals on a 2x2 state."""
    rng = np.random.default_rng(61)
    R, N, H, d = 2, 6, 3, 6
    S0 = rng.standard_normal((R, H, d, d))
    k = _unit(rng.standard_normal((R, N, H, d)))
    v = rng.standard_normal((R, N, H, d))
    alpha = rng.uniform(0.5, 1, (R, N, H))
    S = orc.prefill(k, v, alpha, np.zeros((R, N, H)), S0)
    assert np.max(np.abs(S - np.prod(alpha, axis=1)[..., None, None] * S0)) < 1e-13
    assert np.all(orc.prefill(k, v, alpha, np.zeros((R, N, H))) == 0.0)
    Q, _ = np.linalg.qr(rng.standard_normal((d, d)))
    kq = np.broadcast_to(Q[:, :N - 1].T[None, :, None, :], (R, N - 1, H, d)).copy()
    S = orc.prefill(kq, v[:, : N - 1], np.ones((R, N - 1, H)), np.ones((R, N - 1, H)))
    for n in range(N - 1):
        assert np.max(np.abs(S @ Q[:, n] - v[:, n])) < 1e-12
    assert np.max(np.abs(S @ Q[:, N - 1])) < 1e-12
    F = Fraction
    ks = [(F(3, 5), F(4, 5)), (F(0), F(1)), (F(-5, 13), F(12, 13))]
    vs = [(F(1), F(-2)), (F(1, 2), F(3)), (F(-1, 3), F(1, 7))]
    al = [F(1, 2), F(3, 4), F(9, 10)]
    be = [F(1, 5), F(1), F(2, 3)]
    Sx = [[F(0), F(0)], [F(0), F(0)]]
    for n in range(3):
        Sx = _exact_gdn(Sx, ks[n], vs[n], al[n], be[n])
    f = lambda x: np.array(x, dtype=np.float64)  # noqa: E731
    got = orc.prefill(f(ks)[None, :, None], f(vs)[None, :, None], f(al)[None, :, None], f(be)[None, :, None])
    assert np.max(np.abs(got[0, 0] - f([[float(x) for x in row] for row in Sx]))) < 1e-15


def check_relabel_invariance(orc):
    """Permuting the new beams of step t (and remapping the parents of step t+1) permutes the outputs
    of step t and leaves every later output unchanged."""
    S_ctx, steps = random_problem(71, R=2, H=2, d_k=4, d_v=5, beams=(5, 5, 5, 5))
    t_perm = 2                                   # 1-based step whose beams are relabelled
    perm = np.array([3, 0, 4, 1, 2])             # old beam b moves to position perm[b]
    inv = np.argsort(perm)
    p_steps = [dict(s) for s in steps]
    s = steps[t_perm - 1]
    p_steps[t_perm - 1] = {key: (val[:, inv] if key != "j" else val) for key, val in s.items()}
    nxt = steps[t_perm]
    p_steps[t_perm] = dict(nxt, parent=perm[nxt["parent"]].astype(np.int32))
    for run in (lambda st: orc.decode_fullstate(S_ctx, st)["o"],
                lambda st: {key: v["o"] for key, v in orc.decode_replay(S_ctx, st, 5, 4)["heads"].items()}):
        a, b = run(steps), run(p_steps)
        for key in a:
            for t in range(len(steps)):
                ref = a[key][t][inv] if t == t_perm - 1 else a[key][t]
                assert np.max(np.abs(ref - b[key][t])) < 1e-12, (key, t)


def check_duplicate_beams(orc):
    """Two beams with the same parent and the same inputs produce the same output."""
    S_ctx, steps = random_problem(81, R=1, H=2, d_k=5, d_v=5, beams=(4, 4, 4))
    for s in steps[1:]:
        for key in ("q", "k", "v", "alpha", "beta"):
            s[key][:, 3] = s[key][:, 1]
        s["parent"][:, 3] = s["parent"][:, 1]
    fs, rp = run_both(orc, S_ctx, steps)
    for key in fs["o"]:
        for t in (1, 2):
            assert np.array_equal(fs["o"][key][t][3], fs["o"][key][t][1])
            assert np.array_equal(rp["heads"][key]["o"][t][3], rp["heads"][key]["o"][t][1])


def check_ancestry_hand_table(orc):
    """Chain tables for max_beams = 3, max_steps = 3, worked out by hand from the placement rule
    slot(t, b) = 3 (t - 1) + b and the parents below (step 3 keeps only 2 beams)."""
    parents = [np.array([0, 0, 0]), np.array([2, 0, 0]), np.array([1, 2])]
    hand = [
        [[0, -1, -1], [1, -1, -1], [2, -1, -1]],
        [[2, 3, -1], [0, 4, -1], [0, 5, -1]],
        [[0, 4, 6], [0, 5, 7], [-1, -1, -1]],
    ]
    got = orc.ancestry_tables(parents, 3, 3)
    for t in range(3):
        assert got[t].dtype == np.int32
        assert got[t].tolist() == hand[t], (t, got[t].tolist())
    bad = False
    try:
        orc.ancestry_update(got[0], np.array([0, 3]), 2, 3, 3)
    except ValueError:
        bad = True
    assert bad, "out-of-range parent must be rejected"


ALL_CHECKS = [
    check_forms_agree, check_records, check_exact_rational, check_beta_zero, check_orthonormal_recall,
    check_superposition, check_single_beam_is_sequential, check_prefill, check_relabel_invariance,
    check_duplicate_beams, check_ancestry_hand_table,
]
