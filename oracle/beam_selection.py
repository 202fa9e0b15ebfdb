"""CPU oracle for the beam-selection step that produces the next decode step's parents.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the CPU-baseline leg of the benchmark
may import this module.  It shares no code with the HIP library.

What is computed.  "Scientific Impact Assessment: OneLA", §1 Core Contribution: beams are pruned,
reordered and fanned out between decode steps, and each surviving beam names its parent; the ancestry
index then follows those parent links.  The pages do not spell out the selection rule.  Our reading is
the plain beam-search step:
  * every current beam b (of n_prev) proposes every candidate token c (of n_cand) with the score
        s[b, c] = beam_score[b] + logp[b, c]          (one float32 addition, round to nearest even);
  * the n_beams candidates with the highest scores survive; among equal scores the candidate with the
    smaller flat index f = b * n_cand + c ranks first, so the result is unique;
  * survivors are listed best first: new beam i has parent[i] = f_i // n_cand, token[i] = f_i % n_cand
    and score[i] = s_i.
The same rule is applied to every request independently.  NaN scores have no rank under this rule and
are outside its domain; -inf is an ordinary (lowest) score.
"""

from __future__ import annotations

import numpy as np

__all__ = ["candidate_scores", "beam_select"]


def candidate_scores(beam_scores: np.ndarray, logp: np.ndarray) -> np.ndarray:
    """s[r, b, c] = beam_scores[r, b] + logp[r, b, c], one float32 addition per candidate.

    beam_scores: [R, n_prev] float32; logp: [R, n_prev, n_cand] float32.  Returns float32 [R, n_prev, n_cand].
    """
    bs = np.asarray(beam_scores, dtype=np.float32)
    lp = np.asarray(logp, dtype=np.float32)
    if bs.ndim != 2 or lp.ndim != 3 or lp.shape[:2] != bs.shape:
        raise ValueError(f"shapes {bs.shape} and {lp.shape} do not match [R, n_prev] and [R, n_prev, n_cand]")
    return (bs[:, :, None] + lp).astype(np.float32)


def beam_select(beam_scores: np.ndarray, logp: np.ndarray, n_beams: int):
    """Top-n_beams candidates per request, best first, ties to the smaller flat index.

    Returns (parent [R, n_beams] int32, token [R, n_beams] int32, score [R, n_beams] float32).
    """
    s = candidate_scores(beam_scores, logp)
    R, n_prev, n_cand = s.shape
    n = n_prev * n_cand
    if not 1 <= n_beams <= n:
        raise ValueError(f"n_beams {n_beams} must be in 1..{n}")
    flat = s.reshape(R, n)
    if np.isnan(flat).any():
        raise ValueError("NaN scores have no rank")
    parent = np.empty((R, n_beams), np.int32)
    token = np.empty((R, n_beams), np.int32)
    score = np.empty((R, n_beams), np.float32)
    idx = np.arange(n, dtype=np.int64)
    for r in range(R):
        # primary key: score, descending; secondary key: flat index, ascending (lexsort sorts by the last key)
        order = np.lexsort((idx, -flat[r].astype(np.float64)))[:n_beams]
        parent[r] = order // n_cand
        token[r] = order % n_cand
        score[r] = flat[r, order]
    return parent, token, score
