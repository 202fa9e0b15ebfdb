"""CPU oracle for the large-beam Gated DeltaNet (GDN) decode step.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the CPU-baseline leg of the benchmark
may import this module.  It shares no code with the HIP library; inputs come from the seeded
generator, everything else is written here in plain numpy, in float64.

What is computed (sources are the OneLA pages):
  * "Scientific Impact Assessment: OneLA", §1 Core Contribution: one shared post-prefill state S_ctx;
    per-beam append-only transition records of size O(d_v + d_k); projection replay, because GDN
    reads the earlier state only through two vector contractions (with the key and the query); an
    ancestry index so that beams prune, reorder and fan out without moving records.
  * Same page, "Additional Observations": only two vector projections of the state are ever needed,
    so the full matrix is never rebuilt, not even during replay.
  * Same page, §2 Methodological Rigor: the method is an exact reformulation (not an approximation).
  * "OneLA: Scaling Linear-Attention Decoding to Large Beams in Generative Recommendation" (paper
    index page), "Builds on": Gated Delta Networks.  Its gated delta rule is the recurrence:
        S_t = alpha_t S_{t-1} (I - beta_t k_t k_t^T) + beta_t v_t k_t^T,    o_t = S_t q_t,
    S is d_v x d_k, alpha_t and beta_t are scalars per token and head.
  * Same page, Abstract (arXiv): a single prompt-derived state plus compact append-only records;
    only the needed state information is computed; records are never moved or copied.

The transition record is our reading of "O(d_v + d_k) per beam": the triple (alpha_t, k_t, u_t) with
u_t = beta_t (v_t - alpha_t S_{t-1} k_t), from which S_t = alpha_t S_{t-1} + u_t k_t^T.

Two independent forms of the same decode:
  * ``decode_head_fullstate``: every beam carries a dense state updated by the gated delta rule from
    its parent's state (brute force, the plain definition).
  * ``decode_head_replay``: records + ancestry chains; S_{t-1} k_t and S_t q_t come from a decayed
    S_ctx projection plus a replay of the chain's records; no d_v x d_k matrix is formed.

Conventions (our readings; the pages fix none of them):
  * Step t = 1..L.  Step 1 has one pseudo-parent (index 0, the shared state, empty chain).
  * Record placement: the record of beam b at step t lives in slot (t-1)*max_beams + b of the arena
    of its (request, head); slots are the same for every head.
  * Ancestry index: chain_t[b] lists, oldest first, the slots of the records on beam b's history;
    chain_t[b][:t-1] = chain_{t-1}[parent_t[b]], chain_t[b][t-1] = its own slot, the rest is -1;
    rows of beams >= n_beams are all -1.
  * Parents are per (request, beam), shared by every head.
"""

from __future__ import annotations

from typing import Dict, List, Sequence

import numpy as np

__all__ = [
    "gdn_step", "prefill", "sequential_outputs",
    "record_slot", "ancestry_update", "ancestry_tables",
    "decay_products", "decode_head_fullstate", "decode_head_replay",
    "decode_fullstate", "decode_replay",
]


def _f64(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float64)


# ----------------------------------------------------------------------------------------------
# The gated delta rule (dense form)
# ----------------------------------------------------------------------------------------------

def gdn_step(S, k, v, alpha, beta):
    """One gated delta rule update, batched over leading axes.

    S [..., d_v, d_k], k [..., d_k], v [..., d_v], alpha/beta [...]  ->  S' [..., d_v, d_k]

    S' = alpha * S (I - beta k k^T) + beta v k^T.  The product with the rank-one factor is applied
    as S (I - beta k k^T) = S - beta (S k) k^T, which is the same matrix without forming I.
    (Gated Delta Networks, listed under "Builds on" on the OneLA paper index page.)
    """
    S, k, v = _f64(S), _f64(k), _f64(v)
    alpha, beta = _f64(alpha), _f64(beta)
    Sk = np.einsum("...ij,...j->...i", S, k)
    S_damped = S - beta[..., None, None] * (Sk[..., :, None] * k[..., None, :])
    return alpha[..., None, None] * S_damped + beta[..., None, None] * (v[..., :, None] * k[..., None, :])


def prefill(k, v, alpha, beta, S0=None) -> np.ndarray:
    """GDN over a prompt, from S0 (default zero): the shared post-prefill state S_ctx.

    k [R, N, H, d_k], v [R, N, H, d_v], alpha/beta [R, N, H]  ->  S [R, H, d_v, d_k] float64.
    ("Scientific Impact Assessment: OneLA", §1: every beam starts from one post-prefill state.)
    """
    k, v = _f64(k), _f64(v)
    R, N, H, d_k = k.shape
    d_v = v.shape[-1]
    S = np.zeros((R, H, d_v, d_k)) if S0 is None else _f64(S0).copy()
    for n in range(N):
        S = gdn_step(S, k[:, n], v[:, n], alpha[:, n], beta[:, n])
    return S


def sequential_outputs(S0, q, k, v, alpha, beta) -> np.ndarray:
    """One sequence (one beam, no branching): o_n = S_n q_n with S_n = gdn_step(S_{n-1}, ...).

    S0 [d_v, d_k]; q, k [N, d_k]; v [N, d_v]; alpha, beta [N]  ->  o [N, d_v].
    """
    S = _f64(S0)
    out = []
    for n in range(len(alpha)):
        S = gdn_step(S, k[n], v[n], alpha[n], beta[n])
        out.append(S @ _f64(q[n]))
    return np.stack(out)


# ----------------------------------------------------------------------------------------------
# Ancestry index
# ----------------------------------------------------------------------------------------------

def record_slot(t: int, b: int, max_beams: int) -> int:
    """Arena slot of the record that beam b appends at step t (1-based)."""
    return (t - 1) * max_beams + b


def ancestry_update(chain_prev: np.ndarray, parent: np.ndarray, t: int, max_beams: int,
                    max_steps: int) -> np.ndarray:
    """Chain table after step t for one request.

    chain_prev: [B_prev, max_steps] int32 (for t = 1: one row, all -1); parent: [n] ints in [0, B_prev).
    Returns [max_beams, max_steps] int32.  ("Scientific Impact Assessment: OneLA", §1 item (3): the
    ancestry index separates logical beam evolution from where records physically sit.)
    """
    n = len(parent)
    out = np.full((max_beams, max_steps), -1, dtype=np.int32)
    for b in range(n):
        p = int(parent[b])
        if not 0 <= p < chain_prev.shape[0]:
            raise ValueError(f"parent {p} of beam {b} out of range [0, {chain_prev.shape[0]})")
        out[b, : t - 1] = chain_prev[p, : t - 1]
        out[b, t - 1] = record_slot(t, b, max_beams)
    return out


def ancestry_tables(parents: Sequence[np.ndarray], max_beams: int, max_steps: int) -> List[np.ndarray]:
    """Chain tables after every step of one request's decode, from its per-step parent arrays."""
    chain = np.full((1, max_steps), -1, dtype=np.int32)
    tables = []
    for t, par in enumerate(parents, start=1):
        chain = ancestry_update(chain, par, t, max_beams, max_steps)
        tables.append(chain)
    return tables


# ----------------------------------------------------------------------------------------------
# Form 1: FullState (every beam keeps a dense state)
# ----------------------------------------------------------------------------------------------

def decode_head_fullstate(S_ctx, q, k, v, alpha, beta, parents) -> List[np.ndarray]:
    """Dense per-beam states for one (request, head).

    S_ctx [d_v, d_k]; per step t: q[t], k[t] [B_t, d_k], v[t] [B_t, d_v], alpha[t], beta[t] [B_t],
    parents[t] [B_t].  Returns o per step, [B_t, d_v] float64.
    (Paper index page, Abstract: the approach that materialises a full state for every beam.)
    """
    states = _f64(S_ctx)[None]                       # step 0: the single shared state
    outs = []
    for t in range(len(parents)):
        par = np.asarray(parents[t], dtype=np.int64)
        S = gdn_step(states[par], k[t], v[t], alpha[t], beta[t])
        outs.append(np.einsum("bij,bj->bi", S, _f64(q[t])))
        states = S
    return outs


# ----------------------------------------------------------------------------------------------
# Form 2: record replay over the ancestry index
# ----------------------------------------------------------------------------------------------

def decay_products(chain_alpha: np.ndarray):
    """Decays along chains.  chain_alpha [B, n]: alpha of each chain record, oldest first.

    Returns (A [B], c [B, n]): A = product of all n alphas; c[:, j] = product of the alphas of the
    records after j.  Unrolling S_j = alpha_j S_{j-1} + u_j k_j^T along a chain gives
    S_{t-1} = A S_ctx + sum_j c_j u_j k_j^T.
    """
    B, n = chain_alpha.shape
    c = np.ones((B, n))
    for j in range(n):
        for i in range(j + 1, n):
            c[:, j] *= chain_alpha[:, i]
    A = np.ones(B)
    for i in range(n):
        A *= chain_alpha[:, i]
    return A, c


def decode_head_replay(S_ctx, q, k, v, alpha, beta, chains, max_beams: int, max_steps: int) -> Dict:
    """Projection replay for one (request, head).

    chains[t]: [max_beams, max_steps] chain table after step t+1 (from ``ancestry_tables``).
    Returns dict with  o: list of [B_t, d_v];  K [slots, d_k], U [slots, d_v], alpha [slots] arenas
    (float64, NaN where nothing was written);  p: list of S_{t-1} k_t per step.
    ("Scientific Impact Assessment: OneLA", §1 items (1)-(2), "Additional Observations".)
    """
    S_ctx = _f64(S_ctx)
    d_v, d_k = S_ctx.shape
    slots = max_beams * max_steps
    K = np.full((slots, d_k), np.nan)
    U = np.full((slots, d_v), np.nan)
    Aar = np.full(slots, np.nan)
    outs, ps = [], []
    for t0 in range(len(chains)):
        t = t0 + 1
        kt, qt, vt = _f64(k[t0]), _f64(q[t0]), _f64(v[t0])
        at, bt = _f64(alpha[t0]), _f64(beta[t0])
        B = len(at)
        ch = chains[t0][:B, : t - 1].astype(np.int64)          # parent's chain: steps 1..t-1
        A, c = decay_products(Aar[ch])
        Kc, Uc = K[ch], U[ch]                                   # [B, t-1, d_k], [B, t-1, d_v]
        # key projection  p = S_{t-1} k_t
        proj_k = np.einsum("bjd,bd->bj", Kc, kt)
        p = A[:, None] * (kt @ S_ctx.T) + np.einsum("bj,bjv->bv", c * proj_k, Uc)
        u = bt[:, None] * (vt - at[:, None] * p)
        # query projection of the post-update state  S_t q_t = alpha_t S_{t-1} q_t + (k_t . q_t) u_t
        proj_q = np.einsum("bjd,bd->bj", Kc, qt)
        Sq_prev = A[:, None] * (qt @ S_ctx.T) + np.einsum("bj,bjv->bv", c * proj_q, Uc)
        o = at[:, None] * Sq_prev + np.sum(kt * qt, axis=1)[:, None] * u
        own = chains[t0][np.arange(B), t - 1].astype(np.int64)  # the slot each beam appends to
        K[own], U[own], Aar[own] = kt, u, at
        outs.append(o)
        ps.append(p)
    return {"o": outs, "K": K, "U": U, "alpha": Aar, "p": ps}


# ----------------------------------------------------------------------------------------------
# Whole-batch wrappers: R requests x H heads, inputs laid out as the decode step receives them
# ----------------------------------------------------------------------------------------------

def _head_inputs(steps, r, h):
    """Slice (request r, head h) out of per-step arrays q,k [R,B,H,d_k], v [R,B,H,d_v], alpha/beta [R,B,H]."""
    q = [s["q"][r, :, h] for s in steps]
    k = [s["k"][r, :, h] for s in steps]
    v = [s["v"][r, :, h] for s in steps]
    a = [s["alpha"][r, :, h] for s in steps]
    b = [s["beta"][r, :, h] for s in steps]
    return q, k, v, a, b


def decode_fullstate(S_ctx, steps, heads=None) -> Dict:
    """Form 1 over requests and heads.  steps: list of dicts with q, k, v, alpha, beta (float arrays in
    the step layout) and parent [R, B].  ``heads`` optionally restricts to a list of (r, h).
    Returns {"o": {(r, h): [o_t [B_t, d_v]]}}."""
    R, H = S_ctx.shape[:2]
    heads = [(r, h) for r in range(R) for h in range(H)] if heads is None else heads
    out = {}
    for r, h in heads:
        q, k, v, a, b = _head_inputs(steps, r, h)
        out[(r, h)] = decode_head_fullstate(S_ctx[r, h], q, k, v, a, b, [s["parent"][r] for s in steps])
    return {"o": out}


def decode_replay(S_ctx, steps, max_beams: int, max_steps: int, heads=None) -> Dict:
    """Form 2 over requests and heads (same arguments as ``decode_fullstate``).
    Returns {"chains": {r: [tables]}, "heads": {(r, h): decode_head_replay(...)}}."""
    R, H = S_ctx.shape[:2]
    heads = [(r, h) for r in range(R) for h in range(H)] if heads is None else heads
    chains = {}
    res = {}
    for r, h in heads:
        if r not in chains:
            chains[r] = ancestry_tables([s["parent"][r] for s in steps], max_beams, max_steps)
        q, k, v, a, b = _head_inputs(steps, r, h)
        res[(r, h)] = decode_head_replay(S_ctx[r, h], q, k, v, a, b, chains[r], max_beams, max_steps)
    return {"chains": chains, "heads": res}
