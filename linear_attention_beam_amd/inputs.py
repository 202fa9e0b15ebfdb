"""Seeded synthetic inputs for the large-beam Gated DeltaNet decode step.

This module draws random numbers and encodes them; it holds none of the decode arithmetic.  The
oracle (under ``oracle/``) and the HIP path both take their inputs from here and from nowhere else.

The pages publish no workload: the review of OneLA ("Scientific Impact Assessment: OneLA", §2
Methodological Rigor and §5 Strengths & Limitations) says the industrial traffic and the 405 operator
shapes are not released.  The five configurations below stand in for that sweep.  They keep its axes
(request count, beam width, decode length, recurrent geometry) and the structure the abstract names
(hundreds of beams that share one prompt-derived state and diverge over a few decode steps).

Recipe (every configuration):
  * q, k ~ N(0, 1) drawn in float32, divided by their float32 L2 norm, then rounded once to the
    decode dtype (bfloat16 round-to-nearest-even for the bf16 configurations).  Never renormalised.
  * v ~ N(0, 1) float32, rounded to the decode dtype.
  * alpha ~ U(alpha_lo, 1), beta ~ U(0, 1), float32.
  * parents: step 1 has a single pseudo-parent (index 0, the shared state).  Later steps draw each
    new beam's parent independently: uniformly over the previous beams, or from a Zipf law truncated to
    ranks 1..B_prev (P(rank) proportional to rank^-s, parent = rank - 1, beam index = score rank).
  * S_ctx: either N(0, std^2) directly, or the inputs of a prefill of N GDN steps from the zero state
    with the same k/v/alpha/beta distributions (float32, not rounded).  Turning those prefill inputs
    into S_ctx is GDN arithmetic and is done by the caller (the oracle's prefill or the GPU prefill).
  * Streams: numpy PCG64 generators seeded by SeedSequence([0x0E1A, config index, stream, seed, ...]):
    stream 0 draws S_ctx (one generator) or the prefill inputs (one generator per request, drawing
    k, v, alpha, beta in that order); stream 1 the decode inputs (one generator per step and request,
    drawing q, k, v, alpha, beta); stream 2 the parents (one generator per step); stream 3 the
    candidate scores of the beam selection (``select_inputs``).  Chunks are drawn in parallel threads;
    the values do not depend on the thread count.
"""

from __future__ import annotations

import dataclasses
import os
from concurrent.futures import ThreadPoolExecutor
from typing import List, Optional

import numpy as np

__all__ = [
    "Config", "CONFIGS", "config", "StepInputs", "PrefillInputs",
    "decode_inputs", "prefill_inputs", "direct_sctx", "parents_for_step",
    "f32_to_bf16_bits", "bf16_bits_to_f32", "SelectInputs", "select_inputs",
]

_SEED_TAG = 0x0E1A


@dataclasses.dataclass(frozen=True)
class Config:
    """One synthetic workload: R requests x H heads x B beams, L decode steps, state d_v x d_k."""

    index: int
    name: str
    R: int
    H: int
    d_k: int
    d_v: int
    B: int
    L: int
    qkv_dtype: str          # "f32" or "bf16"
    alpha_lo: float         # alpha ~ U(alpha_lo, 1)
    prefill_steps: int      # 0: S_ctx drawn directly with sctx_std
    sctx_std: float
    parent_law: str         # "uniform" or "zipf"
    zipf_s: float

    @property
    def beam_tokens(self) -> int:
        """Beam-tokens in one full decode: one beam advanced one step through all H heads."""
        return self.R * self.B * self.L

    @property
    def in_bytes(self) -> int:
        return 4 if self.qkv_dtype == "f32" else 2


CONFIGS = [
    Config(0, "tiny: R=1 H=1 d=16 B=8 L=3 fp32", 1, 1, 16, 16, 8, 3, "f32", 0.9, 0, 0.1, "uniform", 0.0),
    Config(1, "R=1 H=16 d=128 B=128 L=4 bf16 prefill1024 zipf1.1", 1, 16, 128, 128, 128, 4, "bf16", 0.9,
           1024, 0.0, "zipf", 1.1),
    Config(2, "R=8 H=16 d=128 B=256 L=4 bf16 prefill1024 zipf1.1", 8, 16, 128, 128, 256, 4, "bf16", 0.9,
           1024, 0.0, "zipf", 1.1),
    Config(3, "R=32 H=16 d=128 B=512 L=8 bf16 prefill5120 zipf1.5", 32, 16, 128, 128, 512, 8, "bf16", 0.9,
           5120, 0.0, "zipf", 1.5),
    Config(4, "R=16 H=32 dk=128 dv=256 B=512 L=6 bf16 prefill5120 zipf1.1", 16, 32, 128, 256, 512, 6,
           "bf16", 0.95, 5120, 0.0, "zipf", 1.1),
]


def config(index: int, **overrides) -> Config:
    """Return configuration ``index``, optionally with fields replaced (for scaled-down test cases)."""
    return dataclasses.replace(CONFIGS[index], **overrides) if overrides else CONFIGS[index]


# ----------------------------------------------------------------------------------------------
# bfloat16 encoding (numpy has no bf16 type: values travel as their 16-bit patterns)
# ----------------------------------------------------------------------------------------------

def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (round to nearest, ties to even); return the uint16 bit patterns."""
    bits = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (bits >> np.uint32(16)) & np.uint32(1)
    rounded = bits + np.uint32(0x7FFF) + lsb
    return (rounded >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact float32 values of bfloat16 bit patterns."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _rng(cfg: Config, stream: int, seed: int, *chunk: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([_SEED_TAG, cfg.index, stream, seed, *chunk])))


def _threads() -> int:
    return max(1, min(16, len(os.sched_getaffinity(0))))


def _unit_rows_f32(rng: np.random.Generator, shape) -> np.ndarray:
    x = rng.standard_normal(shape, dtype=np.float32)
    norm = np.sqrt(np.einsum("...i,...i->...", x, x, dtype=np.float32))
    x /= norm[..., None]
    return x


# ----------------------------------------------------------------------------------------------
# Decode-step inputs
# ----------------------------------------------------------------------------------------------

@dataclasses.dataclass
class StepInputs:
    """Inputs of one decode step.  q, k: [R, B, H, d_k]; v: [R, B, H, d_v]; alpha, beta: [R, B, H];
    parent: [R, B] int32.  For bf16 configurations ``q``/``k``/``v`` hold uint16 bit patterns."""

    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    alpha: np.ndarray
    beta: np.ndarray
    parent: np.ndarray
    dtype: str

    def as_f32(self, name: str) -> np.ndarray:
        """The exact float32 values of q, k or v."""
        a = getattr(self, name)
        return bf16_bits_to_f32(a) if self.dtype == "bf16" else a


def parents_for_step(cfg: Config, rng: np.random.Generator, t: int, b_prev: int, n: int) -> np.ndarray:
    """Parents of the n new beams of step t (1-based) for every request: [R, n] int32 in [0, b_prev)."""
    if t == 1 or b_prev == 1:
        return np.zeros((cfg.R, n), dtype=np.int32)
    if cfg.parent_law == "uniform":
        return rng.integers(0, b_prev, size=(cfg.R, n), dtype=np.int64).astype(np.int32)
    ranks = np.arange(1, b_prev + 1, dtype=np.float64)
    w = ranks ** (-cfg.zipf_s)
    cdf = np.cumsum(w) / w.sum()
    cdf[-1] = 1.0
    u = rng.random((cfg.R, n))
    idx = np.searchsorted(cdf, u, side="right")
    return np.minimum(idx, b_prev - 1).astype(np.int32)


def decode_inputs(cfg: Config, seed: int = 0, steps: Optional[int] = None) -> List[StepInputs]:
    """All decode-step inputs of one configuration (``steps`` defaults to cfg.L)."""
    steps = cfg.L if steps is None else steps
    R, B, H = cfg.R, cfg.B, cfg.H
    bf16 = cfg.qkv_dtype == "bf16"
    enc = f32_to_bf16_bits if bf16 else (lambda x: x)
    dt = np.uint16 if bf16 else np.float32
    out = []
    for t in range(1, steps + 1):
        q = np.empty((R, B, H, cfg.d_k), dt)
        k = np.empty((R, B, H, cfg.d_k), dt)
        v = np.empty((R, B, H, cfg.d_v), dt)
        alpha = np.empty((R, B, H), np.float32)
        beta = np.empty((R, B, H), np.float32)

        def fill(r, t=t, q=q, k=k, v=v, alpha=alpha, beta=beta):
            rng = _rng(cfg, 1, seed, t, r)
            q[r] = enc(_unit_rows_f32(rng, (B, H, cfg.d_k)))
            k[r] = enc(_unit_rows_f32(rng, (B, H, cfg.d_k)))
            v[r] = enc(rng.standard_normal((B, H, cfg.d_v), dtype=np.float32))
            alpha[r] = rng.uniform(cfg.alpha_lo, 1.0, size=(B, H))
            beta[r] = rng.uniform(0.0, 1.0, size=(B, H))

        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(fill, range(R)))
        parent = parents_for_step(cfg, _rng(cfg, 2, seed, t), t, 1 if t == 1 else B, B)
        out.append(StepInputs(q, k, v, alpha, beta, parent, cfg.qkv_dtype))
    return out


# ----------------------------------------------------------------------------------------------
# Shared post-prefill state
# ----------------------------------------------------------------------------------------------

def direct_sctx(cfg: Config, seed: int = 0) -> np.ndarray:
    """S_ctx drawn directly as N(0, std^2) float32, [R, H, d_v, d_k] (configurations without prefill)."""
    rng = _rng(cfg, 0, seed)
    return (rng.standard_normal((cfg.R, cfg.H, cfg.d_v, cfg.d_k), dtype=np.float32)
            * np.float32(cfg.sctx_std))


@dataclasses.dataclass
class PrefillInputs:
    """Inputs of the prompt prefill: k [R, N, H, d_k], v [R, N, H, d_v], alpha/beta [R, N, H], float32."""

    k: np.ndarray
    v: np.ndarray
    alpha: np.ndarray
    beta: np.ndarray


def prefill_inputs(cfg: Config, seed: int = 0, steps: Optional[int] = None, requests=None) -> PrefillInputs:
    """Random prompt of ``steps`` (default cfg.prefill_steps) GDN steps for every head of the given
    requests (default: all), arrays indexed by position in ``requests``."""
    n = cfg.prefill_steps if steps is None else steps
    reqs = list(range(cfg.R)) if requests is None else list(requests)
    H = cfg.H
    k = np.empty((len(reqs), n, H, cfg.d_k), np.float32)
    v = np.empty((len(reqs), n, H, cfg.d_v), np.float32)
    alpha = np.empty((len(reqs), n, H), np.float32)
    beta = np.empty((len(reqs), n, H), np.float32)

    def fill(i):
        rng = _rng(cfg, 0, seed, reqs[i])
        k[i] = _unit_rows_f32(rng, (n, H, cfg.d_k))
        v[i] = rng.standard_normal((n, H, cfg.d_v), dtype=np.float32)
        alpha[i] = rng.uniform(cfg.alpha_lo, 1.0, size=(n, H))
        beta[i] = rng.uniform(0.0, 1.0, size=(n, H))

    with ThreadPoolExecutor(_threads()) as ex:
        list(ex.map(fill, range(len(reqs))))
    return PrefillInputs(k, v, alpha, beta)


@dataclasses.dataclass
class SelectInputs:
    """Inputs of one beam-selection step: beam_scores [R, n_prev] and logp [R, n_prev, n_cand], float32."""

    beam_scores: np.ndarray
    logp: np.ndarray


def select_inputs(R: int, n_prev: int, n_cand: int, seed: int = 0, tag: int = 0, ties: bool = False) -> SelectInputs:
    """Synthetic candidate scores for the beam selection that precedes a decode step.

    Stream 3 of the seed sequence.  Per request: beam scores are minus the running sums of Exp(1) draws
    (best beam first, as the score-rank order of the parents); candidate log-probabilities are a
    log-softmax, in float64, of N(0, 2^2) logits, rounded once to float32.  With ``ties`` the logits are
    drawn from 8 integer levels and the beam scores from 4, so many candidate scores are exactly equal.
    """
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([_SEED_TAG, 3, tag, seed, R, n_prev, n_cand])))
    if ties:
        bs = -rng.integers(0, 4, size=(R, n_prev)).astype(np.float64)
        logits = rng.integers(0, 8, size=(R, n_prev, n_cand)).astype(np.float64)
    else:
        bs = -np.cumsum(rng.exponential(1.0, size=(R, n_prev)), axis=1)
        logits = 2.0 * rng.standard_normal((R, n_prev, n_cand))
    m = logits.max(axis=2, keepdims=True)
    lse = m + np.log(np.exp(logits - m).sum(axis=2, keepdims=True))
    return SelectInputs(bs.astype(np.float32), (logits - lse).astype(np.float32))
