"""The decode step on the GPU against closed forms and invariants, with no oracle in the loop: every kernel
(fused bf16 MFMA, fp32 FMA with bf16 or fp32 inputs, materializing replay, FullState) through the C ABI.

  beta = 0                     every record carries u = 0 and o_t = (product of the alphas along the beam's
                               history, this step's included) S_ctx q_t
  alpha = beta = 1, keys       the delta rule stores v under k: o_t = v_j when q_t is the key of step j on the
  orthonormal along a chain    beam's history, and o_t = S_ctx q_t for a direction no key used
  v = 0                        everything is linear in S_ctx, and doubling is exact in binary floating point:
                               o(2 S_ctx) equals 2 o(S_ctx) bit for bit
  relabelling                  permuting the new beams of a step (and remapping the next step's parents)
                               permutes that step's outputs and leaves the later ones unchanged, bit for bit
  duplicates                   two beams with the same parent and inputs get the same output, bit for bit
  alpha = 0                    the step forgets S_ctx and the whole history: o_t = beta (k_t . q_t) v_t
"""

import numpy as np
import pytest
import torch

from linear_attention_beam_amd import inputs, onela
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu

R, H, D, B, L = 2, 3, 128, 48, 4
VARIANTS = {  # name: (qkv dtype, OneLA keyword arguments)
    "fused": ("bf16", {}),
    "fp32_kernel_bf16": ("bf16", dict(force_generic=True)),
    "fp32_kernel_f32": ("f32", {}),
    "materialize": ("bf16", dict(materialize=True)),
    "fullstate": ("bf16", dict(mode="fullstate")),
}


def enc(x, dtype):
    x = np.ascontiguousarray(x, dtype=np.float32)
    return inputs.f32_to_bf16_bits(x) if dtype == "bf16" else x


def dec(x, dtype):
    return inputs.bf16_bits_to_f32(x) if dtype == "bf16" else x


def unit(rng, shape):
    x = rng.standard_normal(shape).astype(np.float32)
    return x / np.linalg.norm(x, axis=-1, keepdims=True)


def parents(rng, t):
    return np.zeros((R, B), np.int32) if t == 1 else rng.integers(0, B, (R, B)).astype(np.int32)


def make_steps(rng, dtype, beta=None, alpha=None):
    steps = []
    for t in range(1, L + 1):
        steps.append(inputs.StepInputs(
            q=enc(unit(rng, (R, B, H, D)), dtype), k=enc(unit(rng, (R, B, H, D)), dtype),
            v=enc(rng.standard_normal((R, B, H, D)), dtype),
            alpha=(rng.uniform(0.9, 1.0, (R, B, H)) if alpha is None else np.full((R, B, H), alpha)).astype(np.float32),
            beta=(rng.uniform(0.0, 1.0, (R, B, H)) if beta is None else np.full((R, B, H), beta)).astype(np.float32),
            parent=parents(rng, t), dtype=dtype))
    return steps


def run(variant, sctx, steps):
    """o of every step (float64 numpy [R, n, H, D]) and the decode state view."""
    dtype, kw = VARIANTS[variant]
    dev = gu.device()
    ctx = onela.OneLA(R, H, D, D, B, L, qkv_dtype=dtype, device=dev, **kw)
    ctx.set_context(torch.from_numpy(np.ascontiguousarray(sctx, np.float32)).to(dev))
    outs = [ctx.step(**gu.upload_step(s, dev)) for s in steps]
    torch.cuda.synchronize()
    assert ctx.status() == onela.ONELA_OK
    view = ctx.view()
    fused = view["fused"]
    res = [o.double().cpu().numpy() for o in outs]
    rec_u = None if view["rec_u"] is None else view["rec_u"].cpu().numpy()
    ctx.close()
    assert fused == (variant == "fused")
    return res, rec_u


def history(steps, r, t, b):
    """Beam indices along the history of beam b after step t: [b at step t, its parent at t-1, ...]."""
    out = [b]
    for j in range(t, 1, -1):
        b = int(steps[j - 1].parent[r, b])
        out.append(b)
    return out


@pytest.mark.parametrize("variant", list(VARIANTS))
def test_beta_zero(variant):
    gu.log(f"closed form beta = 0: {variant}")
    rng = np.random.default_rng(101)
    dtype = VARIANTS[variant][0]
    sctx = rng.standard_normal((R, H, D, D)).astype(np.float32)
    steps = make_steps(rng, dtype, beta=0.0)
    outs, rec_u = run(variant, sctx, steps)
    worst = 0.0
    for t in range(1, L + 1):
        q = dec(steps[t - 1].q, dtype).astype(np.float64)
        for r in range(R):
            for b in range(B):
                hist = history(steps, r, t, b)
                prod = np.ones(H)
                for j, bb in zip(range(t, 0, -1), hist):
                    prod *= steps[j - 1].alpha[r, bb].astype(np.float64)
                for h in range(H):
                    ex = prod[h] * (sctx[r, h].astype(np.float64) @ q[r, b, h])
                    worst = max(worst, float(np.max(np.abs(outs[t - 1][r, b, h] - ex))))
    gu.log(f"  max|o - closed form| = {worst:.3g}")
    assert worst < 1e-3
    if rec_u is not None:
        assert np.all(rec_u[:, :, : L * B] == 0.0)


@pytest.mark.parametrize("variant", list(VARIANTS))
def test_orthonormal_recall(variant):
    """Keys are basis vectors: step t writes under e_{c + t} (c differs per request and head); queries ask for
    the key of a step on the history, or for a basis direction no key used (answered by S_ctx alone)."""
    gu.log(f"closed form alpha = beta = 1, orthonormal keys: {variant}")
    rng = np.random.default_rng(202)
    dtype = VARIANTS[variant][0]
    sctx = rng.standard_normal((R, H, D, D)).astype(np.float32)
    base = rng.integers(0, D - 2 * L, (R, H))
    steps, asks = [], []
    for t in range(1, L + 1):
        k = np.zeros((R, B, H, D), np.float32)
        q = np.zeros((R, B, H, D), np.float32)
        ask = rng.integers(1, t + 2, (R, B, H))  # t + 1: the unused direction e_{c + L + 1}
        for r in range(R):
            for h in range(H):
                k[r, :, h, base[r, h] + t] = 1.0
                for b in range(B):
                    j = ask[r, b, h]
                    q[r, b, h, base[r, h] + (j if j <= t else L + 1)] = 1.0
        v = dec(enc(rng.standard_normal((R, B, H, D)), dtype), dtype)  # values exact in the input dtype
        steps.append(inputs.StepInputs(q=enc(q, dtype), k=enc(k, dtype), v=enc(v, dtype),
                                       alpha=np.ones((R, B, H), np.float32), beta=np.ones((R, B, H), np.float32),
                                       parent=parents(rng, t), dtype=dtype))
        asks.append(ask)
    outs, _ = run(variant, sctx, steps)
    worst = 0.0
    for t in range(1, L + 1):
        for r in range(R):
            for b in range(B):
                hist = history(steps, r, t, b)  # hist[t - j] is the beam at step j
                for h in range(H):
                    j = asks[t - 1][r, b, h]
                    if j <= t:
                        ex = dec(steps[j - 1].v, dtype)[r, hist[t - j], h].astype(np.float64)
                    else:
                        ex = sctx[r, h, :, base[r, h] + L + 1].astype(np.float64)
                    worst = max(worst, float(np.max(np.abs(outs[t - 1][r, b, h] - ex))))
    gu.log(f"  max|o - recalled value| = {worst:.3g}")
    assert worst < 1e-3


@pytest.mark.parametrize("variant", list(VARIANTS))
def test_linear_in_context_exactly(variant):
    gu.log(f"v = 0: o(2 S_ctx) == 2 o(S_ctx) bit for bit: {variant}")
    rng = np.random.default_rng(303)
    dtype = VARIANTS[variant][0]
    sctx = rng.standard_normal((R, H, D, D)).astype(np.float32)
    steps = make_steps(rng, dtype)
    for s in steps:
        s.v[:] = 0
    a, _ = run(variant, sctx, steps)
    b2, _ = run(variant, 2.0 * sctx, steps)
    for t in range(L):
        assert np.any(a[t] != 0.0)
        assert np.array_equal(b2[t], 2.0 * a[t]), t


@pytest.mark.parametrize("variant", list(VARIANTS))
def test_relabelling_and_duplicates(variant):
    gu.log(f"beam relabelling and duplicate beams, bit for bit: {variant}")
    rng = np.random.default_rng(404)
    dtype = VARIANTS[variant][0]
    sctx = rng.standard_normal((R, H, D, D)).astype(np.float32)
    steps = make_steps(rng, dtype)
    for s in steps[1:]:  # beam 7 duplicates beam 2 (same parent, same inputs)
        for name in ("q", "k", "v", "alpha", "beta"):
            getattr(s, name)[:, 7] = getattr(s, name)[:, 2]
        s.parent[:, 7] = s.parent[:, 2]
    perm = rng.permutation(B)  # step 2's beam b moves to position perm[b]
    inv = np.argsort(perm)
    p_steps = list(steps)
    s2 = steps[1]
    p_steps[1] = inputs.StepInputs(*(np.ascontiguousarray(getattr(s2, f)[:, inv])
                                     for f in ("q", "k", "v", "alpha", "beta", "parent")), dtype)
    s3 = steps[2]
    p_steps[2] = inputs.StepInputs(s3.q, s3.k, s3.v, s3.alpha, s3.beta, perm[s3.parent].astype(np.int32), dtype)
    a, _ = run(variant, sctx, steps)
    p, _ = run(variant, sctx, p_steps)
    for t in range(1, L):
        assert np.array_equal(a[t][:, 7], a[t][:, 2]), f"duplicate beams differ at step {t + 1}"
    assert np.array_equal(p[0], a[0])
    assert np.array_equal(p[1], a[1][:, inv]), "relabelled step"
    for t in range(2, L):
        assert np.array_equal(p[t], a[t]), f"step {t + 1} after the relabelled one"


@pytest.mark.parametrize("variant", list(VARIANTS))
def test_alpha_zero(variant):
    """alpha = 0 forgets everything before the step: S_t = beta v k^T, so o_t = beta (k . q) v for every beam,
    whatever S_ctx and the history hold (all decay products along the chains are 0)."""
    gu.log(f"closed form alpha = 0: {variant}")
    rng = np.random.default_rng(505)
    dtype = VARIANTS[variant][0]
    sctx = rng.standard_normal((R, H, D, D)).astype(np.float32)
    steps = make_steps(rng, dtype, alpha=0.0)
    outs, _ = run(variant, sctx, steps)
    worst = 0.0
    for t, s in enumerate(steps):
        q, k, v = (dec(x, dtype).astype(np.float64) for x in (s.q, s.k, s.v))
        ex = s.beta[..., None].astype(np.float64) * np.sum(k * q, axis=-1, keepdims=True) * v
        worst = max(worst, float(np.max(np.abs(outs[t] - ex))))
    gu.log(f"  max|o - closed form| = {worst:.3g}")
    assert worst < 1e-3
