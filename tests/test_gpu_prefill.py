"""GPU prefill (onela_prefill) against the float64 oracle prefill.  d_k = 128 with d_v in {16, 32, 64, 128, 256}
runs the chunked MFMA kernel (32-token chunks: token counts that leave a ragged last chunk, or fewer tokens than
one chunk); other head sizes run the row-parallel fp32 kernel (sizes that are not multiples of its 32-column
groups or 128-row workgroups).  Also: no tokens, and decays small enough (or zero) to exercise the folding of
the decay scale into the state (fp32 kernel) and the running decay products (MFMA kernel)."""

import numpy as np
import pytest
import torch

import oracle
from linear_attention_beam_amd import inputs, onela
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu

TOL = 2e-4


def run_prefill(cfg, pf: inputs.PrefillInputs, max_beams=8, max_steps=2, qkv_dtype="f32"):
    """The chunked kernel keeps its per-chunk T in the decode-state part of the workspace, whose size follows
    max_beams, max_steps and qkv_dtype: the default (8 beams, 2 steps, float32) holds a few chunks per
    (request, head), so longer prompts run in several segments."""
    dev = gu.device()
    ctx = onela.OneLA(cfg.R, cfg.H, cfg.d_k, cfg.d_v, max_beams, max_steps, qkv_dtype=qkv_dtype, device=dev)
    out = torch.full((cfg.R, cfg.H, cfg.d_v, cfg.d_k), float("nan"), dtype=torch.float32, device=dev)
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)  # noqa: E731
    ctx.prefill(t(pf.k), t(pf.v), t(pf.alpha), t(pf.beta), sctx_out=out)
    torch.cuda.synchronize()
    got = out.double().cpu().numpy()
    st = ctx.view()["sctx_t"].double().cpu().numpy()
    ctx.close()
    assert np.array_equal(st, np.swapaxes(got, -1, -2)), "installed S_ctx^T differs from the returned S_ctx"
    return got


def check(cfg, pf, **ws):
    got = run_prefill(cfg, pf, **ws)
    ref = oracle.prefill(pf.k, pf.v, pf.alpha, pf.beta)
    assert np.all(np.isfinite(got))
    err = float(np.max(np.abs(got - ref))) if got.size else 0.0
    gu.log(f"  max|S err|={err:.3g} (max|S|={float(np.max(np.abs(ref))) if ref.size else 0.0:.3g})")
    assert err < TOL
    return got, ref


@pytest.mark.parametrize("d_k,d_v,N", [
    (128, 128, 100), (16, 16, 17), (64, 32, 1), (96, 200, 33), (256, 256, 40), (40, 7, 16), (1, 1, 5),
    (200, 130, 31), (128, 256, 48), (128, 64, 70), (128, 32, 33), (128, 16, 65), (128, 128, 1), (128, 96, 40),
    (128, 256, 300),
])
def test_prefill_shapes(d_k, d_v, N):
    cfg = inputs.config(2, R=2, H=3, d_k=d_k, d_v=d_v, prefill_steps=N)
    gu.log(f"prefill d_k={d_k} d_v={d_v} N={N}")
    check(cfg, inputs.prefill_inputs(cfg, seed=5))


def test_prefill_no_tokens():
    cfg = inputs.config(2, R=2, H=3, prefill_steps=0)
    pf = inputs.prefill_inputs(cfg, steps=0)
    got = run_prefill(cfg, pf)
    assert np.all(got == 0.0)


@pytest.mark.parametrize("alpha_hi,zeros", [(0.3, False), (0.05, True), (1.0, True)])
def test_prefill_small_and_zero_decay(alpha_hi, zeros):
    """alpha ~ U(0, alpha_hi), optionally with exact zeros (a full reset of the state at that token)."""
    cfg = inputs.config(2, R=2, H=4, prefill_steps=70)
    pf = inputs.prefill_inputs(cfg, seed=6)
    rng = np.random.default_rng(7)
    pf.alpha = rng.uniform(0.0, alpha_hi, size=pf.alpha.shape).astype(np.float32)
    if zeros:
        pf.alpha[:, ::9] = 0.0
    gu.log(f"prefill with alpha ~ U(0, {alpha_hi}) zeros={zeros}")
    check(cfg, pf)


def test_prefill_long_every_head():
    """A 5120-token prompt on 4 heads: the decay scale is folded back many times."""
    cfg = inputs.config(3, R=1, H=4)
    gu.log(f"prefill {cfg.prefill_steps} tokens, R=1 H=4")
    check(cfg, inputs.prefill_inputs(cfg, seed=8))


@pytest.mark.parametrize("spread,alpha_lo", [(0.0, 1.0), (0.05, 1.0), (0.05, 0.99), (1.0, 1.0)])
def test_prefill_correlated_keys_no_decay(spread, alpha_lo):
    """Keys nearly parallel (k_i = unit(k_0 + spread * noise); spread 0: one key for every token), beta near 1,
    and no or little decay: the chunked kernel's (I + M) then has its largest off-diagonal entries, and the fp32
    kernel's state never shrinks.  Both must still follow the float64 recurrence."""
    for d_v in (128, 96):  # 128: chunked MFMA kernel; 96: row-parallel fp32 kernel
        cfg = inputs.config(2, R=1, H=2, d_v=d_v, prefill_steps=130)
        pf = inputs.prefill_inputs(cfg, seed=9)
        rng = np.random.default_rng(10)
        k0 = rng.standard_normal((1, 1, cfg.H, cfg.d_k))
        k = k0 + spread * rng.standard_normal(pf.k.shape)
        pf.k = (k / np.linalg.norm(k, axis=-1, keepdims=True)).astype(np.float32)
        pf.beta = rng.uniform(0.9, 1.0, size=pf.beta.shape).astype(np.float32)
        pf.alpha = rng.uniform(alpha_lo, 1.0, size=pf.alpha.shape).astype(np.float32)
        gu.log(f"prefill, correlated keys (spread {spread}), alpha ~ U({alpha_lo}, 1), d_v={d_v}")
        check(cfg, pf)


@pytest.mark.parametrize("max_beams,max_steps,qkv_dtype,what", [
    (512, 8, "bf16", "one segment"),
    (1, 1, "f32", "scratch below one chunk: row-parallel fp32 kernel"),
    (16, 1, "bf16", "segments of one or two chunks"),
])
def test_prefill_scratch_sizes(max_beams, max_steps, qkv_dtype, what):
    cfg = inputs.config(2, R=1, H=2, prefill_steps=200)
    gu.log(f"prefill 200 tokens, workspace for {max_beams} beams x {max_steps} steps ({qkv_dtype}): {what}")
    check(cfg, inputs.prefill_inputs(cfg, seed=11), max_beams=max_beams, max_steps=max_steps, qkv_dtype=qkv_dtype)


@pytest.mark.parametrize("mode,generic", [("fullstate", False), ("replay", True), ("replay", False)])
def test_prefill_then_decode(mode, generic):
    """The decode after a prefill, in every mode.  The prefill's scratch is the decode state of the workspace
    (per-beam states for FullState, records and chains otherwise), so the first steps must not see any of it:
    S matches the oracle prefill, and every head's o (and u, keys, alphas, chains) the oracle decode from it."""
    cfg = inputs.config(1, R=1, H=4, B=48, L=3, prefill_steps=150)
    pf = inputs.prefill_inputs(cfg, seed=12)
    steps = inputs.decode_inputs(cfg)
    gu.log(f"prefill {cfg.prefill_steps} tokens then {cfg.L} steps, mode={mode} generic={generic}")
    run = gu.GpuRun(cfg, steps, prefill=pf, mode=mode, force_generic=generic, sctx_out=True)
    assert run.status == onela.ONELA_OK
    sctx = run.sctx_gpu.double().cpu().numpy()
    assert float(np.max(np.abs(sctx - oracle.prefill(pf.k, pf.v, pf.alpha, pf.beta)))) < TOL
    chains = gu.all_chains(steps, cfg.B, cfg.L, cfg.R)
    for h in range(cfg.H):
        ref, _ = gu.oracle_head(sctx[0, h], steps, 0, h, cfg.B, cfg.L)
        e_o, e_u = gu.compare_head(run, steps, ref, chains[0], 0, h, check_records=mode == "replay")
        gu.log(f"  head {h}: max|o err|={e_o:.3g} max|u err|={e_u:.3g}")
    # a second prompt on the same handle: its scratch overwrites the first decode's state, then a new decode
    pf2 = inputs.prefill_inputs(cfg, seed=13)
    steps2 = inputs.decode_inputs(cfg, seed=14)
    dev = gu.device()
    t = lambda a: torch.from_numpy(a).to(dev)  # noqa: E731
    out = torch.empty((cfg.R, cfg.H, cfg.d_v, cfg.d_k), dtype=torch.float32, device=dev)
    run.ctx.prefill(t(pf2.k), t(pf2.v), t(pf2.alpha), t(pf2.beta), sctx_out=out)
    run.outs = [run.ctx.step(**gu.upload_step(s, dev)) for s in steps2]
    torch.cuda.synchronize()
    assert run.ctx.status() == onela.ONELA_OK
    run.view = run.ctx.view()
    sctx2 = out.double().cpu().numpy()
    assert float(np.max(np.abs(sctx2 - oracle.prefill(pf2.k, pf2.v, pf2.alpha, pf2.beta)))) < TOL
    chains2 = gu.all_chains(steps2, cfg.B, cfg.L, cfg.R)
    for h in range(cfg.H):
        ref, _ = gu.oracle_head(sctx2[0, h], steps2, 0, h, cfg.B, cfg.L)
        e_o, e_u = gu.compare_head(run, steps2, ref, chains2[0], 0, h, check_records=mode == "replay")
        gu.log(f"  second prompt, head {h}: max|o err|={e_o:.3g} max|u err|={e_u:.3g}")


@pytest.mark.parametrize("i", range(12))
def test_prefill_random_shapes(i):
    """A seeded sweep: requests, heads, head sizes (half on the chunked kernel, d_k = 128), prompt length and
    the workspace the scratch comes from (so one, several or no chunks per segment), against the oracle."""
    rng = np.random.default_rng([0x9F11, i])
    R, H = int(rng.integers(1, 4)), int(rng.integers(1, 5))
    if i % 2 == 0:
        d_k, d_v = 128, int(rng.choice([16, 32, 64, 128, 256]))
    else:
        d_k, d_v = int(rng.integers(1, 257)), int(rng.integers(1, 257))
    N = int(rng.integers(0, 400))
    max_beams, max_steps = int(rng.choice([1, 4, 16, 64])), int(rng.integers(1, 4))
    qkv = str(rng.choice(["f32", "bf16"]))
    cfg = inputs.config(2, R=R, H=H, d_k=d_k, d_v=d_v, prefill_steps=N)
    gu.log(f"prefill random {i}: R={R} H={H} d_k={d_k} d_v={d_v} N={N} workspace {max_beams} x {max_steps} {qkv}")
    check(cfg, inputs.prefill_inputs(cfg, seed=30 + i), max_beams=max_beams, max_steps=max_steps, qkv_dtype=qkv)
