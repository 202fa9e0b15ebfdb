"""GPU edge cases against the oracle: ragged and varying beam counts, every fused tile size and d_v,
request x head counts that are not a multiple of the 8 XCDs, 64-step chains, determinism, a parent out of
range, host-side argument and state errors, reset and reuse."""

import ctypes

import numpy as np
import pytest
import torch

import oracle
from linear_attention_beam_amd import inputs, onela
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu


def ragged_steps(steps, beams):
    """Keep beams[t] beams at step t; parents of kept beams are folded into the previous step's range."""
    out = []
    b_prev = 1
    for s, n in zip(steps, beams):
        par = (s.parent[:, :n] % b_prev).astype(np.int32)
        out.append(inputs.StepInputs(np.ascontiguousarray(s.q[:, :n]), np.ascontiguousarray(s.k[:, :n]),
                                     np.ascontiguousarray(s.v[:, :n]), np.ascontiguousarray(s.alpha[:, :n]),
                                     np.ascontiguousarray(s.beta[:, :n]), par, s.dtype))
        b_prev = n
    return out


def short_prefill_sctx(cfg, tokens=48):
    pf = inputs.prefill_inputs(cfg, steps=tokens)
    return oracle.prefill(pf.k, pf.v, pf.alpha, pf.beta)


def check_all_heads(run, cfg, steps, sctx, max_beams, max_steps, check_records=True):
    chains = gu.all_chains(steps, max_beams, max_steps, cfg.R)
    worst = 0.0
    for r in range(cfg.R):
        for h in range(cfg.H):
            ref, _ = gu.oracle_head(sctx[r, h], steps, r, h, max_beams, max_steps)
            e_o, _ = gu.compare_head(run, steps, ref, chains[r], r, h, check_records=check_records)
            worst = max(worst, e_o)
    return worst


RAGGED = [1, 37, 100, 64, 99]


@pytest.mark.parametrize("d_v,tile,generic", [
    (128, 16, False), (128, 32, False), (256, 16, False), (256, 32, False), (64, 0, False), (256, 0, False),
    (32, 16, False), (96, 32, False), (128, 0, True),
])
def test_ragged_beams(d_v, tile, generic):
    cfg = inputs.config(2, R=3, H=5, d_v=d_v, B=100, L=len(RAGGED))
    gu.log(f"ragged beams {RAGGED} d_v={d_v} tile={tile} generic={generic} (R*H=15)")
    steps = ragged_steps(inputs.decode_inputs(cfg), RAGGED)
    sctx = short_prefill_sctx(cfg)
    try:
        run = gu.GpuRun(cfg, steps, sctx=sctx, tile_beams=tile, force_generic=generic, max_beams=128, max_steps=6)
    except onela.OnelaError as e:
        if e.status == onela.ONELA_ERR_UNSUPPORTED:
            pytest.skip(f"device LDS limit: {e}")
        raise
    assert run.view["fused"] == (not generic)
    assert run.status == onela.ONELA_OK
    gu.log(f"  max|o err|={check_all_heads(run, cfg, steps, sctx, 128, 6):.3g}")


@pytest.mark.parametrize("d_k,d_v,tile", [
    (64, 128, 16), (64, 128, 32), (64, 256, 32), (64, 64, 0), (64, 96, 16), (64, 32, 32),
    (256, 128, 0), (256, 256, 16), (256, 64, 32), (256, 32, 0), (256, 160, 32),
])
def test_fused_head_sizes(d_k, d_v, tile):
    """d_k = 64 and 256 on the fused kernel (rows of 8 or 32 pieces, 2 or 8 matrix-core k-steps; one workgroup
    per compute unit at 256): ragged beam counts, every head and record against the oracle."""
    cfg = inputs.config(2, R=3, H=5, d_k=d_k, d_v=d_v, B=100, L=len(RAGGED))
    gu.log(f"fused d_k={d_k} ragged beams {RAGGED} d_v={d_v} tile={tile}")
    steps = ragged_steps(inputs.decode_inputs(cfg, seed=7), RAGGED)
    sctx = short_prefill_sctx(cfg)
    run = gu.GpuRun(cfg, steps, sctx=sctx, tile_beams=tile, max_beams=128, max_steps=6)
    assert run.view["fused"] and run.status == onela.ONELA_OK
    gu.log(f"  max|o err|={check_all_heads(run, cfg, steps, sctx, 128, 6):.3g}")


@pytest.mark.parametrize("d_k,tile", [(64, 16), (64, 32), (256, 16), (256, 32)])
def test_fused_head_sizes_long_chains(d_k, tile):
    """d_k = 64 and 256, 40 steps of 32 beams: late tiles have more distinct records than LDS holds and take
    the memory path (d_k / 8 lanes per beam for the key dot products)."""
    cfg = inputs.config(1, R=1, H=3, d_k=d_k, d_v=64, B=32, L=40)
    gu.log(f"fused d_k={d_k}, 40 steps, tile={tile}")
    steps = inputs.decode_inputs(cfg)
    sctx = short_prefill_sctx(cfg)
    run = gu.GpuRun(cfg, steps, sctx=sctx, tile_beams=tile)
    assert run.view["fused"] and run.status == onela.ONELA_OK
    gu.log(f"  max|o err|={check_all_heads(run, cfg, steps, sctx, cfg.B, cfg.L):.3g}")


@pytest.mark.parametrize("d_v,tile", [(128, 16), (96, 32), (224, 16), (32, 0)])
def test_odd_record_capacity(d_v, tile):
    """max_beams = 37: the slots of a (request, head) are not a multiple of 16, so the fused kernel's last
    16-slot tile of u records is partial (the arena is padded); every head and record checked."""
    cfg = inputs.config(2, R=2, H=3, d_v=d_v, B=37, L=3)
    gu.log(f"odd record capacity: B=37 L=3 d_v={d_v} tile={tile}")
    steps = inputs.decode_inputs(cfg)
    sctx = short_prefill_sctx(cfg)
    run = gu.GpuRun(cfg, steps, sctx=sctx, tile_beams=tile)
    assert run.view["fused"] and run.status == onela.ONELA_OK
    gu.log(f"  max|o err|={check_all_heads(run, cfg, steps, sctx, cfg.B, cfg.L):.3g}")


def test_tiles_and_xcd_mapping_agree():
    """R*H = 16 (a multiple of 8, XCD-grouped mapping) and every tile size give the same outputs."""
    cfg = inputs.config(2, R=2, H=8, B=96, L=3)
    steps = inputs.decode_inputs(cfg)
    sctx = short_prefill_sctx(cfg)
    runs = [gu.GpuRun(cfg, steps, sctx=sctx, tile_beams=t) for t in (16, 32)]
    for run in runs[1:]:
        for t in range(cfg.L):
            assert (run.outs[t] - runs[0].outs[t]).abs().max().item() <= 1e-6
    gu.log(f"  max|o err|={check_all_heads(runs[-1], cfg, steps, sctx, cfg.B, cfg.L):.3g}")


@pytest.mark.parametrize("generic", [False, True])
def test_64_step_chains(generic):
    cfg = inputs.config(1, R=1, H=2, d_v=32, B=16, L=64)
    gu.log(f"64 steps, generic={generic}")
    steps = inputs.decode_inputs(cfg)
    sctx = short_prefill_sctx(cfg)
    run = gu.GpuRun(cfg, steps, sctx=sctx, force_generic=generic)
    gu.log(f"  max|o err|={check_all_heads(run, cfg, steps, sctx, cfg.B, cfg.L):.3g}")


@pytest.mark.parametrize("d_k,d_v", [(256, 256), (64, 64)])
def test_64_step_chains_head_sizes(d_k, d_v):
    """64-step chains at the largest and smallest fused head sizes (d_k = d_v = 256 needs about 124 KB of LDS per
    32-beam tile at L = 64)."""
    cfg = inputs.config(1, R=1, H=2, d_k=d_k, d_v=d_v, B=16, L=64)
    gu.log(f"64 steps, d_k={d_k} d_v={d_v}")
    steps = inputs.decode_inputs(cfg)
    sctx = short_prefill_sctx(cfg)
    run = gu.GpuRun(cfg, steps, sctx=sctx)
    assert run.view["fused"] and run.status == onela.ONELA_OK
    gu.log(f"  max|o err|={check_all_heads(run, cfg, steps, sctx, cfg.B, cfg.L):.3g}")


def test_deterministic():
    cfg = inputs.config(2, R=2, H=4, B=256, L=4)
    steps = inputs.decode_inputs(cfg)
    sctx = short_prefill_sctx(cfg)
    a = gu.GpuRun(cfg, steps, sctx=sctx)
    b = gu.GpuRun(cfg, steps, sctx=sctx)
    for t in range(cfg.L):
        assert torch.equal(a.outs[t], b.outs[t])
    assert torch.equal(a.view["rec_u"], b.view["rec_u"])


@pytest.mark.parametrize("ci", [3, 4])
def test_deterministic_full_size(ci):
    """Two decodes of a full-size workload agree bit for bit: the processing order places siblings the same way
    in every run, so the tiles, and which of them read their records from memory instead of LDS, repeat."""
    cfg = inputs.config(ci)
    gu.log(f"determinism at full size: {cfg.name}")
    steps = inputs.decode_inputs(cfg)
    sctx = inputs.direct_sctx(cfg)
    a = gu.GpuRun(cfg, steps, sctx=sctx)
    outs_a = [o.clone() for o in a.outs]
    u_a = a.view["rec_u"].clone()
    a.ctx.close()
    del a
    b = gu.GpuRun(cfg, steps, sctx=sctx)
    for t in range(cfg.L):
        assert torch.equal(outs_a[t].view(torch.int32), b.outs[t].view(torch.int32)), f"step {t + 1}"
    assert torch.equal(u_a.view(torch.int32), b.view["rec_u"].view(torch.int32))


@pytest.mark.parametrize("mode", ["replay", "fullstate"])
def test_parent_out_of_range_is_flagged(mode):
    cfg = inputs.config(2, R=2, H=2, B=32, L=3)
    steps = inputs.decode_inputs(cfg)
    bad = [inputs.StepInputs(s.q, s.k, s.v, s.alpha, s.beta, s.parent.copy(), s.dtype) for s in steps]
    bad[1].parent[1, 5] = cfg.B          # out of range in request 1 only
    sctx = short_prefill_sctx(cfg)
    run = gu.GpuRun(cfg, bad, sctx=sctx, mode=mode)
    assert run.status == onela.ONELA_ERR_BAD_PARENT
    chains = gu.all_chains(steps[:1], cfg.B, cfg.L, cfg.R)
    for h in range(cfg.H):               # request 0 is untouched by request 1's bad index
        ref, _ = gu.oracle_head(sctx[0, h], bad, 0, h, cfg.B, cfg.L)
        for t in range(cfg.L):
            assert np.max(np.abs(run.head_o(t, 0, h) - ref["o"][t])) <= gu.TOL
    assert np.array_equal(run.view["chains"][0, 0].cpu().numpy(), chains[0][0])
    run.ctx.reset()
    assert run.ctx.status() == onela.ONELA_OK


def test_host_errors_leave_state_unchanged():
    cfg = inputs.config(2, R=1, H=2, B=8, L=2)
    steps = inputs.decode_inputs(cfg)
    dev = gu.device()
    ctx = onela.OneLA(cfg.R, cfg.H, cfg.d_k, cfg.d_v, cfg.B, 2, device=dev)
    d = gu.upload_step(steps[0], dev)
    with pytest.raises(onela.OnelaError) as e:       # no context yet
        ctx.step(**d)
    assert e.value.status == onela.ONELA_ERR_STATE
    ctx.set_context(torch.zeros((1, 2, 128, 128), device=dev))
    h, s = ctx.handle, torch.cuda.current_stream().cuda_stream
    ptrs = [d[k].data_ptr() for k in ("q", "k", "v", "alpha", "beta", "parent")]
    o = torch.empty((1, 8, 2, 128), device=dev)
    for n_beams in (0, 9):
        st = onela.lib().onela_step(h, n_beams, *ptrs, o.data_ptr(), s)
        assert st == onela.ONELA_ERR_INVALID_ARG
    st = onela.lib().onela_step(h, 8, *ptrs[:2], None, *ptrs[3:], o.data_ptr(), s)
    assert st == onela.ONELA_ERR_INVALID_ARG
    assert onela.onela_get_view(h).t == 0
    ctx.step(**d)
    ctx.step(**gu.upload_step(steps[1], dev))
    with pytest.raises(onela.OnelaError) as e:       # both steps of the context are used
        ctx.step(**gu.upload_step(steps[1], dev))
    assert e.value.status == onela.ONELA_ERR_CAPACITY
    assert onela.onela_get_view(h).t == 2
    with pytest.raises(ValueError):                  # wrong dtype is caught by the binding
        ctx.step(d["q"].float(), d["k"], d["v"], d["alpha"], d["beta"], d["parent"])
    bad_ws = torch.empty(1024, dtype=torch.uint8, device=dev)
    with pytest.raises(onela.OnelaError) as e:
        onela.onela_create(ctx.cfg, bad_ws.data_ptr(), 1024)
    assert e.value.status == onela.ONELA_ERR_CAPACITY
    ctx.close()


def test_reset_and_reuse():
    """A second decode on the same context after reset matches the oracle (records are overwritten)."""
    cfg = inputs.config(2, R=2, H=3, B=48, L=3)
    sctx = short_prefill_sctx(cfg)
    first = inputs.decode_inputs(cfg, seed=1)
    second = inputs.decode_inputs(cfg, seed=2)
    dev = gu.device()
    ctx = onela.OneLA(cfg.R, cfg.H, cfg.d_k, cfg.d_v, cfg.B, cfg.L, device=dev)
    ctx.set_context(torch.from_numpy(sctx.astype(np.float32)).to(dev))
    for s in first:
        ctx.step(**gu.upload_step(s, dev))
    ctx.reset()
    outs = [ctx.step(**gu.upload_step(s, dev)) for s in second]
    torch.cuda.synchronize()
    for r in range(cfg.R):
        for h in range(cfg.H):
            ref, _ = gu.oracle_head(sctx[r, h], second, r, h, cfg.B, cfg.L)
            for t in range(cfg.L):
                got = outs[t][r, :, h].double().cpu().numpy()
                assert np.max(np.abs(got - ref["o"][t])) <= gu.TOL


def test_context_transpose_is_exact():
    cfg = inputs.config(2, R=2, H=3, B=8, L=1)
    sctx = np.random.default_rng(5).standard_normal((2, 3, 128, 128)).astype(np.float32)
    dev = gu.device()
    ctx = onela.OneLA(cfg.R, cfg.H, 128, 128, 8, 1, device=dev)
    ctx.set_context(torch.from_numpy(sctx).to(dev))
    torch.cuda.synchronize()
    assert np.array_equal(ctx.view()["sctx_t"].cpu().numpy(), np.swapaxes(sctx, -1, -2))


@pytest.mark.parametrize("d_k,d_v,dtype", [(130, 72, "f32"), (64, 256, "bf16"), (256, 256, "bf16"), (16, 16, "f32"),
                                            (128, 128, "bf16")])
def test_materializing_replay(d_k, d_v, dtype):
    """The comparison path that rebuilds each beam's dense parent state: every head against the oracle, including
    uneven column groups (d_k = 130 splits 44/43/43) and the 1024-thread case (d_k = d_v = 256)."""
    cfg = inputs.config(2, R=2, H=2, d_k=d_k, d_v=d_v, B=40, L=4, qkv_dtype=dtype)
    gu.log(f"materializing replay d_k={d_k} d_v={d_v} {dtype}")
    steps = inputs.decode_inputs(cfg)
    sctx = short_prefill_sctx(cfg)
    run = gu.GpuRun(cfg, steps, sctx=sctx, materialize=True)
    assert not run.view["fused"]
    assert run.status == onela.ONELA_OK
    gu.log(f"  max|o err|={check_all_heads(run, cfg, steps, sctx, cfg.B, cfg.L):.3g}")


@pytest.mark.parametrize("generic", [False, True])
def test_single_beam_is_sequential_gdn(generic):
    """One beam for 24 steps is plain sequential GDN from S_ctx: compared with the oracle's sequential
    recurrence (the dense update, no records or chains)."""
    cfg = inputs.config(1, R=2, H=3, B=1, L=24)
    gu.log(f"single beam, 24 steps, generic={generic}")
    steps = inputs.decode_inputs(cfg)
    for s in steps:
        s.parent[:] = 0
    sctx = short_prefill_sctx(cfg)
    run = gu.GpuRun(cfg, steps, sctx=sctx, force_generic=generic)
    worst = 0.0
    for r in range(cfg.R):
        for h in range(cfg.H):
            f = lambda name: np.stack([gu._f32(s, name, r, h)[0] for s in steps])  # noqa: E731
            ref = oracle.sequential_outputs(sctx[r, h], f("q"), f("k"), f("v"),
                                            np.array([s.alpha[r, 0, h] for s in steps]),
                                            np.array([s.beta[r, 0, h] for s in steps]))
            got = np.stack([run.head_o(t, r, h)[0] for t in range(cfg.L)])
            worst = max(worst, float(np.max(np.abs(got - ref))))
    gu.log(f"  max|o err|={worst:.3g}")
    assert worst <= gu.TOL


def test_many_beams():
    """8192 beams per request (128 tiles of 64 per (request, head)), Zipf(1.1) parents, every head."""
    cfg = inputs.config(2, R=1, H=2, B=8192, L=3)
    gu.log("8192 beams, R=1 H=2 L=3")
    steps = inputs.decode_inputs(cfg)
    sctx = short_prefill_sctx(cfg)
    run = gu.GpuRun(cfg, steps, sctx=sctx)
    assert run.view["fused"] and run.status == onela.ONELA_OK
    gu.log(f"  max|o err|={check_all_heads(run, cfg, steps, sctx, cfg.B, cfg.L):.3g}")
