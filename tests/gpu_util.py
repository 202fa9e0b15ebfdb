"""Helpers of the GPU parity tests: run the decode through libonela, run the CPU oracle on the same seeded
inputs, and compare them element by element.

Bars (from the arithmetic of the path): chain tables, record placement, record keys and record alphas
are compared bit for bit; outputs o and record vectors u (float32 on the GPU, float64 in the oracle)
within max-abs 1e-3.
"""

import sys

import numpy as np
import torch

import oracle
from linear_attention_beam_amd import inputs, onela

TOL = 1e-3


def log(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def device():
    return torch.device("cuda", 0)


def to_torch(a: np.ndarray) -> torch.Tensor:
    if a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a))


def upload_step(s: inputs.StepInputs, dev=None):
    dev = device() if dev is None else dev
    return dict(q=to_torch(s.q).to(dev), k=to_torch(s.k).to(dev), v=to_torch(s.v).to(dev),
                alpha=to_torch(s.alpha).to(dev), beta=to_torch(s.beta).to(dev),
                parent=to_torch(s.parent.astype(np.int32)).to(dev))


def _f32(s: inputs.StepInputs, name, r, h):
    a = getattr(s, name)[r, :, h]
    return inputs.bf16_bits_to_f32(a) if s.dtype == "bf16" else a


def head_steps(steps, r, h):
    """Oracle inputs of one (request, head): per-step dicts shaped [1, B, 1, ...]."""
    out = []
    for s in steps:
        out.append(dict(q=_f32(s, "q", r, h)[None, :, None], k=_f32(s, "k", r, h)[None, :, None],
                        v=_f32(s, "v", r, h)[None, :, None], alpha=s.alpha[r, :, h][None, :, None],
                        beta=s.beta[r, :, h][None, :, None], parent=s.parent[r][None]))
    return out


def oracle_head(sctx_rh, steps, r, h, max_beams, max_steps):
    """Oracle replay of one head: (result dict, chain tables of request r)."""
    res = oracle.decode_replay(np.asarray(sctx_rh, np.float64)[None, None], head_steps(steps, r, h), max_beams,
                               max_steps)
    return res["heads"][(0, 0)], res["chains"][0]


def oracle_prefill_head(pf: inputs.PrefillInputs, r_idx, h):
    """Oracle prefill of one head; r_idx indexes the requests drawn in ``pf``."""
    sl = slice(r_idx, r_idx + 1)
    return oracle.prefill(pf.k[sl, :, h:h + 1], pf.v[sl, :, h:h + 1], pf.alpha[sl, :, h:h + 1],
                          pf.beta[sl, :, h:h + 1])[0, 0]


class GpuRun:
    """One decode through libonela.  ``outs[t]`` stays on the device."""

    def __init__(self, cfg: inputs.Config, steps, sctx=None, prefill=None, mode="replay", force_generic=False,
                 tile_beams=0, max_beams=None, max_steps=None, sctx_out=False, materialize=False):
        dev = device()
        self.cfg = cfg
        self.max_beams = cfg.B if max_beams is None else max_beams
        self.max_steps = len(steps) if max_steps is None else max_steps
        self.ctx = onela.OneLA(cfg.R, cfg.H, cfg.d_k, cfg.d_v, self.max_beams, self.max_steps,
                               qkv_dtype=cfg.qkv_dtype, mode=mode, force_generic=force_generic,
                               tile_beams=tile_beams, device=dev, materialize=materialize)
        self.sctx_gpu = None
        if sctx is not None:
            self.ctx.set_context(torch.from_numpy(np.asarray(sctx, np.float32)).to(dev))
        else:
            t = lambda a: torch.from_numpy(a).to(dev)  # noqa: E731
            out = (torch.empty((cfg.R, cfg.H, cfg.d_v, cfg.d_k), dtype=torch.float32, device=dev)
                   if sctx_out else None)
            self.ctx.prefill(t(prefill.k), t(prefill.v), t(prefill.alpha), t(prefill.beta), sctx_out=out)
            self.sctx_gpu = out
        self.outs = []
        for i, s in enumerate(steps, start=1):
            self.outs.append(self.ctx.step(**upload_step(s, dev)))
        torch.cuda.synchronize()
        self.status = self.ctx.status()
        self.view = self.ctx.view()

    def head_o(self, t0, r, h, n=None):
        o = self.outs[t0][r, :, h]
        return (o if n is None else o[:n]).double().cpu().numpy()


def compare_head(run: GpuRun, steps, ref, chains, r, h, check_records=True, tol=TOL):
    """Compare one (request, head) against the oracle; returns the max errors, raises on a mismatch."""
    err_o, err_u = 0.0, 0.0
    B_max = run.max_beams
    v = run.view
    for t0, s in enumerate(steps):
        n = s.parent.shape[1]
        got = run.head_o(t0, r, h)
        assert np.all(np.isfinite(got)), (r, h, t0)
        e = float(np.max(np.abs(got - ref["o"][t0]))) if n else 0.0
        eu = 0.0
        if check_records and v["rec_u"] is not None:
            slots = t0 * B_max + np.arange(n)
            sl = torch.from_numpy(slots).to(v["rec_u"].device)
            gu = v["rec_u"][r, h].index_select(0, sl).double().cpu().numpy()
            eu = float(np.max(np.abs(gu - ref["U"][slots])))
            gk = v["rec_k"][r, h].index_select(0, sl)
            if s.dtype == "bf16":
                assert np.array_equal(gk.view(torch.int16).cpu().numpy().view(np.uint16), s.k[r, :, h]), \
                    f"record keys r={r} h={h} t={t0 + 1}"
            else:
                assert np.array_equal(gk.cpu().numpy(), s.k[r, :, h]), f"record keys r={r} h={h} t={t0 + 1}"
            ga = v["rec_alpha"][r, h].index_select(0, sl).cpu().numpy()
            assert np.array_equal(ga, s.alpha[r, :, h]), f"record alphas r={r} h={h} t={t0 + 1}"
        assert e <= tol and eu <= tol, f"mismatch r={r} h={h} t={t0 + 1}: max|o err|={e:.3g} max|u err|={eu:.3g}"
        assert np.array_equal(v["chains"][t0, r].cpu().numpy(), chains[t0]), f"chain table r={r} t={t0 + 1}"
        err_o, err_u = max(err_o, e), max(err_u, eu)
    return err_o, err_u


def all_chains(steps, max_beams, max_steps, R):
    return [oracle.ancestry_tables([s.parent[r] for s in steps], max_beams, max_steps) for r in range(R)]
