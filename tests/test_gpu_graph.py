"""A whole decode captured as one HIP graph (torch.cuda.CUDAGraph) and replayed: a serving loop with static shapes
can capture the steps once.  onela_reset enqueues nothing and no step clears memory with a memset, so a replay is
a complete decode from the context.  Every replay, with eager decodes and syncs between the replays, must equal
the eager decode bit for bit, and the eager decode must match the oracle."""

import numpy as np
import pytest
import torch

from linear_attention_beam_amd import inputs, onela
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("kind", ["fused", "fused_dv256", "fp32_kernel"])
def test_captured_decode_replays_bit_for_bit(kind):
    if kind == "fp32_kernel":
        cfg = inputs.config(0, R=2, H=2, B=40, L=4)  # float32 inputs, d = 16: the fp32 kernel
    elif kind == "fused_dv256":
        cfg = inputs.config(2, R=2, H=2, d_v=256, B=72, L=4, prefill_steps=0, sctx_std=0.1)
    else:
        cfg = inputs.config(2, R=2, H=3, B=96, L=5, prefill_steps=0, sctx_std=0.1)
    gu.log(f"graph {kind}: R={cfg.R} H={cfg.H} d_k={cfg.d_k} d_v={cfg.d_v} B={cfg.B} L={cfg.L} {cfg.qkv_dtype}")
    dev = gu.device()
    steps = inputs.decode_inputs(cfg, seed=7)
    ds = [gu.upload_step(s, dev) for s in steps]
    outs = [torch.empty((cfg.R, cfg.B, cfg.H, cfg.d_v), dtype=torch.float32, device=dev) for _ in range(cfg.L)]
    sctx = inputs.direct_sctx(cfg, seed=7)
    ctx = onela.OneLA(cfg.R, cfg.H, cfg.d_k, cfg.d_v, cfg.B, cfg.L, qkv_dtype=cfg.qkv_dtype, device=dev)
    ctx.set_context(torch.from_numpy(sctx).to(dev))

    def decode():
        ctx.reset()
        for t in range(cfg.L):
            ctx.step(**ds[t], out=outs[t])

    side = torch.cuda.Stream(device=dev)
    side.wait_stream(torch.cuda.current_stream(dev))
    with torch.cuda.stream(side):
        decode()
    torch.cuda.current_stream(dev).wait_stream(side)
    torch.cuda.synchronize()
    assert ctx.status() == onela.ONELA_OK
    ref = [o.clone() for o in outs]
    # the eager decode against the oracle (request 0, head 0), so that the bits compared below are the right ones
    oref, _ = gu.oracle_head(sctx[0, 0], steps, 0, 0, cfg.B, cfg.L)
    for t in range(cfg.L):
        got = ref[t][0, :, 0, :].cpu().numpy()
        assert np.max(np.abs(got - oref["o"][t])) < gu.TOL, t

    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        decode()
    torch.cuda.synchronize()
    for rep in range(3):
        for o in outs:
            o.fill_(float("nan"))
        graph.replay()
        torch.cuda.synchronize()
        for t in range(cfg.L):
            assert torch.equal(outs[t], ref[t]), (rep, t)
        decode()  # eager work between the replays
        torch.cuda.synchronize()
        for t in range(cfg.L):
            assert torch.equal(outs[t], ref[t]), (rep, t)
    del graph
    ctx.close()
