"""Multi-layer beam-search decode on synthetic weights: the GDN beam-decode library in its surroundings.

A weight-free stand-in for an end-to-end generative-recommendation decode ("Scientific Impact Assessment:
OneLA", §1: hundreds of beams decoded for a few steps from one prompt-derived state per layer; beams are
pruned, reordered and fanned out between steps).  The trained model is not available, so every weight is
random; what is real is the data flow:

  * n_layers GDN layers, each with its own decode context (onela_create) and its own S_ctx from a prompt
    prefill (onela_prefill on synthetic prompt inputs: a stand-in, since a true multi-layer prefill would feed
    each layer the previous layer's per-token outputs);
  * per step and layer: q, k, v, alpha, beta projected from the hidden state by one random matrix (a plain
    library GEMM), q and k L2-normalised in float32, alpha = a_lo + (1 - a_lo) sigmoid(.), beta = sigmoid(.);
    onela_step; the head outputs projected back and added to the hidden state;
  * after the last layer, candidate log-probabilities from a random vocabulary matrix, and onela_beam_select
    picks the survivors, whose parents every layer consumes on the next step and whose tokens' embeddings are
    the next step's input.

Every step of the recurrence, the ancestry index and the beam selection run in libonela; the projections and
the log-softmax are torch operations on the GPU (library GEMMs and elementwise kernels).
"""

from __future__ import annotations

import dataclasses
from typing import List, Optional

from . import inputs as _inputs
from . import onela

__all__ = ["StackConfig", "GDNStack"]


@dataclasses.dataclass(frozen=True)
class StackConfig:
    R: int = 32           # requests
    B: int = 512          # beams
    L: int = 8            # decode steps
    layers: int = 4
    H: int = 16
    d_k: int = 128
    d_v: int = 128
    D: int = 2048         # hidden size
    n_cand: int = 256     # candidate tokens per beam and step
    prefill_tokens: int = 64
    alpha_lo: float = 0.9
    seed: int = 0


class GDNStack:
    """n_layers GDN layers with random weights on one GPU, decoding with beam search."""

    def __init__(self, cfg: StackConfig, device=None):
        import torch
        self.torch = torch
        self.cfg = c = cfg
        self.device = torch.device("cuda", 0) if device is None else torch.device(device)
        g = torch.Generator(device="cpu").manual_seed(0x0E1A + cfg.seed)
        bf = torch.bfloat16

        def rnd(*shape, scale):
            return (torch.randn(*shape, generator=g) * scale).to(self.device, bf)

        self.n_proj = c.H * (2 * c.d_k + c.d_v) + 2 * c.H
        self.w_in = [rnd(c.D, self.n_proj, scale=c.D ** -0.5) for _ in range(c.layers)]
        self.w_out = [rnd(c.H * c.d_v, c.D, scale=(c.H * c.d_v) ** -0.5) for _ in range(c.layers)]
        self.emb = rnd(c.n_cand, c.D, scale=1.0)
        self.w_vocab = rnd(c.D, c.n_cand, scale=c.D ** -0.5)
        self.x_prompt = rnd(c.R, 1, c.D, scale=1.0)
        self.ctx = [onela.OneLA(c.R, c.H, c.d_k, c.d_v, c.B, c.L, device=self.device) for _ in range(c.layers)]
        self.sctx = []
        for layer, ctx in enumerate(self.ctx):
            pcfg = _inputs.config(2, R=c.R, H=c.H, d_k=c.d_k, d_v=c.d_v, prefill_steps=c.prefill_tokens,
                                  alpha_lo=c.alpha_lo)
            pf = _inputs.prefill_inputs(pcfg, seed=100 + layer)
            t = lambda a: torch.from_numpy(a).to(self.device)  # noqa: E731
            out = torch.empty((c.R, c.H, c.d_v, c.d_k), dtype=torch.float32, device=self.device)
            ctx.prefill(t(pf.k), t(pf.v), t(pf.alpha), t(pf.beta), sctx_out=out)
            self.sctx.append(out)
        need = max(onela.onela_beam_select_scratch(c.R, n_prev, c.n_cand, self._n_beams(n_prev))
                   for n_prev in (1, c.B))
        self.scratch = torch.empty(max(need, 1), dtype=torch.uint8, device=self.device)
        self.record: Optional[List[dict]] = None

    def _layer(self, layer: int, x, parent):
        """One GDN layer on hidden state x [R, n, D] (bf16); returns the new hidden state."""
        torch, c = self.torch, self.cfg
        R, n = x.shape[0], x.shape[1]
        p = (x.reshape(R * n, c.D) @ self.w_in[layer]).float().reshape(R, n, self.n_proj)
        o1 = c.H * c.d_k
        q = p[..., :o1].reshape(R, n, c.H, c.d_k)
        k = p[..., o1:2 * o1].reshape(R, n, c.H, c.d_k)
        v = p[..., 2 * o1:2 * o1 + c.H * c.d_v].reshape(R, n, c.H, c.d_v)
        ab = p[..., 2 * o1 + c.H * c.d_v:].reshape(R, n, c.H, 2)
        q = (q / q.norm(dim=-1, keepdim=True)).to(torch.bfloat16).contiguous()
        k = (k / k.norm(dim=-1, keepdim=True)).to(torch.bfloat16).contiguous()
        v = v.to(torch.bfloat16).contiguous()
        alpha = (c.alpha_lo + (1.0 - c.alpha_lo) * torch.sigmoid(ab[..., 0])).contiguous()
        beta = torch.sigmoid(ab[..., 1]).contiguous()
        o = self.ctx[layer].step(q, k, v, alpha, beta, parent)
        if self.record is not None:
            self.record[-1]["layers"].append(dict(q=q.cpu(), k=k.cpu(), v=v.cpu(), alpha=alpha.cpu(),
                                                  beta=beta.cpu(), o=o.cpu()))
        y = o.reshape(R * n, c.H * c.d_v).to(torch.bfloat16) @ self.w_out[layer]
        return (x.float() + y.float().reshape(R, n, c.D)).to(torch.bfloat16)

    def _n_beams(self, n_prev: int) -> int:
        """Beams kept after a step from n_prev beams: B, or every candidate while there are fewer."""
        return min(self.cfg.B, n_prev * self.cfg.n_cand)

    def _logp(self, x):
        torch, c = self.torch, self.cfg
        R, n = x.shape[0], x.shape[1]
        logits = (x.reshape(R * n, c.D) @ self.w_vocab).float().reshape(R, n, c.n_cand)
        return torch.log_softmax(logits, dim=-1).contiguous()

    def decode(self, record: bool = False):
        """One full beam-search decode of L steps; returns (tokens [L][R, B], final beam scores [R, B])."""
        torch, c = self.torch, self.cfg
        self.record = [] if record else None
        for ctx in self.ctx:
            ctx.reset()
        scores = torch.zeros((c.R, 1), dtype=torch.float32, device=self.device)
        logp = self._logp(self.x_prompt)
        tokens_out = []
        parent, token, scores_next = onela.beam_select(scores, logp, self._n_beams(1), scratch=self.scratch)
        for t in range(1, c.L + 1):
            if self.record is not None:
                self.record.append(dict(beam_scores=scores.cpu(), logp=logp.cpu(), parent=parent.cpu(),
                                        token=token.cpu(), scores=scores_next.cpu(), layers=[]))
            scores = scores_next
            tokens_out.append(token)
            x = self.emb[token.long()]  # [R, B, D]
            for layer in range(c.layers):
                x = self._layer(layer, x, parent)
            logp = self._logp(x)
            if t < c.L:
                parent, token, scores_next = onela.beam_select(scores, logp, self._n_beams(scores.shape[1]),
                                                               scratch=self.scratch)
        for ctx in self.ctx:
            if ctx.status() != onela.ONELA_OK:
                raise RuntimeError("a parent index was out of range")
        return tokens_out, scores

    def close(self):
        for ctx in self.ctx:
            ctx.close()
