#!/usr/bin/env python3
"""Benchmark of the large-beam Gated DeltaNet decode step on one MI355X.

One bench "step" is one whole decode of the workload: L onela_step calls (ancestry index update, shared
S_ctx contraction, key and query replay, record append, output: one fused kernel per call) over
R requests x B beams x H heads, after onela_reset.  Inputs (all L steps) and the context are resident in
HBM before timing starts.  value = beam-tokens per second = R * B * L / seconds per decode.

Prints one JSON line.  Extra objects:
  roofline      the fused step kernel: algorithmic HBM bytes per launch (compulsory traffic, counted from
                the run's own chain tables) / its average launch time from HIP events in the timed region
  cpu_baseline  the float64 CPU oracle (record-replay form) timed on whole requests of the same workload
  fullstate     the controlled FullState path (dense per-beam state) on the same inputs
  materialize   the materializing-replay path (each beam's dense parent state rebuilt every step) on the same
                inputs
  hbm_probe     copy and fill bandwidth of plain torch kernels on the same GPU (context for the fraction)
  beam_select   the beam selection that produces each step's parents (top B of B x 256 candidate scores per
                request), timed on its own with HIP events; not part of the decode step above
  prefill       onela_prefill of the workload's prompt (the context the decode starts from), against the dense
                bf16 MFMA peak for the chunked kernels (d_k = 128), else the fp32 vector-ALU peak
  stack         a whole beam-search decode through several GDN layers with random weights (projections as
                library GEMMs, one decode context per layer, the GPU beam selection between steps) at the
                workload's R, H, B, L and head sizes; context for the step's share of a model's decode
"""

from __future__ import annotations

import argparse
import dataclasses
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0        # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0    # MI355X dense bf16 MFMA
FP32_PEAK_TFLOPS = 157.3     # MI355X fp32 vector: 256 CUs x 64 lanes x 2 (FMA) x 2 (packed) x 2.4 GHz
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "fused_step_traffic.json")
FUSED_SRC = os.path.join(ROOT, "linear_attention_beam_amd", "csrc", "step_fused.hip")


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def kernel_source_hash() -> str:
    return hashlib.sha256(open(FUSED_SRC, "rb").read()).hexdigest()[:16]


def algorithmic_bytes(cfg, chains, parents):
    """Compulsory HBM bytes of each decode step's fused launch.

    chains: [L, R, B, L] int32 tables read back from the run; parents: per-step [R, B] int32.
    Per step: S_ctx (bf16 high + low halves), q/k/v, alpha/beta, parents, the chain rows read (distinct
    parents) and written, o (float32), the appended records, and the distinct ancestor records read.
    """
    R, H, dk, dv, B, L = cfg.R, cfg.H, cfg.d_k, cfg.d_v, cfg.B, cfg.L
    s_in = cfg.in_bytes
    rec = dk * s_in + 4 * dv + 4
    out = []
    for t in range(1, L + 1):
        nbytes = R * H * dv * dk * 4                      # S_ctx hi + lo
        nbytes += R * B * H * (2 * dk + dv) * s_in        # q, k, v
        nbytes += R * B * H * 8 + R * B * 4               # alpha, beta, parents
        nbytes += R * B * H * dv * 4                      # o
        nbytes += R * B * H * rec                         # records appended
        nbytes += R * B * L * 4                           # chain table written
        anc = 0
        if t > 1:
            prev = chains[t - 2]
            for r in range(R):
                ps = np.unique(parents[t - 1][r])
                rows = prev[r, ps, : t - 1]
                anc += np.unique(rows).size
                nbytes += ps.size * (t - 1) * 4           # chain rows read
        nbytes += anc * H * rec                           # distinct ancestor records read
        out.append(nbytes)
    return out


def hbm_probe(torch, dev, gib: float = 2.0):
    """Achievable HBM bandwidth with plain torch kernels on this GPU: copy (1 read + 1 write) and fill (write
    only), best of 5.  Context for the roofline fraction; not part of the timed decode."""
    n = int(gib * (1 << 30)) // 4
    x = torch.ones(n, dtype=torch.float32, device=dev)
    y = torch.empty_like(x)

    def best(fn, nbytes):
        fn()
        torch.cuda.synchronize()
        out = 0.0
        for _ in range(5):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            fn()
            b.record()
            torch.cuda.synchronize()
            out = max(out, nbytes / (a.elapsed_time(b) * 1e-3) / 1e9)
        return out

    res = {"copy_GBs": best(lambda: y.copy_(x), 8.0 * n), "fill_GBs": best(lambda: y.fill_(2.0), 4.0 * n)}
    del x, y
    return res


def select_bench(torch, dev, cfg, n_cand: int = 256, reps: int = 20, with_cpu: bool = True):
    """Beam selection at the workload's shape: R requests, B current beams x n_cand candidates -> B survivors."""
    from linear_attention_beam_amd import inputs, onela
    R, n_prev, n_beams = cfg.R, cfg.B, cfg.B
    si = inputs.select_inputs(R, n_prev, n_cand, seed=0)
    bs = torch.from_numpy(si.beam_scores).to(dev)
    lp = torch.from_numpy(si.logp).to(dev)
    need = onela.onela_beam_select_scratch(R, n_prev, n_cand, n_beams)
    scratch = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    for _ in range(3):
        onela.beam_select(bs, lp, n_beams, scratch=scratch)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        onela.beam_select(bs, lp, n_beams, scratch=scratch)
    b.record()
    torch.cuda.synchronize()
    us = a.elapsed_time(b) / reps * 1e3
    nbytes = R * n_prev * n_cand * 4 + R * n_prev * 4 + R * n_beams * 12
    out = {"shape": f"R={R} n_prev={n_prev} n_cand={n_cand} -> n_beams={n_beams}", "us_per_call": us,
           "candidates_per_s": R * n_prev * n_cand / (us * 1e-6), "algorithmic_bytes": nbytes,
           "achieved_GBs": nbytes / (us * 1e-6) / 1e9}
    if with_cpu:
        import oracle
        t0 = time.perf_counter()
        oracle.beam_select(si.beam_scores, si.logp, n_beams)
        out["cpu_oracle_ms"] = (time.perf_counter() - t0) * 1e3
    return out


def prefill_bench(torch, ctx, ctx_in, cfg, stream, reps: int = 5, with_cpu: bool = True):
    """onela_prefill of the workload's prompt (R x H heads x N tokens, float32 inputs resident in HBM), timed
    with HIP events on the stream it runs on.  The recurrence is 4 d_k d_v float32 FLOPs per token and head
    (two FMAs per state element), sequential over tokens.  For d_k = 128 and d_v in {16, 32, 64, 128, 256} the
    library runs it in chunked form on the matrix cores: per 32-token chunk and head, G = K K^T (lower 16 x 16
    blocks, 3 x 16 x 16 x 128, once per chunk), Y = K S^T (32 x d_v x 128), U = T X (32 x d_v x 32) and the
    state update (128 x d_v x 32), each as three bf16 products (high/low halves): that MFMA work against the
    bf16 peak is the roofline; the rate of the equivalent float32 recurrence is reported beside it."""
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ctx.prefill(*ctx_in)
    torch.cuda.synchronize()
    a.record(stream)
    for _ in range(reps):
        ctx.prefill(*ctx_in)
    b.record(stream)
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / reps
    heads, N = cfg.R * cfg.H, cfg.prefill_steps
    flops = 4.0 * cfg.d_k * cfg.d_v * N * heads
    nbytes = 4.0 * heads * N * (cfg.d_k + cfg.d_v + 2) + 4.0 * heads * cfg.d_k * cfg.d_v * 3
    chunked = cfg.d_k == 128 and cfg.d_v in (16, 32, 64, 128, 256)
    if chunked:
        chunks = -(-N // 32)
        per_chunk = 3 * 2.0 * (3 * 16 * 16 * 128 + 32 * cfg.d_v * 128 + 32 * cfg.d_v * 32 + 128 * cfg.d_v * 32)
        mfma_flops = per_chunk * chunks * heads
        roof = {"bound": "mfma", "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s", "dtype": "bf16 (high/low halves)",
                "achieved": mfma_flops / (ms * 1e-3) / 1e12,
                "frac": mfma_flops / (ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, "mfma_flops": mfma_flops}
    else:
        roof = {"bound": "alu", "peak": FP32_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": flops / (ms * 1e-3) / 1e12 / FP32_PEAK_TFLOPS}
    out = {"shape": f"R={cfg.R} H={cfg.H} N={N} d_k={cfg.d_k} d_v={cfg.d_v}", "ms_per_call": ms,
           "kernel": "chunked MFMA" if chunked else "row-parallel fp32",
           "tokens_per_s": cfg.R * N / (ms * 1e-3), "fp32_flops": flops,
           "achieved_TFLOPs": flops / (ms * 1e-3) / 1e12,
           "roofline": roof,
           "algorithmic_bytes": nbytes, "achieved_GBs": nbytes / (ms * 1e-3) / 1e9,
           "note": "call time: the prefill kernels plus the state's transpose and bf16 split"}
    if with_cpu:
        import oracle
        pf_k = ctx_in[0][:1, :, :1].cpu().numpy()
        pf_v = ctx_in[1][:1, :, :1].cpu().numpy()
        pf_a = ctx_in[2][:1, :, :1].cpu().numpy()
        pf_b = ctx_in[3][:1, :, :1].cpu().numpy()
        t0 = time.perf_counter()
        oracle.prefill(pf_k, pf_v, pf_a, pf_b)
        one = time.perf_counter() - t0
        out["cpu_oracle_ms_est"] = one * heads * 1e3
        out["cpu_sample"] = f"one head x {N} tokens in {one * 1e3:.0f} ms, scaled by {heads} heads"
    return out


def stack_bench(torch, cfg, layers: int, step_ms: float, reps: int = 3):
    """Whole beam-search decodes through ``layers`` random-weight GDN layers (hidden size H * d_v, 256
    candidates), timed end to end with HIP events around the calls on the current stream."""
    from linear_attention_beam_amd import harness
    sc = harness.StackConfig(R=cfg.R, B=cfg.B, L=cfg.L, layers=layers, H=cfg.H, d_k=cfg.d_k, d_v=cfg.d_v,
                             D=cfg.H * cfg.d_v, n_cand=256, prefill_tokens=64, alpha_lo=cfg.alpha_lo)
    stack = harness.GDNStack(sc)
    stack.decode()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        stack.decode()
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / reps
    stack.close()
    del stack
    return {"shape": f"layers={layers} D={sc.D} n_cand={sc.n_cand} R={sc.R} H={sc.H} B={sc.B} L={sc.L}",
            "ms_per_decode": ms, "beam_tokens_per_s": cfg.beam_tokens / (ms * 1e-3),
            "step_share_est": layers * step_ms / ms,
            "note": "step_share_est = layers x the decode-step time measured above / this time; the first "
                    "step decodes min(B, 256) beams, so the share is an upper estimate"}


def cpu_baseline(cfg, steps, budget_s: float):
    """Time the CPU oracle's record-replay decode on whole requests (every head, beam and step)."""
    import oracle
    from linear_attention_beam_amd import inputs
    try:
        import threadpoolctl
        blas_threads = max((i.get("num_threads", 1) for i in threadpoolctl.threadpool_info()
                            if i.get("user_api") == "blas"), default=1)
    except Exception:  # noqa: BLE001
        blas_threads = None
    cores = len(os.sched_getaffinity(0))

    def head_steps(r, h):
        f = inputs.bf16_bits_to_f32 if cfg.qkv_dtype == "bf16" else (lambda x: x)
        return [dict(q=f(s.q[r, :, h])[None, :, None], k=f(s.k[r, :, h])[None, :, None],
                     v=f(s.v[r, :, h])[None, :, None], alpha=s.alpha[r, :, h][None, :, None],
                     beta=s.beta[r, :, h][None, :, None], parent=s.parent[r][None]) for s in steps]

    # The decode's cost does not depend on the values of S_ctx, so the state comes from the seeded generator
    # (same shape) rather than from a float64 prefill of 5120 tokens per head, which would dominate the run.
    sctx_all = inputs.direct_sctx(dataclasses.replace(cfg, sctx_std=0.1))
    elapsed, reqs = 0.0, 0
    while reqs < cfg.R and (reqs == 0 or elapsed < budget_s):
        r = reqs
        hs = [head_steps(r, h) for h in range(cfg.H)]
        t0 = time.perf_counter()
        for h in range(cfg.H):
            oracle.decode_replay(sctx_all[r, h][None, None], hs[h], cfg.B, cfg.L)
        elapsed += time.perf_counter() - t0
        reqs += 1
    return {"value": reqs * cfg.B * cfg.L / elapsed, "unit": "beam-tokens/s", "cores": cores,
            "blas_threads": blas_threads, "kind": "oracle",
            "sample": f"requests 0..{reqs - 1} of {cfg.R}: every head, beam and decode step (record-replay form, "
                      f"float64 numpy; S_ctx of the same shape from the seeded generator)",
            "seconds": round(elapsed, 3)}


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20, help="timed decodes")
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", type=int, default=3, help="workload index (default 3: R=32 H=16 B=512 L=8)")
    ap.add_argument("--tile-beams", type=int, default=0)
    ap.add_argument("--cpu-budget", type=float, default=20.0, help="seconds of CPU-baseline work")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-fullstate", action="store_true")
    ap.add_argument("--no-select", action="store_true", help="skip the beam-selection measurement")
    ap.add_argument("--no-materialize", action="store_true", help="skip the materializing-replay comparison")
    ap.add_argument("--no-stack", action="store_true", help="skip the multi-layer random-weight decode")
    ap.add_argument("--stack-layers", type=int, default=4)
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="before the benchmark, run a 1 GiB float32 elementwise copy three times (reads 1 GiB, writes "
                         "1 GiB) so hardware counters of a known-size transfer sit in the same profile")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE={world}): the decode shards "
              "by request or head with no exchange between GPUs, so N GPUs give N independent copies of this "
              "measurement.", file=sys.stderr)
        sys.exit(2)

    import torch
    from linear_attention_beam_amd import inputs, onela

    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    cfg = inputs.config(args.config)
    if args.calibrate_copy:
        src = torch.ones(1 << 28, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.mul(src, 1.0, out=dst)
        torch.cuda.synchronize()
        del src, dst
    log(f"[bench] workload: {cfg.name}")
    t0 = time.time()
    steps = inputs.decode_inputs(cfg)
    pf = inputs.prefill_inputs(cfg) if cfg.prefill_steps else None
    log(f"[bench] inputs generated in {time.time() - t0:.1f}s")

    def up(a):
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    dsteps = [dict(q=up(s.q), k=up(s.k), v=up(s.v), alpha=up(s.alpha), beta=up(s.beta), parent=up(s.parent))
              for s in steps]
    outs = [torch.empty((cfg.R, cfg.B, cfg.H, cfg.d_v), dtype=torch.float32, device=dev) for _ in range(cfg.L)]

    ctx = onela.OneLA(cfg.R, cfg.H, cfg.d_k, cfg.d_v, cfg.B, cfg.L, qkv_dtype=cfg.qkv_dtype,
                      tile_beams=args.tile_beams, device=dev)
    stream = torch.cuda.current_stream(dev)
    ev = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731
    e0, e1 = ev(), ev()
    ctx_in = [up(pf.k), up(pf.v), up(pf.alpha), up(pf.beta)] if pf is not None else [up(inputs.direct_sctx(cfg))]
    torch.cuda.synchronize()
    e0.record(stream)
    if pf is not None:
        ctx.prefill(*ctx_in)
    else:
        ctx.set_context(*ctx_in)
    e1.record(stream)
    torch.cuda.synchronize()
    context_ms = e0.elapsed_time(e1)
    log(f"[bench] context ready ({'prefill ' + str(cfg.prefill_steps) + ' tokens' if pf else 'set_context'}: "
        f"{context_ms:.2f} ms)")
    prefill_line = None
    if pf is not None:
        prefill_line = prefill_bench(torch, ctx, ctx_in, cfg, stream, with_cpu=not args.no_cpu_baseline)
        log(f"[bench] prefill: {prefill_line['ms_per_call']:.3f} ms/call, {prefill_line['achieved_TFLOPs']:.1f} "
            f"TFLOP/s fp32")
    del ctx_in

    def decode(events=None):
        ctx.reset()
        for t in range(cfg.L):
            if events is not None:
                events[t][0].record(stream)
            ctx.step(**dsteps[t], out=outs[t])
            if events is not None:
                events[t][1].record(stream)

    for _ in range(args.warmup):
        decode()
    torch.cuda.synchronize()
    if ctx.status() != onela.ONELA_OK:
        raise RuntimeError("device flag: parent index out of range")
    view = ctx.view()
    chains = view["chains"].cpu().numpy()
    per_launch_bytes = algorithmic_bytes(cfg, chains, [s.parent for s in steps])
    log(f"[bench] warmup done; algorithmic bytes per decode {sum(per_launch_bytes) / 1e9:.3f} GB")

    launch_events = [[[ev(), ev()] for _ in range(cfg.L)] for _ in range(args.steps)]
    start, stop = ev(), ev()
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    start.record(stream)
    for k in range(args.steps):
        decode(launch_events[k])
    stop.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    total_ms = start.elapsed_time(stop)
    ms_per_step = total_ms / args.steps
    kernel_ms = np.array([[e[0].elapsed_time(e[1]) for e in row] for row in launch_events])  # [K, L]
    kernel_avg_ms = float(kernel_ms.mean())
    achieved = sum(per_launch_bytes) / (kernel_ms.sum(axis=1).mean() * 1e-3) / 1e9
    value = cfg.beam_tokens / (ms_per_step * 1e-3)
    log(f"[bench] {args.steps} decodes: {ms_per_step:.4f} ms/decode (wall {wall / args.steps * 1e3:.4f}), "
        f"{value:.4g} beam-tokens/s; fused kernel avg {kernel_avg_ms * 1e3:.1f} us/launch, {achieved:.0f} GB/s")
    per_step_us = [round(float(x) * 1e3, 2) for x in kernel_ms.mean(axis=0)]

    traffic = None
    if os.path.exists(TRAFFIC_FILE):
        tr = json.load(open(TRAFFIC_FILE))
        key = f"config{args.config}"
        if tr.get("kernel_hash") == kernel_source_hash() and key in tr.get("configs", {}):
            traffic = tr["configs"][key]["bytes_per_launch"]
    mfma_flops = 8.0 * cfg.d_v * cfg.d_k * cfg.R * cfg.B * cfg.H * cfg.L   # (k and q) x (hi and lo) x 2 flops
    line = {
        "metric": "beam-tokens/sec of GDN beam-decode step",
        "value": value,
        "unit": "beam-tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.qkv_dtype,
        "data": "synthetic",
        "config": {"workload": cfg.name, "requests": cfg.R, "heads": cfg.H, "d_k": cfg.d_k, "d_v": cfg.d_v,
                   "beams": cfg.B, "decode_steps": cfg.L, "prefill_tokens": cfg.prefill_steps,
                   "beam_tokens_per_step": cfg.beam_tokens, "tile_beams": args.tile_beams or "auto"},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS,
                     "traffic": (sum(traffic) / len(traffic)) if traffic else None,
                     "kernel": "onela::step_fused_kernel",
                     "algorithmic_bytes_per_launch": sum(per_launch_bytes) / cfg.L,
                     "kernel_avg_us": kernel_avg_ms * 1e3, "kernel_us_by_decode_step": per_step_us,
                     "mfma_frac": mfma_flops / (kernel_ms.sum(axis=1).mean() * 1e-3) / (BF16_PEAK_TFLOPS * 1e12)},
        "context_ms": context_ms,
        # recurrent state kept per (beam, head) after the last step: a dense fp32 matrix (FullState) against the
        # records appended along one chain (one per step: k in the input dtype, u fp32, alpha fp32)
        "state_capacity": {"fullstate_bytes": cfg.d_v * cfg.d_k * 4,
                           "records_bytes": cfg.L * (cfg.d_k * cfg.in_bytes + 4 * cfg.d_v + 4),
                           "ratio": cfg.d_v * cfg.d_k * 4 / (cfg.L * (cfg.d_k * cfg.in_bytes + 4 * cfg.d_v + 4))},
    }
    if prefill_line is not None:
        line["prefill"] = prefill_line
    line["hbm_probe"] = hbm_probe(torch, dev)
    if not args.no_select:
        line["beam_select"] = select_bench(torch, dev, cfg, with_cpu=not args.no_cpu_baseline)
        log(f"[bench] beam selection {line['beam_select']['shape']}: {line['beam_select']['us_per_call']:.1f} us/call")
    sctx_host = np.ascontiguousarray(np.swapaxes(view["sctx_t"].cpu().numpy(), -1, -2))
    del view
    ctx.close()
    del ctx

    if not args.no_fullstate:
        fs = onela.OneLA(cfg.R, cfg.H, cfg.d_k, cfg.d_v, cfg.B, cfg.L, qkv_dtype=cfg.qkv_dtype, mode="fullstate",
                         device=dev)
        fs.set_context(torch.from_numpy(sctx_host).to(dev))

        def fs_decode():
            fs.reset()
            for t in range(cfg.L):
                fs.step(**dsteps[t], out=outs[t])

        fs_decode()
        torch.cuda.synchronize()
        reps = 3
        a, b = ev(), ev()
        a.record(stream)
        for _ in range(reps):
            fs_decode()
        b.record(stream)
        torch.cuda.synchronize()
        fs_ms = a.elapsed_time(b) / reps
        fs_bytes = 2.0 * cfg.R * cfg.B * cfg.H * cfg.d_k * cfg.d_v * 4 * cfg.L
        # compulsory: each distinct parent's state read once per step, every child's state written once
        st_bytes = cfg.H * cfg.d_k * cfg.d_v * 4.0
        fs_compulsory = sum(st_bytes * (len(np.unique(s.parent[r])) + s.parent.shape[1])
                            for s in steps for r in range(cfg.R))
        line["fullstate"] = {"ms_per_step": fs_ms, "beam_tokens_per_s": cfg.beam_tokens / (fs_ms * 1e-3),
                             "state_bytes_per_decode": fs_bytes,
                             "achieved_GBs": fs_bytes / (fs_ms * 1e-3) / 1e9,
                             "compulsory_bytes_per_decode": fs_compulsory,
                             "compulsory_GBs": fs_compulsory / (fs_ms * 1e-3) / 1e9,
                             "note": "state_bytes counts every child's read of its parent's state; siblings share "
                                     "it through the caches, so compulsory_bytes counts each distinct parent once",
                             "replay_speedup": fs_ms / ms_per_step}
        log(f"[bench] FullState: {fs_ms:.3f} ms/decode; replay is {fs_ms / ms_per_step:.1f}x faster")
        fs.close()
        del fs

    if not args.no_materialize:
        mz = onela.OneLA(cfg.R, cfg.H, cfg.d_k, cfg.d_v, cfg.B, cfg.L, qkv_dtype=cfg.qkv_dtype, materialize=True,
                         device=dev)
        mz.set_context(torch.from_numpy(sctx_host).to(dev))

        def mz_decode():
            mz.reset()
            for t in range(cfg.L):
                mz.step(**dsteps[t], out=outs[t])

        mz_decode()
        torch.cuda.synchronize()
        reps = 3
        a, b = ev(), ev()
        a.record(stream)
        for _ in range(reps):
            mz_decode()
        b.record(stream)
        torch.cuda.synchronize()
        mz_ms = a.elapsed_time(b) / reps
        flops = sum(2.0 * cfg.R * cfg.B * cfg.H * cfg.d_k * cfg.d_v * (t + 2) for t in range(cfg.L))
        line["materialize"] = {"ms_per_step": mz_ms, "beam_tokens_per_s": cfg.beam_tokens / (mz_ms * 1e-3),
                               "fp32_flops_per_decode": flops, "achieved_TFLOPs": flops / (mz_ms * 1e-3) / 1e12,
                               "replay_speedup": mz_ms / ms_per_step}
        log(f"[bench] materializing replay: {mz_ms:.3f} ms/decode; projection replay is {mz_ms / ms_per_step:.1f}x "
            "faster")
        mz.close()
        del mz

    if not args.no_stack:
        line["stack"] = stack_bench(torch, cfg, args.stack_layers, ms_per_step)
        st = line["stack"]
        log(f"[bench] {args.stack_layers}-layer decode: {st['ms_per_decode']:.3f} ms, "
            f"{st['beam_tokens_per_s']:.4g} beam-tokens/s; decode steps ~{100 * st['step_share_est']:.0f}%")

    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(cfg, steps, args.cpu_budget)
        log(f"[bench] CPU oracle: {line['cpu_baseline']['value']:.4g} beam-tokens/s "
            f"({line['cpu_baseline']['sample']})")
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
