#!/usr/bin/env python3
"""Benchmark of the large-beam Gated DeltaNet decode step on one MI355X.

One bench "step" is one whole decode of the workload: L onela_step calls (ancestry index update, shared
S_ctx contraction, key and query replay, record append, output: at step 1 one fused kernel, later an
ancestry-plan kernel and the fused kernel) over R requests x B beams x H heads, after onela_reset.  Inputs
(all L steps) and the context are resident in HBM before timing starts.  value = beam-tokens per second =
R * B * L / (median seconds per decode over the timed decodes, HIP events at each decode's two ends).

Prints one JSON line.  Extra objects:
  roofline      one onela_step (its two kernels): algorithmic HBM bytes per step (compulsory traffic, counted
                from the run's own chain tables) / the step's median time from HIP events around each step on
                its stream, in a second pass of the timed decodes.  `fused_kernel_only`: the same bytes over the
                fused kernel's own time (plan kernel and launch gap left out) from the committed rocprofv3
                trace, when it was taken on the current kernel source
  configs       the same measurement (decode time, rate, bytes, fraction, FullState speed-up, CPU oracle) for
                each workload of the table (default: the four GPU-sized workloads, the headline one included)
  cpu_baseline  the float64 CPU oracle (record-replay form) timed on (request, head) pairs of the same
                workload, scaled to beam-tokens/s of whole requests
  fullstate     the controlled FullState path (dense per-beam state) on the same inputs
  materialize   the materializing-replay path (each beam's dense parent state rebuilt every step) on the same
                inputs
  hbm_probe     read-only, 2:3 read:write mix, copy and write-only bandwidth of plain streaming kernels
                (libonela_probe.so) on the same GPU, and the first decode step's traffic (the same rows read
                and written at the workload's shape) from a plain kernel without the arithmetic (context for
                the fraction)
  beam_select   the beam selection that produces each step's parents (top B of B x 256 candidate scores per
                request), timed on its own with HIP events; not part of the decode step above
  prefill       onela_prefill of the workload's prompt (the context the decode starts from), against the dense
                bf16 MFMA peak for the chunked kernels (d_k = 128), else the fp32 vector-ALU peak
  geometry_sweep  decode time, bytes and fraction over d_k x d_v in {64, 128, 256}^2 at one workload shape
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
FP32_PEAK_TFLOPS = 78.6      # MI355X fp32 vector without packed FP32: 256 CUs x 64 lanes x 2 (FMA) x 2.4 GHz
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "fused_step_traffic.json")
FUSED_SRC = os.path.join(ROOT, "linear_attention_beam_amd", "csrc", "step_fused.hip")


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def kernel_source_hash() -> str:
    """Hash of the step kernels' source code, comments and blank lines left out (the code the counters ran)."""
    lines = []
    for line in open(FUSED_SRC, encoding="utf-8"):
        code = line.split("//", 1)[0].rstrip()
        if code:
            lines.append(code)
    return hashlib.sha256("\n".join(lines).encode()).hexdigest()[:16]


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


def step_traffic_probe(torch, dev, lib, cfg, reps: int = 5):
    """The first decode step's traffic without its arithmetic (onela_probe_step_traffic: the same k, q, v, alpha,
    beta and S_ctx reads and o, u, key and alpha writes, one plain workgroup per (request, head, 32-beam tile)) at
    the workload's shape, best of ``reps``: the rate this access pattern reaches on this GPU."""
    import ctypes
    R, B, H, dv, slots = cfg.R, cfg.B, cfg.H, cfg.d_v, cfg.B * cfg.L
    fn = lib.onela_probe_step_traffic
    fn.argtypes = [ctypes.c_void_p] * 10 + [ctypes.c_int] * 5 + [ctypes.c_void_p]
    fn.restype = ctypes.c_int
    bf = torch.bfloat16
    k = torch.ones((R, B, H, 128), dtype=bf, device=dev)
    q = torch.ones((R, B, H, 128), dtype=bf, device=dev)
    v = torch.ones((R, B, H, dv), dtype=bf, device=dev)
    ab = torch.ones((2, R, B, H), dtype=torch.float32, device=dev)
    sctx = torch.ones((R * H, 128, dv), dtype=torch.float32, device=dev)
    o = torch.empty((R, B, H, dv), dtype=torch.float32, device=dev)
    u = torch.empty((R * H, slots, dv), dtype=torch.float32, device=dev)
    rk = torch.empty((R * H, slots, 128), dtype=bf, device=dev)
    ra = torch.empty((R * H, slots), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)
    args = [t.data_ptr() for t in (k, q, v, ab[0], ab[1], sctx, o, u, rk, ra)] + [R, B, H, dv, slots,
                                                                                    stream.cuda_stream]
    nbytes = R * B * H * (2 * 256 + 2 * dv + 8 + 4 * dv + 4 * dv + 256 + 4) + R * H * 128 * dv * 4
    if fn(*args) != 0:
        raise RuntimeError("onela_probe_step_traffic failed")
    torch.cuda.synchronize()
    best_us = float("inf")
    for _ in range(reps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        fn(*args)
        b.record(stream)
        torch.cuda.synchronize()
        best_us = min(best_us, a.elapsed_time(b) * 1e3)
    del k, q, v, ab, sctx, o, u, rk, ra
    return {"workload": cfg.name, "bytes": nbytes, "us": best_us, "GBs": nbytes / (best_us * 1e-6) / 1e9,
            "kernel": "onela_probe_step_traffic (one 256-thread workgroup per request, head and 32-beam tile)"}


def hbm_probe(torch, dev, cfg=None, gib: float = 2.0):
    """Bandwidth of plain streaming kernels (libonela_probe.so, 16-byte accesses, one element per thread) on this
    GPU, best of 5 each:
    read-only, the 2:3 read:write mix of the decode step, copy (1:1) and write-only.  Context for the roofline
    fraction (whose peak stays the published 8 TB/s); not part of the timed decode."""
    import ctypes
    path = os.path.join(ROOT, "linear_attention_beam_amd", "lib", "libonela_probe.so")
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with `python -m linear_attention_beam_amd.build`")
    lib = ctypes.CDLL(path)
    lib.onela_probe_stream.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int,
                                       ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p]
    lib.onela_probe_stream.restype = ctypes.c_int
    n = int(gib * (1 << 30)) // 16                      # 16-byte elements per stream
    src = torch.ones(2 * n * 4, dtype=torch.float32, device=dev)
    dst = torch.empty(3 * n * 4, dtype=torch.float32, device=dev)
    grid = 0  # one element per thread: faster than any grid-stride form of these kernels on this GPU
    sink = torch.empty(256, dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)

    def best(mode, nbytes):
        def run():
            rc = lib.onela_probe_stream(src.data_ptr(), dst.data_ptr(), n, mode, sink.data_ptr(), grid,
                                        stream.cuda_stream)
            if rc != 0:
                raise RuntimeError(f"onela_probe_stream mode {mode} failed ({rc})")
        run()
        torch.cuda.synchronize()
        out = 0.0
        for _ in range(5):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            run()
            b.record(stream)
            torch.cuda.synchronize()
            out = max(out, nbytes / (a.elapsed_time(b) * 1e-3) / 1e9)
        return out

    res = {"read_GBs": best(0, 32.0 * n), "mix_2r3w_GBs": best(1, 80.0 * n), "copy_GBs": best(2, 32.0 * n),
           "write_GBs": best(3, 16.0 * n), "bytes_per_stream": 16 * n,
           "kernel": "onela_probe_stream (16-byte loads/stores, one element per thread)"}
    del src, dst, sink
    if cfg is not None:
        res["step1_traffic"] = step_traffic_probe(torch, dev, lib, cfg)
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
    state update (128 x d_v x 32), each as three bf16 products (high/low halves).  The roofline counts the
    method's own work (the recurrence's 4 d_k d_v FLOPs per token and head) against the bf16 MFMA peak; the
    MFMA products actually issued (the chunked form's extra work and the three-way split) are reported beside
    it as mfma_issued."""
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
    achieved = flops / (ms * 1e-3) / 1e12
    if chunked:
        chunks = -(-N // 32)
        per_chunk = 3 * 2.0 * (3 * 16 * 16 * 128 + 32 * cfg.d_v * 128 + 32 * cfg.d_v * 32 + 128 * cfg.d_v * 32)
        mfma_flops = per_chunk * chunks * heads
        roof = {"bound": "mfma", "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s", "dtype": "bf16 (high/low halves)",
                "work": "4 d_k d_v FLOPs per token and head (the recurrence's own work)",
                "achieved": achieved, "frac": achieved / BF16_PEAK_TFLOPS,
                "mfma_issued_flops": mfma_flops, "mfma_issued_TFLOPs": mfma_flops / (ms * 1e-3) / 1e12,
                "mfma_issued_frac": mfma_flops / (ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS}
    else:
        roof = {"bound": "alu", "peak": FP32_PEAK_TFLOPS, "unit": "TFLOP/s",
                "work": "4 d_k d_v FLOPs per token and head", "achieved": achieved,
                "frac": achieved / FP32_PEAK_TFLOPS}
    out = {"shape": f"R={cfg.R} H={cfg.H} N={N} d_k={cfg.d_k} d_v={cfg.d_v}", "ms_per_call": ms,
           "kernel": "chunked MFMA" if chunked else "row-parallel fp32",
           "tokens_per_s": cfg.R * N / (ms * 1e-3), "fp32_flops": flops,
           "achieved_TFLOPs": achieved,
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
    """Time the CPU oracle's record-replay decode on (request, head) pairs of the workload (every beam and step
    of each pair), as many as fit the budget (at least one), scaled to beam-tokens/s of whole requests."""
    import oracle
    from linear_attention_beam_amd import inputs
    try:
        import threadpoolctl
        blas_threads = max((i.get("num_threads", 1) for i in threadpoolctl.threadpool_info()
                            if i.get("user_api") == "blas"), default=1)
    except Exception:  # noqa: BLE001
        blas_threads = None
    cores = len(os.sched_getaffinity(0))
    f = inputs.bf16_bits_to_f32 if cfg.qkv_dtype == "bf16" else (lambda x: x)

    def head_steps(r, h):
        return [dict(q=f(s.q[r, :, h])[None, :, None], k=f(s.k[r, :, h])[None, :, None],
                     v=f(s.v[r, :, h])[None, :, None], alpha=s.alpha[r, :, h][None, :, None],
                     beta=s.beta[r, :, h][None, :, None], parent=s.parent[r][None]) for s in steps]

    # The decode's cost does not depend on the values of S_ctx, so the state comes from the seeded generator
    # (same shape) rather than from a float64 prefill of the prompt, which would dominate the run.
    sctx_all = inputs.direct_sctx(dataclasses.replace(cfg, sctx_std=0.1))
    elapsed, pairs = 0.0, 0
    while pairs < cfg.R * cfg.H and (pairs == 0 or elapsed < budget_s):
        r, h = divmod(pairs, cfg.H)
        hs = head_steps(r, h)
        t0 = time.perf_counter()
        oracle.decode_replay(sctx_all[r, h][None, None], hs, cfg.B, cfg.L)
        elapsed += time.perf_counter() - t0
        pairs += 1
    return {"value": pairs * cfg.B * cfg.L / cfg.H / elapsed, "unit": "beam-tokens/s", "cores": cores,
            "blas_threads": blas_threads, "kind": "oracle",
            "sample": f"{pairs} of {cfg.R * cfg.H} (request, head) pairs, each with every beam and decode step "
                      f"(record-replay form, float64 numpy; S_ctx of the same shape from the seeded generator); "
                      f"rate = pairs x B x L / H / seconds",
            "seconds": round(elapsed, 3)}


def upload(torch, dev, a):
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev)


def profile_of(config_index: int):
    """The committed rocprofv3 figures of a workload (HBM bytes per step from the counter runs, kernel times per
    step from the trace), if they were taken on the current kernel source."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    tr = json.load(open(TRAFFIC_FILE))
    key = f"config{config_index}"
    if tr.get("kernel_hash") == kernel_source_hash() and key in tr.get("configs", {}):
        return tr["configs"][key]
    return None


def traffic_of(config_index: int):
    prof = profile_of(config_index)
    return prof["bytes_per_launch"] if prof else None


def fused_kernel_roofline(config_index: int, bytes_by_step):
    """The step's algorithmic bytes over the fused kernel's own rocprof time (plan kernel and launch gap left
    out), from the committed trace of the current kernel source; None without one."""
    prof = profile_of(config_index)
    if not prof or "fused_us" not in prof or len(prof["fused_us"]) != len(bytes_by_step):
        return None
    us = prof["fused_us"]
    achieved = sum(bytes_by_step) / (sum(us) * 1e-6) / 1e9
    return {"kernel": "step_fused_kernel", "us_by_decode_step": us, "plan_us_by_decode_step": prof.get("plan_us"),
            "achieved": achieved, "frac": achieved / HBM_PEAK_GBS,
            "source": "rocprofv3 kernel trace of the default bench (profiles/, same kernel source hash)"}


SWEEP_SIZES = (64, 128, 256)


def geometry_sweep(torch, onela, inputs, dev, sizes, steps: int = 10, warmup: int = 2):
    """Decode time over head geometries d_k x d_v (the pages' operator sweep varies the recurrent geometry; its
    shapes are not listed): R=16 requests x H=16 heads x 512 beams, 6 steps, Zipf(1.1) parents, alpha ~ U(0.95, 1),
    S_ctx drawn directly (the step's time does not depend on its values).  Each point: the median of `steps`
    decodes timed with HIP events, algorithmic bytes from the run's own chain tables, and which kernel ran."""
    points = []
    for d_k in sizes:
        for d_v in sizes:
            cfg = inputs.config(4, R=16, H=16, d_k=d_k, d_v=d_v, B=512, L=6, prefill_steps=0, sctx_std=0.05,
                                name=f"R=16 H=16 dk={d_k} dv={d_v} B=512 L=6 bf16 zipf1.1")
            steps_in = inputs.decode_inputs(cfg)
            dsteps = [dict(q=upload(torch, dev, s.q), k=upload(torch, dev, s.k), v=upload(torch, dev, s.v),
                           alpha=upload(torch, dev, s.alpha), beta=upload(torch, dev, s.beta),
                           parent=upload(torch, dev, s.parent)) for s in steps_in]
            outs = [torch.empty((cfg.R, cfg.B, cfg.H, cfg.d_v), dtype=torch.float32, device=dev)
                    for _ in range(cfg.L)]
            ctx = onela.OneLA(cfg.R, cfg.H, cfg.d_k, cfg.d_v, cfg.B, cfg.L, qkv_dtype=cfg.qkv_dtype, device=dev)
            ctx.set_context(upload(torch, dev, inputs.direct_sctx(cfg)))
            stream = torch.cuda.current_stream(dev)
            ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(steps)]
            for k in range(warmup + steps):
                ctx.reset()
                if k >= warmup:
                    ev[k - warmup][0].record(stream)
                for t in range(cfg.L):
                    ctx.step(**dsteps[t], out=outs[t])
                if k >= warmup:
                    ev[k - warmup][1].record(stream)
            torch.cuda.synchronize()
            if ctx.status() != onela.ONELA_OK:
                raise RuntimeError("device flag: parent index out of range")
            view = ctx.view()
            nbytes = sum(algorithmic_bytes(cfg, view["chains"].cpu().numpy(), [s.parent for s in steps_in]))
            ms = float(np.median([a.elapsed_time(b) for a, b in ev]))
            points.append({"d_k": d_k, "d_v": d_v, "kernel": "fused" if view["fused"] else "fp32",
                           "ms_per_decode": ms,
                           "beam_tokens_per_s": cfg.beam_tokens / (ms * 1e-3),
                           "algorithmic_bytes_per_decode": nbytes,
                           "achieved_GBs": nbytes / (ms * 1e-3) / 1e9,
                           "frac": nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS})
            log(f"[bench] sweep d_k={d_k} d_v={d_v}: {ms:.3f} ms/decode, {points[-1]['frac']:.3f} of peak "
                f"({points[-1]['kernel']})")
            del view
            ctx.close()
            del ctx, dsteps, outs
            torch.cuda.empty_cache()
    return {"workload": "R=16 H=16 B=512 L=6 bf16 zipf1.1, S_ctx drawn directly; d_k x d_v over "
                        + ", ".join(str(x) for x in sizes),
            "timing": "HIP events around each decode (the plan and fused launches and the gaps between them); "
                      "median over the timed decodes",
            "points": points}


def measure_config(torch, onela, inputs, dev, index: int, args, headline: bool):
    """Decode benchmark of one workload: the context from a GPU prefill of the workload's prompt, W warm-up
    decodes, then two timed passes of K decodes on the stream the steps run on: HIP events at each decode's ends
    only (the decode time and throughput), then HIP events around every step as well (the per-launch times of
    the roofline; each event pair adds a marker between the steps, about 60 us per decode at cfg 3).  Returns
    the per-config record and, for the headline workload, the objects the rest of the line needs."""
    cfg = inputs.config(index)
    t0 = time.time()
    steps = inputs.decode_inputs(cfg)
    pf = inputs.prefill_inputs(cfg) if cfg.prefill_steps else None
    log(f"[bench] config{index} {cfg.name}: inputs generated in {time.time() - t0:.1f}s")
    dsteps = [dict(q=upload(torch, dev, s.q), k=upload(torch, dev, s.k), v=upload(torch, dev, s.v),
                   alpha=upload(torch, dev, s.alpha), beta=upload(torch, dev, s.beta),
                   parent=upload(torch, dev, s.parent)) for s in steps]
    outs = [torch.empty((cfg.R, cfg.B, cfg.H, cfg.d_v), dtype=torch.float32, device=dev) for _ in range(cfg.L)]
    ctx = onela.OneLA(cfg.R, cfg.H, cfg.d_k, cfg.d_v, cfg.B, cfg.L, qkv_dtype=cfg.qkv_dtype,
                      tile_beams=args.tile_beams if headline else 0, device=dev)
    stream = torch.cuda.current_stream(dev)
    ev = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731
    ctx_in = ([upload(torch, dev, pf.k), upload(torch, dev, pf.v), upload(torch, dev, pf.alpha),
               upload(torch, dev, pf.beta)] if pf is not None else [upload(torch, dev, inputs.direct_sctx(cfg))])
    torch.cuda.synchronize()
    e0, e1 = ev(), ev()
    e0.record(stream)
    if pf is not None:
        ctx.prefill(*ctx_in)
    else:
        ctx.set_context(*ctx_in)
    e1.record(stream)
    torch.cuda.synchronize()
    extra = {"context_ms": e0.elapsed_time(e1)}
    if headline and pf is not None:
        extra["prefill"] = prefill_bench(torch, ctx, ctx_in, cfg, stream, with_cpu=not args.no_cpu_baseline)
        log(f"[bench] prefill: {extra['prefill']['ms_per_call']:.3f} ms/call, "
            f"{extra['prefill']['achieved_TFLOPs']:.1f} TFLOP/s of the recurrence's own work")
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
    per_step_bytes = algorithmic_bytes(cfg, chains, [s.parent for s in steps])

    K = args.steps
    # pass 1: events at the decode's ends (onela_reset enqueues nothing, so a decode is its L steps)
    ends = [[ev(), ev()] for _ in range(K)]
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    for k in range(K):
        ends[k][0].record(stream)
        decode()
        ends[k][1].record(stream)
    torch.cuda.synchronize()
    wall = (time.perf_counter() - wall0) / K
    decode_ms = np.array([a.elapsed_time(b) for a, b in ends])
    ms = float(np.median(decode_ms))
    # pass 2: events around every step as well
    step_events = [[[ev(), ev()] for _ in range(cfg.L)] for _ in range(K)]
    torch.cuda.synchronize()
    for k in range(K):
        decode(step_events[k])
    torch.cuda.synchronize()
    step_ms = np.array([[e[0].elapsed_time(e[1]) for e in row] for row in step_events])     # [K, L]
    decode_ms_step_events = np.array([row[0][0].elapsed_time(row[-1][1]) for row in step_events])
    step_med = np.median(step_ms, axis=0)                                                    # [L]
    # the roofline's time: the median decode's steps (the step of each launch pair, its gaps excluded)
    step_sum = float(np.median(step_ms.sum(axis=1)))
    achieved = sum(per_step_bytes) / (step_sum * 1e-3) / 1e9
    mfma_flops = 8.0 * cfg.d_v * cfg.d_k * cfg.R * cfg.B * cfg.H * cfg.L   # (k and q) x (hi and lo) x 2 flops
    traffic = traffic_of(index)
    rec = {
        "workload": cfg.name,
        "ms_per_step": ms,
        "beam_tokens_per_s": cfg.beam_tokens / (ms * 1e-3),
        "decode_ms_min_max": [float(decode_ms.min()), float(decode_ms.max())],
        "decode_ms_with_step_events": float(np.median(decode_ms_step_events)),
        "algorithmic_bytes_per_launch": sum(per_step_bytes) / cfg.L,
        "algorithmic_bytes_by_decode_step": per_step_bytes,
        "step_us_by_decode_step": [round(float(x) * 1e3, 2) for x in step_med],
        "achieved_GBs": achieved,
        "frac": achieved / HBM_PEAK_GBS,
        "traffic_bytes_per_launch": (sum(traffic) / len(traffic)) if traffic else None,
        "mfma_frac": mfma_flops / (step_sum * 1e-3) / (BF16_PEAK_TFLOPS * 1e12),
        "wall_ms_per_decode": wall * 1e3,
    }
    fk = fused_kernel_roofline(index, per_step_bytes)
    rec["frac_fused_kernel_only"] = fk["frac"] if fk else None
    log(f"[bench] config{index}: {ms:.4f} ms/decode (median of {K}), {rec['beam_tokens_per_s']:.4g} beam-tokens/s, "
        f"{achieved:.0f} GB/s = {rec['frac']:.3f} of peak; steps {rec['step_us_by_decode_step']} us")
    sctx_host = np.ascontiguousarray(np.swapaxes(view["sctx_t"].cpu().numpy(), -1, -2))
    del view
    if headline:
        extra.update(ctx=ctx, steps=steps, dsteps=dsteps, outs=outs, cfg=cfg, sctx_host=sctx_host, stream=stream,
                     step_ms=step_ms, chains=chains)
    else:
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
        times = []
        for _ in range(3):
            a, b = ev(), ev()
            a.record(stream)
            fs_decode()
            b.record(stream)
            torch.cuda.synchronize()
            times.append(a.elapsed_time(b))
        fs_ms = float(np.median(times))
        rec["fullstate_ms_per_step"] = fs_ms
        rec["fullstate_speedup"] = fs_ms / ms
        if headline:
            fs_bytes = 2.0 * cfg.R * cfg.B * cfg.H * cfg.d_k * cfg.d_v * 4 * cfg.L
            # compulsory: each distinct parent's state read once per step, every child's state written once
            st_bytes = cfg.H * cfg.d_k * cfg.d_v * 4.0
            fs_compulsory = sum(st_bytes * (len(np.unique(s.parent[r])) + s.parent.shape[1])
                                for s in steps for r in range(cfg.R))
            extra["fullstate"] = {
                "ms_per_step": fs_ms, "beam_tokens_per_s": cfg.beam_tokens / (fs_ms * 1e-3),
                "state_bytes_per_decode": fs_bytes, "achieved_GBs": fs_bytes / (fs_ms * 1e-3) / 1e9,
                "compulsory_bytes_per_decode": fs_compulsory,
                "compulsory_GBs": fs_compulsory / (fs_ms * 1e-3) / 1e9,
                "note": "state_bytes counts every child's read of its parent's state; siblings share it through the "
                        "caches, so compulsory_bytes counts each distinct parent once",
                "replay_speedup": fs_ms / ms}
        log(f"[bench] config{index} FullState: {fs_ms:.3f} ms/decode; replay is {fs_ms / ms:.1f}x faster")
        fs.close()
        del fs

    if not args.no_cpu_baseline:
        budget = args.cpu_budget if headline else args.cpu_budget / 3
        rec["cpu_baseline"] = cpu_baseline(cfg, steps, budget)
        log(f"[bench] config{index} CPU oracle: {rec['cpu_baseline']['value']:.4g} beam-tokens/s "
            f"({rec['cpu_baseline']['seconds']} s)")
    return rec, extra


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20, help="timed decodes per workload")
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", type=int, default=3, help="headline workload (default 3: R=32 H=16 B=512 L=8)")
    ap.add_argument("--table-configs", default="1,2,3,4",
                    help="workloads of the per-config table (comma-separated indices, or 'none')")
    ap.add_argument("--tile-beams", type=int, default=0)
    ap.add_argument("--cpu-budget", type=float, default=20.0,
                    help="seconds of CPU-oracle work for the headline workload (a third of it for each other one)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-fullstate", action="store_true")
    ap.add_argument("--no-select", action="store_true", help="skip the beam-selection measurement")
    ap.add_argument("--no-materialize", action="store_true", help="skip the materializing-replay comparison")
    ap.add_argument("--no-stack", action="store_true", help="skip the multi-layer random-weight decode")
    ap.add_argument("--stack-layers", type=int, default=4)
    ap.add_argument("--no-sweep", action="store_true", help="skip the head-geometry sweep")
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
    if args.calibrate_copy:
        src = torch.ones(1 << 28, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.mul(src, 1.0, out=dst)
        torch.cuda.synchronize()
        del src, dst

    rec, extra = measure_config(torch, onela, inputs, dev, args.config, args, headline=True)
    cfg, ctx = extra["cfg"], extra["ctx"]
    ms_per_step = rec["ms_per_step"]
    line = {
        "metric": "beam-tokens/sec of GDN beam-decode step",
        "value": rec["beam_tokens_per_s"],
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
        "roofline": {"bound": "hbm", "achieved": rec["achieved_GBs"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": rec["frac"], "traffic": rec["traffic_bytes_per_launch"],
                     "kernel": "onela_step: ancestry_plan_kernel (steps >= 2) + step_fused_kernel",
                     "algorithmic_bytes_per_launch": rec["algorithmic_bytes_per_launch"],
                     "kernel_avg_us": float(np.mean(rec["step_us_by_decode_step"])),
                     "kernel_us_by_decode_step": rec["step_us_by_decode_step"],
                     "timing": "HIP events around each onela_step on its stream, in a second pass of the timed "
                               "decodes; median per decode step (value and ms_per_step: events at each decode's "
                               "ends only, median over the first pass)",
                     "mfma_frac": rec["mfma_frac"],
                     "fused_kernel_only": fused_kernel_roofline(args.config, rec["algorithmic_bytes_by_decode_step"])},
        "context_ms": extra["context_ms"],
        # recurrent state kept per (beam, head) after the last step: a dense fp32 matrix (FullState) against the
        # records appended along one chain (one per step: k in the input dtype, u fp32, alpha fp32)
        "state_capacity": {"fullstate_bytes": cfg.d_v * cfg.d_k * 4,
                           "records_bytes": cfg.L * (cfg.d_k * cfg.in_bytes + 4 * cfg.d_v + 4),
                           "ratio": cfg.d_v * cfg.d_k * 4 / (cfg.L * (cfg.d_k * cfg.in_bytes + 4 * cfg.d_v + 4))},
    }
    if "prefill" in extra:
        line["prefill"] = extra["prefill"]
    if "fullstate" in extra:
        line["fullstate"] = extra["fullstate"]
    line["hbm_probe"] = hbm_probe(torch, dev, cfg)
    st1 = line["hbm_probe"]["step1_traffic"]
    # step 1 of the timed decodes against the same traffic from a plain kernel
    st1["decode_step1_us"] = rec["step_us_by_decode_step"][0]
    st1["probe_over_decode_step1"] = st1["us"] / rec["step_us_by_decode_step"][0]
    log(f"[bench] probes: read {line['hbm_probe']['read_GBs']:.0f}, 2:3 mix {line['hbm_probe']['mix_2r3w_GBs']:.0f}, "
        f"copy {line['hbm_probe']['copy_GBs']:.0f}, write {line['hbm_probe']['write_GBs']:.0f} GB/s; "
        f"step-1 traffic of {st1['workload']}: {st1['GBs']:.0f} GB/s ({st1['us']:.1f} us)")
    if not args.no_select:
        line["beam_select"] = select_bench(torch, dev, cfg, with_cpu=not args.no_cpu_baseline)
        log(f"[bench] beam selection {line['beam_select']['shape']}: {line['beam_select']['us_per_call']:.1f} us/call")

    if not args.no_materialize:
        stream, dsteps, outs = extra["stream"], extra["dsteps"], extra["outs"]
        mz = onela.OneLA(cfg.R, cfg.H, cfg.d_k, cfg.d_v, cfg.B, cfg.L, qkv_dtype=cfg.qkv_dtype, materialize=True,
                         device=dev)
        mz.set_context(torch.from_numpy(extra["sctx_host"]).to(dev))

        def mz_decode():
            mz.reset()
            for t in range(cfg.L):
                mz.step(**dsteps[t], out=outs[t])

        mz_decode()
        torch.cuda.synchronize()
        times = []
        for _ in range(3):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            mz_decode()
            b.record(stream)
            torch.cuda.synchronize()
            times.append(a.elapsed_time(b))
        mz_ms = float(np.median(times))
        flops = sum(2.0 * cfg.R * cfg.B * cfg.H * cfg.d_k * cfg.d_v * (t + 2) for t in range(cfg.L))
        line["materialize"] = {"ms_per_step": mz_ms, "beam_tokens_per_s": cfg.beam_tokens / (mz_ms * 1e-3),
                               "fp32_flops_per_decode": flops, "achieved_TFLOPs": flops / (mz_ms * 1e-3) / 1e12,
                               "replay_speedup": mz_ms / ms_per_step}
        log(f"[bench] materializing replay: {mz_ms:.3f} ms/decode; projection replay is {mz_ms / ms_per_step:.1f}x "
            "faster")
        mz.close()
        del mz
    ctx.close()
    del ctx, extra

    if not args.no_stack:
        line["stack"] = stack_bench(torch, cfg, args.stack_layers, ms_per_step)
        st = line["stack"]
        log(f"[bench] {args.stack_layers}-layer decode: {st['ms_per_decode']:.3f} ms, "
            f"{st['beam_tokens_per_s']:.4g} beam-tokens/s; decode steps ~{100 * st['step_share_est']:.0f}%")

    if not args.no_sweep:
        line["geometry_sweep"] = geometry_sweep(torch, onela, inputs, dev, SWEEP_SIZES)

    if "cpu_baseline" in rec:
        line["cpu_baseline"] = rec["cpu_baseline"]
    table = {}
    if args.table_configs != "none":
        for idx in (int(x) for x in args.table_configs.split(",")):
            if idx == args.config:
                table[f"config{idx}"] = rec
            else:
                table[f"config{idx}"], _ = measure_config(torch, onela, inputs, dev, idx, args, headline=False)
                torch.cuda.empty_cache()
        line["configs"] = table
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
