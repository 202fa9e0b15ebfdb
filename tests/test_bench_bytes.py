"""The algorithmic byte count behind bench.py's roofline fraction, against a case counted by hand (CPU)."""

import numpy as np

import bench
import oracle
from linear_attention_beam_amd import inputs


def test_algorithmic_bytes_hand_count():
    # one request, 2 heads, d_k = 4, d_v = 2, bf16 inputs, 3 beams, 2 steps; a record is 4*2 + 4*2 + 4 = 20 bytes
    cfg = inputs.config(1, R=1, H=2, d_k=4, d_v=2, B=3, L=2)
    assert cfg.in_bytes == 2
    parents = [np.array([[0, 0, 0]], np.int32), np.array([[2, 2, 0]], np.int32)]
    chains = np.stack(oracle.ancestry_tables([p[0] for p in parents], 3, 2))[:, None]  # [L, R, B, L]
    # step 1: S_ctx 1*2*2*4*4 = 64; q, k, v 1*3*2*(8+2)*2 = 120; alpha, beta 1*3*2*8 = 48 and parents 1*3*4 = 12;
    # o 1*3*2*2*4 = 48; appended records 1*3*2*20 = 120; chain table 1*3*2*4 = 24
    step1 = 64 + 120 + 48 + 12 + 48 + 120 + 24
    # step 2 adds the chain rows of the 2 distinct parents (0 and 2: 2 * 1 * 4 bytes) and their 2 distinct
    # records (slots 0 and 2), read once per head: 2 * 2 * 20
    step2 = step1 + 8 + 80
    assert bench.algorithmic_bytes(cfg, chains, parents) == [step1, step2] == [436, 524]


def test_fused_kernel_roofline_uses_only_a_profile_of_this_kernel(tmp_path, monkeypatch):
    """The fused kernel's own fraction comes from the committed trace only when that trace was taken on the
    current kernel source: bytes over the summed per-step kernel times, against the 8 TB/s peak."""
    import json
    prof = {"kernel_hash": bench.kernel_source_hash(),
            "configs": {"config3": {"bytes_per_launch": [1.0, 1.0], "fused_us": [100.0, 150.0],
                                    "plan_us": [0.0, 8.0]}}}
    path = tmp_path / "traffic.json"
    path.write_text(json.dumps(prof))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(path))
    r = bench.fused_kernel_roofline(3, [600e6, 900e6])
    # 1.5 GB over 250 us = 6000 GB/s = 0.75 of 8000 GB/s
    assert abs(r["achieved"] - 6000.0) < 1e-6 and abs(r["frac"] - 0.75) < 1e-12
    assert bench.fused_kernel_roofline(4, [1.0, 1.0]) is None           # no record of that workload
    assert bench.fused_kernel_roofline(3, [1.0, 1.0, 1.0]) is None      # another decode length
    prof["kernel_hash"] = "0" * 16                                       # taken on other code
    path.write_text(json.dumps(prof))
    assert bench.fused_kernel_roofline(3, [600e6, 900e6]) is None
    assert bench.traffic_of(3) is None


def test_bench_refuses_more_than_one_gpu():
    """bench.py measures one GPU: --gpus above 1 (or a multi-rank launch) exits with a message before any GPU
    work, with a nonzero status."""
    import os
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    for argv, env in ((["--gpus", "2"], {}), ([], {"WORLD_SIZE": "4"})):
        r = subprocess.run([sys.executable, os.path.join(root, "bench.py"), *argv], capture_output=True, text=True,
                           env={**os.environ, **env}, timeout=120)
        assert r.returncode == 2 and "one GPU only" in r.stderr and r.stdout == ""
