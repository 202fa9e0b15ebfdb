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
