"""The allocation-free beam selection (onela_beam_select_noalloc, library-held scratch) against the entry point
that takes a caller scratch (onela_beam_select), through the C ABI, bit for bit: several calls in a row on one
GPU, each smaller than the one before, so that every call after the first finds the previous call's contents
in the shared array."""

import numpy as np
import pytest
import torch

import oracle
from linear_attention_beam_amd import inputs, onela
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu


def select_noalloc(bs, lp, n_beams):
    R, n_prev, n_cand = (int(x) for x in lp.shape)
    dev = lp.device
    parent = torch.empty((R, n_beams), dtype=torch.int32, device=dev)
    token = torch.empty((R, n_beams), dtype=torch.int32, device=dev)
    scores = torch.empty((R, n_beams), dtype=torch.float32, device=dev)
    onela.onela_beam_select_noalloc(R, n_prev, n_cand, n_beams, bs.data_ptr(), lp.data_ptr(), parent.data_ptr(),
                                    token.data_ptr(), scores.data_ptr(), torch.cuda.current_stream(dev).cuda_stream)
    return parent, token, scores


def check_pair(R, n_prev, n_cand, n_beams, seed):
    gu.log(f"noalloc select R={R} n_prev={n_prev} n_cand={n_cand} n_beams={n_beams} seed={seed}")
    dev = gu.device()
    si = inputs.select_inputs(R, n_prev, n_cand, seed=seed)
    bs, lp = torch.from_numpy(si.beam_scores).to(dev), torch.from_numpy(si.logp).to(dev)
    got = [x.cpu().numpy() for x in select_noalloc(bs, lp, n_beams)]
    ref = [x.cpu().numpy() for x in onela.beam_select(bs, lp, n_beams)]
    torch.cuda.synchronize()
    for name, a, b in zip(("parent", "token", "score"), got, ref):
        assert np.array_equal(a.view(np.uint32), b.view(np.uint32)), name
    if R * n_prev * n_cand <= 40000:
        want = oracle.beam_select(si.beam_scores, si.logp, n_beams)
        assert np.array_equal(got[0], want[0]) and np.array_equal(got[1], want[1])


def test_noalloc_matches_caller_scratch_entry_point():
    # the full 32 x 512 x 256 -> 512 shape (4 MiB of scratch), then smaller ones: one chunk pass, two chunk
    # passes, and one that needs no scratch at all
    check_pair(32, 512, 256, 512, seed=0)
    check_pair(3, 100, 300, 512, seed=1)
    check_pair(4, 512, 256, 2048, seed=2)
    check_pair(2, 64, 64, 100, seed=3)


def test_noalloc_rejects_oversized_selection():
    dev = gu.device()
    R, n_prev, n_cand, n_beams = 32, 512, 256, 2048  # 16 MiB of scratch
    assert onela.onela_beam_select_scratch(R, n_prev, n_cand, n_beams) > 8 << 20
    bs = torch.zeros((R, n_prev), device=dev)
    lp = torch.zeros((R, n_prev, n_cand), device=dev)
    with pytest.raises(onela.OnelaError) as e:
        select_noalloc(bs, lp, n_beams)
    assert e.value.status == onela.ONELA_ERR_CAPACITY
