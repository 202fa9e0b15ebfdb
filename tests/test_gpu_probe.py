"""The bench's bandwidth probes (libonela_probe.so) move the bytes they claim: the streaming modes write what they
read, and the step-traffic probe writes every key and alpha record of the shape it is given."""

import ctypes
import os

import numpy as np
import pytest
import torch

from tests import gpu_util as gu

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "linear_attention_beam_amd", "lib", "libonela_probe.so")


def probe_lib():
    if not os.path.exists(LIB):
        raise RuntimeError(f"{LIB} is missing: build it first")
    lib = ctypes.CDLL(LIB)
    lib.onela_probe_stream.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int,
                                       ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p]
    lib.onela_probe_stream.restype = ctypes.c_int
    lib.onela_probe_step_traffic.argtypes = [ctypes.c_void_p] * 10 + [ctypes.c_int] * 5 + [ctypes.c_void_p]
    lib.onela_probe_step_traffic.restype = ctypes.c_int
    return lib


@pytest.mark.parametrize("grid", [0, 7])
def test_stream_modes(grid):
    lib, dev = probe_lib(), gu.device()
    n = 1000                                     # 16-byte elements per stream (not a multiple of 256)
    gu.log(f"probe stream modes, n={n}, grid={grid}")
    src = torch.randn(2 * n * 4, device=dev)
    dst = torch.full((3 * n * 4,), -7.0, device=dev)
    sink = torch.zeros(max(grid, 1) * 256, device=dev)
    s = torch.cuda.current_stream().cuda_stream
    assert lib.onela_probe_stream(src.data_ptr(), dst.data_ptr(), n, 1, sink.data_ptr(), grid, s) == 0
    torch.cuda.synchronize()
    a, b = src[:4 * n], src[4 * n:]
    assert torch.equal(dst[:4 * n], a) and torch.equal(dst[4 * n:8 * n], b) and torch.equal(dst[8 * n:], a + b)
    dst.fill_(-7.0)
    assert lib.onela_probe_stream(src.data_ptr(), dst.data_ptr(), n, 2, sink.data_ptr(), grid, s) == 0
    torch.cuda.synchronize()
    assert torch.equal(dst[:4 * n], a) and bool((dst[4 * n:] == -7.0).all())
    assert lib.onela_probe_stream(src.data_ptr(), dst.data_ptr(), n, 3, sink.data_ptr(), grid, s) == 0
    torch.cuda.synchronize()
    assert torch.equal(dst[:4 * n], torch.tensor([1.0, 2.0, 3.0, 4.0], device=dev).repeat(n))
    if grid:  # the grid-stride read leaves one partial sum per thread; together they sum the whole source
        assert lib.onela_probe_stream(src.data_ptr(), dst.data_ptr(), n, 0, sink.data_ptr(), grid, s) == 0
        torch.cuda.synchronize()
        assert abs(float(sink.double().sum()) - float(src.double().sum())) < 1e-2


@pytest.mark.parametrize("d_v", [128, 256, 96])
def test_step_traffic_writes_every_record(d_v):
    lib, dev = probe_lib(), gu.device()
    R, B, H, slots = 2, 96, 3, 200
    gu.log(f"step-traffic probe R={R} B={B} H={H} d_v={d_v} slots={slots}")
    g = torch.Generator(device="cpu").manual_seed(5)
    k = torch.randn((R, B, H, 128), generator=g).to(torch.bfloat16).to(dev)
    q = torch.randn((R, B, H, 128), generator=g).to(torch.bfloat16).to(dev)
    v = torch.randn((R, B, H, d_v), generator=g).to(torch.bfloat16).to(dev)
    alpha = torch.rand((R, B, H), generator=g).to(dev)
    beta = torch.rand((R, B, H), generator=g).to(dev)
    sctx = torch.randn((R * H, 128, d_v), generator=g).to(dev)
    o = torch.full((R, B, H, d_v), float("nan"), device=dev)
    u = torch.full((R * H, slots, d_v), float("nan"), device=dev)
    rk = torch.zeros((R * H, slots, 128), dtype=torch.bfloat16, device=dev)
    ra = torch.full((R * H, slots), -1.0, device=dev)
    args = [t.data_ptr() for t in (k, q, v, alpha, beta, sctx, o, u, rk, ra)]
    s = torch.cuda.current_stream().cuda_stream
    assert lib.onela_probe_step_traffic(*args, R, B, H, d_v, slots, s) == 0
    torch.cuda.synchronize()
    # the key and alpha records of slot b are the inputs of beam b; slots past B are untouched
    want_k = k.permute(0, 2, 1, 3).reshape(R * H, B, 128)
    assert torch.equal(rk[:, :B].view(torch.int16), want_k.contiguous().view(torch.int16))
    assert bool((rk[:, B:].view(torch.int16) == 0).all())
    want_a = (alpha + beta).permute(0, 2, 1).reshape(R * H, B)
    assert torch.equal(ra[:, :B], want_a) and bool((ra[:, B:] == -1.0).all())
    # every o row and every u row of slots < B is written (the values are folded bits, never NaN)
    assert not bool(torch.isnan(o).any()) and not bool(torch.isnan(u[:, :B]).any())
    assert bool(torch.isnan(u[:, B:]).all())
    # a bad shape is refused without a launch
    assert lib.onela_probe_step_traffic(*args, R, B + 1, H, d_v, slots, s) == 1
