"""libonela_probe.so (the bench's bandwidth probe) loads without a GPU and exports what include/onela_probe.h
declares; bad arguments are refused on the host (nothing is enqueued for them)."""

import ctypes
import os

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "linear_attention_beam_amd", "lib", "libonela_probe.so")


@pytest.mark.skipif(not os.path.exists(LIB), reason="libonela_probe.so not built")
def test_probe_exports_and_argument_checks():
    lib = ctypes.CDLL(LIB)
    fn = lib.onela_probe_stream
    fn.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int, ctypes.c_void_p, ctypes.c_int,
                   ctypes.c_void_p]
    fn.restype = ctypes.c_int
    assert fn(None, None, 16, 7, None, 1, None) == 1      # unknown mode
    assert fn(None, None, 0, 2, None, 1, None) == 1       # empty
    assert fn(None, None, 16, 2, None, -1, None) == 1     # negative grid
    assert fn(None, None, 16, 1, None, 1, None) == 1      # the mix needs both buffers
    assert fn(None, None, 16, 0, None, 1, None) == 1      # read needs src and the sink


@pytest.mark.skipif(not os.path.exists(LIB), reason="libonela_probe.so not built")
def test_step_traffic_probe_argument_checks():
    lib = ctypes.CDLL(LIB)
    fn = lib.onela_probe_step_traffic
    fn.argtypes = [ctypes.c_void_p] * 10 + [ctypes.c_int] * 5 + [ctypes.c_void_p]
    fn.restype = ctypes.c_int
    buf = ctypes.create_string_buffer(64)
    p = [ctypes.addressof(buf)] * 10
    assert fn(*([None] + p[1:]), 1, 32, 1, 128, 32, None) == 1   # a missing buffer
    assert fn(*p, 1, 48, 1, 128, 64, None) == 1                    # B not a multiple of 32
    assert fn(*p, 1, 32, 1, 100, 32, None) == 1                    # d_v not a multiple of 32
    assert fn(*p, 1, 32, 1, 512, 32, None) == 1                    # d_v above 256
    assert fn(*p, 1, 32, 1, 128, 16, None) == 1                    # fewer slots than beams
    assert fn(*p, 0, 32, 1, 128, 32, None) == 1                    # no requests
