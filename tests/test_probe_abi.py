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
