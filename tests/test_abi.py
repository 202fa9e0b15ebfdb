"""The C ABI without a GPU: the library loads, exports every function include/onela.h declares, and
checks configurations on the host (onela_workspace_size touches no device)."""

import ctypes
import os
import re

import pytest

from linear_attention_beam_amd import onela

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "onela.h")

pytestmark = pytest.mark.skipif(not os.path.exists(onela.LIB_PATH), reason="libonela.so not built")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(onela_\w+)\s*\(", text, flags=re.M)))


def test_every_declared_symbol_is_exported():
    names = declared_functions()
    assert len(names) >= 11, names
    lib = ctypes.CDLL(onela.LIB_PATH)
    for name in names:
        assert hasattr(lib, name), f"{name} declared in onela.h but not exported"
    assert set(names) == set(onela._SIGNATURES), "binding and header disagree"


def cfg(**kw):
    base = dict(num_requests=2, num_heads=3, d_k=128, d_v=128, max_beams=64, max_steps=4,
                qkv_dtype=onela.ONELA_BF16, mode=onela.ONELA_MODE_REPLAY, flags=0, tile_beams=0)
    base.update(kw)
    return onela.onela_config(**base)


def expected_bytes(c):
    """Workspace layout documented in the header, regions rounded up to 256 bytes."""
    up = lambda x: (x + 255) // 256 * 256  # noqa: E731
    R, H, dk, dv, B, L = c.num_requests, c.num_heads, c.d_k, c.d_v, c.max_beams, c.max_steps
    s_in = 2 if c.qkv_dtype == onela.ONELA_BF16 else 4
    fused = (c.mode == onela.ONELA_MODE_REPLAY and c.qkv_dtype == onela.ONELA_BF16 and not c.flags
             and dk in (64, 128, 256) and dv % 32 == 0)
    total = 256 + up(R * H * dk * dv * 4) + up(R * H * dk * dv * 4 if fused else 0) + up(L * R * B * L * 4)
    a16 = lambda x: (x + 15) // 16 * 16  # noqa: E731
    # per (request, tile of 16 or 32 beams) plans: nd and up to 64 distinct slots, the tile's beams, one byte per
    # (beam, chain position) with the positions of a beam padded to a multiple of 8; the larger of the two tile
    # sizes, then the processing order rank[R][B]
    L8 = -(-L // 8) * 8
    plan = up(max(R * (-(-B // nb)) * (a16(4 + 4 * 64) + 4 * nb + a16(nb * L8)) for nb in (16, 32))) + R * B * 4
    total += up(plan if fused else 0)
    if c.mode == onela.ONELA_MODE_REPLAY:
        slots = B * L
        u_elems = slots * dv
        total += up(R * H * slots * dk * s_in) + up(R * H * u_elems * 4) + up(R * H * slots * 4)
    else:
        total += up(2 * R * H * B * dk * dv * 4)
    return total


@pytest.mark.parametrize("kw", [
    {}, dict(d_v=256), dict(qkv_dtype=onela.ONELA_F32, d_k=16, d_v=16), dict(mode=onela.ONELA_MODE_FULLSTATE),
    dict(flags=onela.ONELA_FLAG_FORCE_GENERIC), dict(flags=onela.ONELA_FLAG_MATERIALIZE), dict(d_k=64, d_v=100),
    dict(max_steps=64, max_beams=1), dict(max_steps=3, max_beams=5, d_v=7), dict(max_steps=3, max_beams=5, d_v=96),
])
def test_workspace_size(kw):
    c = cfg(**kw)
    assert onela.onela_workspace_size(c) == expected_bytes(c)


@pytest.mark.parametrize("kw", [
    dict(num_requests=0), dict(num_heads=-1), dict(d_k=0), dict(d_v=257), dict(max_beams=0),
    dict(max_steps=0), dict(max_steps=65), dict(qkv_dtype=7), dict(mode=2), dict(flags=4), dict(tile_beams=48), dict(tile_beams=64),
])
def test_bad_config_is_rejected(kw):
    with pytest.raises(onela.OnelaError) as e:
        onela.onela_workspace_size(cfg(**kw))
    assert e.value.status == onela.ONELA_ERR_INVALID_ARG


def test_status_strings():
    for code in range(7):
        assert onela.status_name(code).startswith("ONELA_")
    assert onela.status_name(99) == "unknown onela_status"


@pytest.mark.parametrize("R,n_prev,n_cand,n_beams", [(32, 512, 256, 512), (1, 1, 5, 3), (2, 64, 64, 2048),
                                                     (3, 100, 300, 700), (1, 128, 128, 100)])
def test_beam_select_scratch(R, n_prev, n_cand, n_beams):
    """Two buffers of the keys that survive the first reduce pass over 8192-key chunks; none when a request has
    at most 8192 candidates (one workgroup selects them directly)."""
    n = n_prev * n_cand
    expect = 0 if n <= 8192 else 2 * R * ((n + 8191) // 8192) * n_beams * 8
    assert onela.onela_beam_select_scratch(R, n_prev, n_cand, n_beams) == expect


@pytest.mark.parametrize("args,status", [
    ((0, 4, 8, 1), onela.ONELA_ERR_INVALID_ARG), ((1, 4, 8, 33), onela.ONELA_ERR_INVALID_ARG),
    ((1, 4, 8, 0), onela.ONELA_ERR_INVALID_ARG), ((1, 65536, 65536, 8), onela.ONELA_ERR_INVALID_ARG),
    ((1, 64, 64, 2049), onela.ONELA_ERR_UNSUPPORTED),
])
def test_beam_select_bad_args(args, status):
    with pytest.raises(onela.OnelaError) as e:
        onela.onela_beam_select_scratch(*args)
    assert e.value.status == status
