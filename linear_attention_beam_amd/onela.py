"""ctypes binding of libonela (include/onela.h): the same entry points, argument marshalling only.

Every step of the decode runs in the HIP library; nothing here computes.  When the library has not been
built (``python -m linear_attention_beam_amd.build``), loading it raises instead of falling back.

``OneLA`` wraps a handle for PyTorch callers: it allocates the workspace as a torch tensor on the GPU,
checks tensor shapes and dtypes, and passes data pointers and the current HIP stream.
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "lib", "libonela.so")

ONELA_OK = 0
ONELA_ERR_INVALID_ARG = 1
ONELA_ERR_STATE = 2
ONELA_ERR_CAPACITY = 3
ONELA_ERR_DEVICE = 4
ONELA_ERR_BAD_PARENT = 5
ONELA_ERR_UNSUPPORTED = 6

ONELA_F32 = 0
ONELA_BF16 = 1
ONELA_MODE_REPLAY = 0
ONELA_MODE_FULLSTATE = 1
ONELA_FLAG_FORCE_GENERIC = 1
ONELA_FLAG_MATERIALIZE = 2


class onela_config(ctypes.Structure):
    _fields_ = [(name, ctypes.c_int32) for name in (
        "num_requests", "num_heads", "d_k", "d_v", "max_beams", "max_steps", "qkv_dtype", "mode", "flags",
        "tile_beams")]


class onela_view(ctypes.Structure):
    _fields_ = [("t", ctypes.c_int32), ("n_beams", ctypes.c_int32), ("slots", ctypes.c_int32),
                ("fused", ctypes.c_int32), ("rec_k", ctypes.c_void_p), ("rec_u", ctypes.c_void_p),
                ("rec_alpha", ctypes.c_void_p), ("chains", ctypes.c_void_p), ("sctx_t", ctypes.c_void_p),
                ("fullstate", ctypes.c_void_p)]


class OnelaError(RuntimeError):
    def __init__(self, status: int, where: str, message: str):
        super().__init__(f"{where}: {status_name(status)}: {message}")
        self.status = status


_lib = None
_P = ctypes.c_void_p
_SIGNATURES = {
    "onela_workspace_size": [ctypes.POINTER(onela_config), ctypes.POINTER(ctypes.c_size_t)],
    "onela_create": [ctypes.POINTER(onela_config), _P, ctypes.c_size_t, ctypes.POINTER(_P)],
    "onela_destroy": [_P],
    "onela_set_context": [_P, _P, _P],
    "onela_prefill": [_P, ctypes.c_int32, _P, _P, _P, _P, _P, _P],
    "onela_step": [_P, ctypes.c_int32, _P, _P, _P, _P, _P, _P, _P, _P],
    "onela_reset": [_P, _P],
    "onela_get_status": [_P, _P],
    "onela_get_view": [_P, ctypes.POINTER(onela_view)],
    "onela_beam_select_scratch": [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                  ctypes.POINTER(ctypes.c_size_t)],
    "onela_beam_select": [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, _P, _P, _P, _P, _P, _P,
                          ctypes.c_size_t, _P],
    "onela_beam_select_noalloc": [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, _P, _P, _P, _P,
                                  _P, _P],
    "onela_status_string": [ctypes.c_int],
    "onela_last_error": [],
}


def lib() -> ctypes.CDLL:
    """Load libonela.so once; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m linear_attention_beam_amd.build`")
        handle = ctypes.CDLL(LIB_PATH)
        for name, args in _SIGNATURES.items():
            fn = getattr(handle, name)
            fn.argtypes = args
            fn.restype = ctypes.c_char_p if name in ("onela_status_string", "onela_last_error") else ctypes.c_int
        _lib = handle
    return _lib


def status_name(status: int) -> str:
    return lib().onela_status_string(status).decode()


def _check(status: int, where: str) -> None:
    if status != ONELA_OK:
        raise OnelaError(status, where, lib().onela_last_error().decode())


# ---------------------------------------------------------------------------------------------------
# The C entry points, one to one (pointers and streams are plain integers)
# ---------------------------------------------------------------------------------------------------

def onela_workspace_size(cfg: onela_config) -> int:
    n = ctypes.c_size_t(0)
    _check(lib().onela_workspace_size(ctypes.byref(cfg), ctypes.byref(n)), "onela_workspace_size")
    return n.value


def onela_create(cfg: onela_config, workspace_ptr: int, workspace_bytes: int) -> int:
    h = _P()
    _check(lib().onela_create(ctypes.byref(cfg), workspace_ptr, workspace_bytes, ctypes.byref(h)), "onela_create")
    return h.value


def onela_destroy(h: int) -> None:
    _check(lib().onela_destroy(h), "onela_destroy")


def onela_set_context(h: int, sctx_ptr: int, stream: int) -> None:
    _check(lib().onela_set_context(h, sctx_ptr, stream), "onela_set_context")


def onela_prefill(h: int, n_tokens: int, k_ptr: int, v_ptr: int, alpha_ptr: int, beta_ptr: int,
                  sctx_out_ptr: Optional[int], stream: int) -> None:
    _check(lib().onela_prefill(h, n_tokens, k_ptr, v_ptr, alpha_ptr, beta_ptr, sctx_out_ptr, stream),
           "onela_prefill")


def onela_step(h: int, n_beams: int, q_ptr: int, k_ptr: int, v_ptr: int, alpha_ptr: int, beta_ptr: int,
               parent_ptr: int, o_ptr: int, stream: int) -> None:
    _check(lib().onela_step(h, n_beams, q_ptr, k_ptr, v_ptr, alpha_ptr, beta_ptr, parent_ptr, o_ptr, stream),
           "onela_step")


def onela_reset(h: int, stream: int) -> None:
    _check(lib().onela_reset(h, stream), "onela_reset")


def onela_get_status(h: int, stream: int) -> int:
    """Waits for the stream; returns ONELA_OK or ONELA_ERR_BAD_PARENT (raises on other failures)."""
    s = lib().onela_get_status(h, stream)
    if s not in (ONELA_OK, ONELA_ERR_BAD_PARENT):
        _check(s, "onela_get_status")
    return s


def onela_get_view(h: int) -> onela_view:
    v = onela_view()
    _check(lib().onela_get_view(h, ctypes.byref(v)), "onela_get_view")
    return v


def onela_beam_select_scratch(R: int, n_prev: int, n_cand: int, n_beams: int) -> int:
    n = ctypes.c_size_t(0)
    _check(lib().onela_beam_select_scratch(R, n_prev, n_cand, n_beams, ctypes.byref(n)), "onela_beam_select_scratch")
    return n.value


def onela_beam_select(R: int, n_prev: int, n_cand: int, n_beams: int, beam_scores_ptr: int, logp_ptr: int,
                      parent_ptr: int, token_ptr: int, scores_ptr: int, scratch_ptr: Optional[int], scratch_bytes: int,
                      stream: int) -> None:
    _check(lib().onela_beam_select(R, n_prev, n_cand, n_beams, beam_scores_ptr, logp_ptr, parent_ptr, token_ptr,
                                   scores_ptr, scratch_ptr, scratch_bytes, stream), "onela_beam_select")


def onela_beam_select_noalloc(R: int, n_prev: int, n_cand: int, n_beams: int, beam_scores_ptr: int, logp_ptr: int,
                              parent_ptr: int, token_ptr: int, scores_ptr: int, stream: int) -> None:
    _check(lib().onela_beam_select_noalloc(R, n_prev, n_cand, n_beams, beam_scores_ptr, logp_ptr, parent_ptr,
                                           token_ptr, scores_ptr, stream), "onela_beam_select_noalloc")


# ---------------------------------------------------------------------------------------------------
# PyTorch convenience wrappers
# ---------------------------------------------------------------------------------------------------

def beam_select(beam_scores, logp, n_beams: int, scratch=None):
    """Top n_beams of beam_scores[r, b] + logp[r, b, c] per request, best first (see onela_beam_select).

    beam_scores: [R, n_prev] float32, logp: [R, n_prev, n_cand] float32, both contiguous on one GPU.
    Returns (parent int32 [R, n_beams], token int32 [R, n_beams], scores float32 [R, n_beams]).  ``scratch``
    (a uint8 device tensor of at least onela_beam_select_scratch bytes) is allocated here when not given.
    """
    import torch
    R, n_prev, n_cand = (int(x) for x in logp.shape)
    dev = logp.device
    for name, x, shape in (("beam_scores", beam_scores, (R, n_prev)), ("logp", logp, (R, n_prev, n_cand))):
        if x.device != dev or x.dtype != torch.float32 or tuple(x.shape) != shape or not x.is_contiguous():
            raise ValueError(f"{name}: expected contiguous float32 {shape} on {dev}, got {x.dtype} "
                             f"{tuple(x.shape)} on {x.device}")
    need = onela_beam_select_scratch(R, n_prev, n_cand, n_beams)
    if scratch is None and need:
        scratch = torch.empty(need, dtype=torch.uint8, device=dev)
    parent = torch.empty((R, n_beams), dtype=torch.int32, device=dev)
    token = torch.empty((R, n_beams), dtype=torch.int32, device=dev)
    scores = torch.empty((R, n_beams), dtype=torch.float32, device=dev)
    with torch.cuda.device(dev):
        onela_beam_select(R, n_prev, n_cand, n_beams, beam_scores.data_ptr(), logp.data_ptr(), parent.data_ptr(),
                          token.data_ptr(), scores.data_ptr(), scratch.data_ptr() if need else None,
                          scratch.numel() if need else 0, torch.cuda.current_stream(dev).cuda_stream)
    return parent, token, scores


class OneLA:
    """A decode context on one GPU: R requests x H heads, up to max_beams beams and max_steps steps.

    qkv_dtype: "bf16" or "f32"; mode: "replay" (shared state + records) or "fullstate" (comparison).
    materialize: in replay mode, rebuild every beam's dense parent state each step (comparison path).
    """

    def __init__(self, R: int, H: int, d_k: int, d_v: int, max_beams: int, max_steps: int,
                 qkv_dtype: str = "bf16", mode: str = "replay", force_generic: bool = False,
                 tile_beams: int = 0, device=None, materialize: bool = False):
        import torch
        self._torch = torch
        self.device = torch.device("cuda", torch.cuda.current_device()) if device is None else torch.device(device)
        self.cfg = onela_config(R, H, d_k, d_v, max_beams, max_steps,
                                ONELA_BF16 if qkv_dtype == "bf16" else ONELA_F32,
                                ONELA_MODE_FULLSTATE if mode == "fullstate" else ONELA_MODE_REPLAY,
                                (ONELA_FLAG_FORCE_GENERIC if force_generic else 0)
                                | (ONELA_FLAG_MATERIALIZE if materialize else 0), tile_beams)
        if qkv_dtype not in ("bf16", "f32") or mode not in ("replay", "fullstate"):
            raise ValueError(f"qkv_dtype {qkv_dtype!r} / mode {mode!r}")
        self.qkv_torch_dtype = torch.bfloat16 if qkv_dtype == "bf16" else torch.float32
        self.nbytes = onela_workspace_size(self.cfg)
        with torch.cuda.device(self.device):
            self.workspace = torch.empty(self.nbytes, dtype=torch.uint8, device=self.device)
            if self.workspace.data_ptr() % 256:
                raise RuntimeError("workspace allocation is not 256-byte aligned")
            self.handle = onela_create(self.cfg, self.workspace.data_ptr(), self.nbytes)
        self.n_beams = 1

    # -- helpers ------------------------------------------------------------------------------------
    def _stream(self) -> int:
        return self._torch.cuda.current_stream(self.device).cuda_stream

    def _tensor(self, x, shape, dtype, name):
        if x.device != self.device or x.dtype != dtype or tuple(x.shape) != tuple(shape) or not x.is_contiguous():
            raise ValueError(f"{name}: expected contiguous {dtype} {tuple(shape)} on {self.device}, got "
                             f"{x.dtype} {tuple(x.shape)} on {x.device} (contiguous={x.is_contiguous()})")
        return x.data_ptr()

    # -- API ------------------------------------------------------------------------------------------
    def set_context(self, sctx) -> None:
        c = self.cfg
        ptr = self._tensor(sctx, (c.num_requests, c.num_heads, c.d_v, c.d_k), self._torch.float32, "sctx")
        with self._torch.cuda.device(self.device):
            onela_set_context(self.handle, ptr, self._stream())
        self.n_beams = 1

    def prefill(self, k, v, alpha, beta, sctx_out=None) -> None:
        c = self.cfg
        f32 = self._torch.float32
        N = k.shape[1]
        ptrs = [self._tensor(k, (c.num_requests, N, c.num_heads, c.d_k), f32, "k"),
                self._tensor(v, (c.num_requests, N, c.num_heads, c.d_v), f32, "v"),
                self._tensor(alpha, (c.num_requests, N, c.num_heads), f32, "alpha"),
                self._tensor(beta, (c.num_requests, N, c.num_heads), f32, "beta")]
        out = None if sctx_out is None else self._tensor(sctx_out, (c.num_requests, c.num_heads, c.d_v, c.d_k), f32,
                                                         "sctx_out")
        with self._torch.cuda.device(self.device):
            onela_prefill(self.handle, N, *ptrs, out, self._stream())
        self.n_beams = 1

    def step(self, q, k, v, alpha, beta, parent, out=None):
        c = self.cfg
        n = q.shape[1]
        dt, f32 = self.qkv_torch_dtype, self._torch.float32
        R, H = c.num_requests, c.num_heads
        if out is None:
            out = self._torch.empty((R, n, H, c.d_v), dtype=f32, device=self.device)
        ptrs = [self._tensor(q, (R, n, H, c.d_k), dt, "q"), self._tensor(k, (R, n, H, c.d_k), dt, "k"),
                self._tensor(v, (R, n, H, c.d_v), dt, "v"), self._tensor(alpha, (R, n, H), f32, "alpha"),
                self._tensor(beta, (R, n, H), f32, "beta"),
                self._tensor(parent, (R, n), self._torch.int32, "parent"),
                self._tensor(out, (R, n, H, c.d_v), f32, "out")]
        with self._torch.cuda.device(self.device):
            onela_step(self.handle, n, *ptrs, self._stream())
        self.n_beams = n
        return out

    def reset(self) -> None:
        with self._torch.cuda.device(self.device):
            onela_reset(self.handle, self._stream())
        self.n_beams = 1

    def status(self) -> int:
        with self._torch.cuda.device(self.device):
            return onela_get_status(self.handle, self._stream())

    def view(self) -> dict:
        """Torch views of the decode state inside the workspace (read-only by convention)."""
        torch = self._torch
        v = onela_get_view(self.handle)
        c = self.cfg
        R, H, B, L, dk, dv = c.num_requests, c.num_heads, c.max_beams, c.max_steps, c.d_k, c.d_v
        base = self.workspace.data_ptr()

        def sub(ptr, count, dtype, shape):
            if not ptr:
                return None
            off = ptr - base
            size = torch.empty((), dtype=dtype).element_size()
            return self.workspace[off: off + count * size].view(dtype).reshape(shape)

        slots = v.slots
        return {
            "t": v.t, "n_beams": v.n_beams, "slots": slots, "fused": bool(v.fused),
            "rec_k": sub(v.rec_k, R * H * slots * dk, self.qkv_torch_dtype, (R, H, slots, dk)),
            "rec_u": sub(v.rec_u, R * H * slots * dv, torch.float32, (R, H, slots, dv)),
            "rec_alpha": sub(v.rec_alpha, R * H * slots, torch.float32, (R, H, slots)),
            "chains": sub(v.chains, L * R * B * L, torch.int32, (L, R, B, L)),
            "sctx_t": sub(v.sctx_t, R * H * dk * dv, torch.float32, (R, H, dk, dv)),
            "fullstate": sub(v.fullstate, 2 * R * H * B * dk * dv, torch.float32, (2, R, H, B, dk, dv)),
        }

    def close(self) -> None:
        if getattr(self, "handle", None):
            onela_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:  # noqa: BLE001 - interpreter shutdown
            pass
