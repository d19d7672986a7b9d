"""ctypes binding of libfa_relayout.so (argument marshalling only).

Every function here forwards to the C entry point of the same name declared in
include/fa_relayout.h; all arithmetic runs in the library's HIP kernels.  There
is no fallback: if the library is missing or fails to load, the call raises.
torch supplies device memory and the current HIP stream.
"""
from __future__ import annotations

import ctypes
import math
import os
import threading
from typing import Optional

import torch  # loads torch's HIP runtime first, which the library then shares

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libfa_relayout.so")

FA_OK = 0
STATUS_NAMES = {0: "FA_OK", -1: "FA_EINVAL", -2: "FA_EDIV", -3: "FA_EUNSUPPORTED",
                -4: "FA_EALIGN", -5: "FA_ERANGE", -6: "FA_ELAUNCH", -7: "FA_EDEVICE",
                -8: "FA_EEXEC"}
MASK_TILE = 128

_lib = None
_lock = threading.Lock()

_P = ctypes.c_void_p
_I = ctypes.c_int
_F = ctypes.c_float
SIGNATURES = {
    "attn_fwd_relayout_async": [_P, _P, _P, _P, _I, _I, _I, _I, _I, _F, _P, _P],
    "attn_fwd_relayout": [_P, _P, _P, _P, _I, _I, _I, _I, _I, _F, _P],
    "attn_fwd_slab_to_slab_async": [_P, _P, _P, _P, _I, _I, _I, _I, _I, _F, _P, _P],
    "attn_fwd_slab_to_slab": [_P, _P, _P, _P, _I, _I, _I, _I, _I, _F, _P],
    "attn_fwd_slab_to_slab_ws_async": [_P, _P, _P, _P, _I, _I, _I, _I, _I, _F, _P, _P,
                                       ctypes.c_int64, _P],
    "attn_fwd_plain_async": [_P, _P, _P, _P, _I, _I, _I, _I, _F, _P, _P],
    "attn_fwd_plain": [_P, _P, _P, _P, _I, _I, _I, _I, _F, _P],
    "relayout_to_slabs_async": [_P, _P, _I, _I, _I, _I, _I, _P],
    "relayout_to_slabs": [_P, _P, _I, _I, _I, _I, _I],
    "burst_gap_run_async": [_P, _P, _I, _I, _I, _I, _I, _I, _P],
    "attn_fwd_relayout_instrumented_async": [_P, _P, _P, _P, _I, _I, _I, _I, _I, _F, _P, _I, _P,
                                             ctypes.c_int64, _P, _P],
    "attn_instrumented_stamp_words": [_I, _I, _I],
    "attn_fwd_relayout_ws_async": [_P, _P, _P, _P, _I, _I, _I, _I, _I, _F, _P, _P,
                                   ctypes.c_int64, _P],
    "attn_fwd_plain_ws_async": [_P, _P, _P, _P, _I, _I, _I, _I, _F, _P, _P, ctypes.c_int64, _P],
    "attn_fwd_workspace_bytes": [_I, _I, _I, _I],
    "attn_fwd_relayout_noalloc_async": [_P, _P, _P, _P, _I, _I, _I, _I, _I, _F, _P, _P],
    "attn_status_string": [_I],
    "attn_abi_version": [],
}


RESTYPES = {"attn_status_string": ctypes.c_char_p,
            "attn_instrumented_stamp_words": ctypes.c_int64,
            "attn_fwd_workspace_bytes": ctypes.c_int64}


class FaError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        self.name = STATUS_NAMES.get(status, str(status))
        super().__init__(f"{where}: {self.name} ({attn_status_string(status)})")


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load the HIP library (once); raises if it is not built."""
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(path):
                raise RuntimeError(
                    f"{path} is missing: build it with "
                    "`python -m flashattention_output_re_amd.build`")
            lib = ctypes.CDLL(path)
            for name, args in SIGNATURES.items():
                fn = getattr(lib, name)
                fn.argtypes = args
                fn.restype = RESTYPES.get(name, ctypes.c_int)
            _lib = lib
        return _lib


def attn_status_string(status: int) -> str:
    return load_library().attn_status_string(int(status)).decode()


def attn_abi_version() -> int:
    return load_library().attn_abi_version()


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    if isinstance(stream, torch.cuda.Stream):
        stream = stream.cuda_stream
    return ctypes.c_void_p(int(stream))


def _check_tensor(name: str, t: torch.Tensor, shape: tuple):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != torch.bfloat16:
        raise TypeError(f"{name} must be bfloat16, got {t.dtype}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on a HIP device")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")


def _check_mask(mask: Optional[torch.Tensor], H: int, S: int):
    if mask is None:
        return
    nT = (S + MASK_TILE - 1) // MASK_TILE
    shape = (H, nT, (nT + 63) // 64)
    if mask.dtype not in (torch.int64, torch.uint64):
        raise TypeError("mask must hold 64-bit words")
    if not mask.is_cuda or not mask.is_contiguous() or tuple(mask.shape) != shape:
        raise ValueError(f"mask must be a contiguous device tensor of shape {shape}")


def _raise(status: int, where: str):
    if status != FA_OK:
        raise FaError(status, where)


def attn_fwd_relayout_async(q, k, v, out_slabs, B, H, S, D, P, scale, mask=None, stream=None):
    """Enqueue fused attention + slab store; out_slabs is bf16 [P][B][S/P][H][D]."""
    if P > 0 and S % P == 0:
        for n, t in (("q", q), ("k", k), ("v", v)):
            _check_tensor(n, t, (B, H, S, D))
        _check_tensor("out_slabs", out_slabs, (P, B, S // P, H, D))
        _check_mask(mask, H, S)
    st = load_library().attn_fwd_relayout_async(
        _ptr(q), _ptr(k), _ptr(v), _ptr(out_slabs), B, H, S, D, P, float(scale), _ptr(mask),
        _stream(stream))
    _raise(st, "attn_fwd_relayout_async")


def attn_fwd_relayout(q, k, v, out_slabs, B, H, S, D, P, scale, mask=None):
    """Blocking variant on the null stream."""
    if P > 0 and S % P == 0:
        for n, t in (("q", q), ("k", k), ("v", v)):
            _check_tensor(n, t, (B, H, S, D))
        _check_tensor("out_slabs", out_slabs, (P, B, S // P, H, D))
        _check_mask(mask, H, S)
    st = load_library().attn_fwd_relayout(
        _ptr(q), _ptr(k), _ptr(v), _ptr(out_slabs), B, H, S, D, P, float(scale), _ptr(mask))
    _raise(st, "attn_fwd_relayout")


def attn_fwd_slab_to_slab_async(q_slabs, k_slabs, v_slabs, out_slabs, B, H, S, D, P, scale,
                                mask=None, stream=None):
    """Enqueue the whole Ulysses step: q, k, v and the output are all bf16
    [P][B][S/P][H][D] (sequence-sharded slabs)."""
    if P > 0 and S % P == 0:
        for n, t in (("q_slabs", q_slabs), ("k_slabs", k_slabs), ("v_slabs", v_slabs),
                     ("out_slabs", out_slabs)):
            _check_tensor(n, t, (P, B, S // P, H, D))
        _check_mask(mask, H, S)
    st = load_library().attn_fwd_slab_to_slab_async(
        _ptr(q_slabs), _ptr(k_slabs), _ptr(v_slabs), _ptr(out_slabs), B, H, S, D, P, float(scale),
        _ptr(mask), _stream(stream))
    _raise(st, "attn_fwd_slab_to_slab_async")


def attn_fwd_slab_to_slab_ws_async(q_slabs, k_slabs, v_slabs, out_slabs, B, H, S, D, P, scale,
                                   mask=None, workspace=None, stream=None):
    """attn_fwd_slab_to_slab_async with the last round spread over every
    workgroup; workspace as for attn_fwd_relayout_ws_async (allocated here
    when None)."""
    if P > 0 and S % P == 0:
        for n, t in (("q_slabs", q_slabs), ("k_slabs", k_slabs), ("v_slabs", v_slabs),
                     ("out_slabs", out_slabs)):
            _check_tensor(n, t, (P, B, S // P, H, D))
        _check_mask(mask, H, S)
    ws = _workspace(workspace, B, H, S, D, q_slabs.device)
    st = load_library().attn_fwd_slab_to_slab_ws_async(
        _ptr(q_slabs), _ptr(k_slabs), _ptr(v_slabs), _ptr(out_slabs), B, H, S, D, P, float(scale),
        _ptr(mask), _ptr(ws), _nbytes(ws), _stream(stream))
    _raise(st, "attn_fwd_slab_to_slab_ws_async")
    return ws


def attn_fwd_slab_to_slab(q_slabs, k_slabs, v_slabs, out_slabs, B, H, S, D, P, scale, mask=None):
    """Blocking variant on the null stream."""
    if P > 0 and S % P == 0:
        for n, t in (("q_slabs", q_slabs), ("k_slabs", k_slabs), ("v_slabs", v_slabs),
                     ("out_slabs", out_slabs)):
            _check_tensor(n, t, (P, B, S // P, H, D))
        _check_mask(mask, H, S)
    st = load_library().attn_fwd_slab_to_slab(
        _ptr(q_slabs), _ptr(k_slabs), _ptr(v_slabs), _ptr(out_slabs), B, H, S, D, P, float(scale),
        _ptr(mask))
    _raise(st, "attn_fwd_slab_to_slab")


def attn_fwd_plain_async(q, k, v, out, B, H, S, D, scale, mask=None, stream=None):
    """Enqueue the same attention writing the plain [B][H][S][D] layout."""
    for n, t in (("q", q), ("k", k), ("v", v), ("out", out)):
        _check_tensor(n, t, (B, H, S, D))
    _check_mask(mask, H, S)
    st = load_library().attn_fwd_plain_async(
        _ptr(q), _ptr(k), _ptr(v), _ptr(out), B, H, S, D, float(scale), _ptr(mask),
        _stream(stream))
    _raise(st, "attn_fwd_plain_async")


def attn_fwd_plain(q, k, v, out, B, H, S, D, scale, mask=None):
    for n, t in (("q", q), ("k", k), ("v", v), ("out", out)):
        _check_tensor(n, t, (B, H, S, D))
    _check_mask(mask, H, S)
    st = load_library().attn_fwd_plain(
        _ptr(q), _ptr(k), _ptr(v), _ptr(out), B, H, S, D, float(scale), _ptr(mask))
    _raise(st, "attn_fwd_plain")


def _check_relayout(plain, out_slabs, B, H, S, D, P):
    if P > 0 and S % P == 0:
        _check_tensor("plain", plain, (B, H, S, D))
        _check_tensor("out_slabs", out_slabs, (P, B, S // P, H, D))


def relayout_to_slabs_async(plain, out_slabs, B, H, S, D, P, stream=None):
    """Enqueue the standalone copy plain [B][H][S][D] -> slabs [P][B][S/P][H][D]."""
    _check_relayout(plain, out_slabs, B, H, S, D, P)
    st = load_library().relayout_to_slabs_async(_ptr(plain), _ptr(out_slabs), B, H, S, D, P,
                                                _stream(stream))
    _raise(st, "relayout_to_slabs_async")


def relayout_to_slabs(plain, out_slabs, B, H, S, D, P):
    _check_relayout(plain, out_slabs, B, H, S, D, P)
    st = load_library().relayout_to_slabs(_ptr(plain), _ptr(out_slabs), B, H, S, D, P)
    _raise(st, "relayout_to_slabs")


def attn_fwd_workspace_bytes(B: int, H: int, S: int, D: int) -> int:
    """Workspace bytes a dense _ws_ call needs on the current device."""
    n = int(load_library().attn_fwd_workspace_bytes(B, H, S, D))
    _raise(n if n < 0 else FA_OK, "attn_fwd_workspace_bytes")
    return n


def _workspace(workspace, B, H, S, D, device):
    """The caller's workspace tensor, or one from torch's allocator."""
    if workspace is not None:
        if not workspace.is_cuda or not workspace.is_contiguous():
            raise ValueError("workspace must be a contiguous device tensor")
        return workspace
    n = attn_fwd_workspace_bytes(B, H, S, D)
    return torch.empty(max(n, 16), dtype=torch.uint8, device=device)


def _nbytes(t):
    return t.numel() * t.element_size()


def attn_fwd_relayout_ws_async(q, k, v, out_slabs, B, H, S, D, P, scale, mask=None,
                               workspace=None, stream=None):
    """Fused attention + slab store with the tail round spread over every
    workgroup; workspace: a device tensor of at least
    attn_fwd_workspace_bytes(B, H, S, D) bytes (allocated here when None)."""
    if P > 0 and S % P == 0:
        for n, t in (("q", q), ("k", k), ("v", v)):
            _check_tensor(n, t, (B, H, S, D))
        _check_tensor("out_slabs", out_slabs, (P, B, S // P, H, D))
        _check_mask(mask, H, S)
    ws = _workspace(workspace, B, H, S, D, q.device)
    st = load_library().attn_fwd_relayout_ws_async(
        _ptr(q), _ptr(k), _ptr(v), _ptr(out_slabs), B, H, S, D, P, float(scale), _ptr(mask),
        _ptr(ws), _nbytes(ws), _stream(stream))
    _raise(st, "attn_fwd_relayout_ws_async")
    return ws


def attn_fwd_plain_ws_async(q, k, v, out, B, H, S, D, scale, mask=None, workspace=None,
                            stream=None):
    """The plain-layout twin of attn_fwd_relayout_ws_async."""
    for n, t in (("q", q), ("k", k), ("v", v), ("out", out)):
        _check_tensor(n, t, (B, H, S, D))
    _check_mask(mask, H, S)
    ws = _workspace(workspace, B, H, S, D, q.device)
    st = load_library().attn_fwd_plain_ws_async(
        _ptr(q), _ptr(k), _ptr(v), _ptr(out), B, H, S, D, float(scale), _ptr(mask), _ptr(ws),
        _nbytes(ws), _stream(stream))
    _raise(st, "attn_fwd_plain_ws_async")
    return ws


def attn_fwd_relayout_noalloc_async(q, k, v, out_slabs, B, H, S, D, P, scale, mask=None,
                                    stream=None):
    """attn_fwd_relayout_ws_async with the library's static workspace: no
    device memory is allocated (calls that overlap on one GPU race)."""
    if P > 0 and S % P == 0:
        for n, t in (("q", q), ("k", k), ("v", v)):
            _check_tensor(n, t, (B, H, S, D))
        _check_tensor("out_slabs", out_slabs, (P, B, S // P, H, D))
        _check_mask(mask, H, S)
    st = load_library().attn_fwd_relayout_noalloc_async(
        _ptr(q), _ptr(k), _ptr(v), _ptr(out_slabs), B, H, S, D, P, float(scale), _ptr(mask),
        _stream(stream))
    _raise(st, "attn_fwd_relayout_noalloc_async")


def attn_instrumented_stamp_words(B: int, H: int, S: int) -> int:
    return int(load_library().attn_instrumented_stamp_words(B, H, S))


BOUNDARY_PIGGYBACK, BOUNDARY_COUPLED, BOUNDARY_ORDERED = 0, 1, 2


def attn_fwd_relayout_instrumented_async(q, k, v, out_slabs, B, H, S, D, P, scale, mask=None,
                                         boundary=BOUNDARY_PIGGYBACK, stamps=None, stream=None):
    """The fused call with per-tile timestamps (include/fa_instrument.h).
    boundary: 0 piggybacked (the product kernel's), 1 completion-coupled,
    2 stores then the next prologue with one wait.  stamps: int32 device
    tensor of at least attn_instrumented_stamp_words(B, H, S) elements.
    Returns the unit counts of the call's two launches."""
    if P > 0 and S % P == 0:
        for n, t in (("q", q), ("k", k), ("v", v)):
            _check_tensor(n, t, (B, H, S, D))
        _check_tensor("out_slabs", out_slabs, (P, B, S // P, H, D))
        _check_mask(mask, H, S)
    if stamps is None or stamps.dtype not in (torch.int32, torch.uint32) or not stamps.is_cuda \
            or not stamps.is_contiguous():
        raise ValueError("stamps must be a contiguous 32-bit device tensor")
    units = (ctypes.c_int * 2)()
    st = load_library().attn_fwd_relayout_instrumented_async(
        _ptr(q), _ptr(k), _ptr(v), _ptr(out_slabs), B, H, S, D, P, float(scale), _ptr(mask),
        int(boundary), _ptr(stamps), stamps.numel(), units, _stream(stream))
    _raise(st, "attn_fwd_relayout_instrumented_async")
    return int(units[0]), int(units[1])


def attention_relayout(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, P: int,
                       scale: Optional[float] = None, mask: Optional[torch.Tensor] = None,
                       out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Convenience form: shapes from q ([B][H][S][D]); allocates the slabs with
    torch when ``out`` is None; scale defaults to 1/sqrt(D)."""
    B, H, S, D = q.shape
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if out is None:
        if P <= 0 or S % P:
            _raise(-2 if P > 0 else -1, "attention_relayout")
        out = torch.empty((P, B, S // P, H, D), dtype=torch.bfloat16, device=q.device)
    attn_fwd_relayout_async(q, k, v, out, B, H, S, D, P, scale, mask, stream)
    return out


def attention_plain(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                    scale: Optional[float] = None, mask: Optional[torch.Tensor] = None,
                    out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    B, H, S, D = q.shape
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if out is None:
        out = torch.empty((B, H, S, D), dtype=torch.bfloat16, device=q.device)
    attn_fwd_plain_async(q, k, v, out, B, H, S, D, scale, mask, stream)
    return out
