"""Thin ctypes binding of libkda.so (include/kda.h).

Argument marshalling only: every step of the forward pass runs in the HIP
kernels behind ``kda_fwd``.  torch supplies device memory (the tensors and the
workspace) and the current HIP stream.  Importing this module loads the
library and raises ImportError when it has not been built; there is no other
code path.

``fwd`` keeps the argument list and order of ``flash_kda.fwd`` in the FlashKDA
README mirror (section "内核 API").
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libkda.so")

KDA_OK, KDA_EINVAL, KDA_EDTYPE, KDA_EWORKSPACE, KDA_EUNSUPPORTED, KDA_EHIP = range(6)
KDA_DTYPE_NONE, KDA_DTYPE_BF16, KDA_DTYPE_FP32 = 0, 1, 2
KDA_STATUS_OK, KDA_STATUS_BAD_CU_SEQLENS, KDA_STATUS_OVERFLOW, KDA_STATUS_SYNC_TIMEOUT = 0, 1, 2, 4
KDA_PATH_AUTO, KDA_PATH_SPLIT, KDA_PATH_FUSED = 0, 1, 2
KDA_PREC_DEFAULT, KDA_PREC_BF16_STATE, KDA_PREC_BF16_INVERSE, KDA_PREC_BF16_STATE_PRODUCTS = 0, 1, 2, 4
KDA_PREC_NEUMANN_FP16 = 8
PATHS = {None: KDA_PATH_AUTO, "auto": KDA_PATH_AUTO, "split": KDA_PATH_SPLIT, "fused": KDA_PATH_FUSED,
         KDA_PATH_AUTO: KDA_PATH_AUTO, KDA_PATH_SPLIT: KDA_PATH_SPLIT, KDA_PATH_FUSED: KDA_PATH_FUSED}
CHUNK = 16

EXPORTS = ("kda_fwd", "kda_fwd_profiled", "kda_fwd_ex", "kda_fwd_parts", "kda_fwd_path", "kda_fwd_path_taken",
           "kda_fwd_num_events", "kda_fwd_segmented", "kda_fwd_segmented_workspace_bytes",
           "kda_fwd_segments", "kda_fwd_precision",
           "kda_decode", "kda_fwd_workspace_bytes", "kda_fwd_workspace_bytes_ex", "kda_get_last_error",
           "kda_version", "kda_fwd_check_status", "kda_workspace_layout", "kda_debug_prep",
           "kda_fwd_fused_noalloc", "kda_debug_set_spin_limit")

if not os.path.exists(LIB_PATH):
    raise ImportError("libkda.so is not built (run gated_delta_rule_prep_amd/build.py or "
                      "__graft_entry__.build()); there is no fallback path")

_lib = ctypes.CDLL(LIB_PATH)
_p = ctypes.c_void_p
_i64 = ctypes.c_int64
_lib.kda_fwd.argtypes = [_p, _p, _p, _p, _p, ctypes.c_float, _p, _p, _p, ctypes.c_float,
                         _p, ctypes.c_int, _p, ctypes.c_int, _p, _i64, _i64, _i64, _i64, _i64, _i64,
                         _p, ctypes.c_size_t, _p]
_lib.kda_fwd.restype = ctypes.c_int
_lib.kda_fwd_profiled.argtypes = _lib.kda_fwd.argtypes + [ctypes.POINTER(ctypes.c_void_p)]
_lib.kda_fwd_profiled.restype = ctypes.c_int
_lib.kda_fwd_ex.argtypes = _lib.kda_fwd.argtypes + [ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                                     ctypes.POINTER(ctypes.c_void_p), ctypes.c_int]
_lib.kda_fwd_ex.restype = ctypes.c_int
_lib.kda_fwd_parts.argtypes = [_i64, _i64, ctypes.c_int]
_lib.kda_fwd_parts.restype = ctypes.c_int
_lib.kda_fwd_path.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int]
_lib.kda_fwd_path.restype = ctypes.c_int
_lib.kda_fwd_path_taken.argtypes = [_p, _p, ctypes.POINTER(ctypes.c_int)]
_lib.kda_fwd_path_taken.restype = ctypes.c_int
_lib.kda_fwd_num_events.argtypes = [_i64, _i64, ctypes.c_int, ctypes.c_int, ctypes.c_int]
_lib.kda_fwd_num_events.restype = ctypes.c_int
_lib.kda_fwd_workspace_bytes_ex.argtypes = [_i64, _i64, _i64, _i64, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                            ctypes.c_int]
_lib.kda_fwd_workspace_bytes_ex.restype = ctypes.c_size_t
_lib.kda_fwd_segmented.argtypes = _lib.kda_fwd.argtypes[:21] + [ctypes.c_int, _p, ctypes.c_size_t, _p]
_lib.kda_fwd_segmented.restype = ctypes.c_int
_lib.kda_fwd_segmented_workspace_bytes.argtypes = [_i64, _i64, _i64, _i64, ctypes.c_int, ctypes.c_int]
_lib.kda_fwd_segmented_workspace_bytes.restype = ctypes.c_size_t
_lib.kda_fwd_precision.argtypes = _lib.kda_fwd.argtypes + [ctypes.c_int]
_lib.kda_fwd_precision.restype = ctypes.c_int
_lib.kda_fwd_segments.argtypes = [_i64, _i64, _i64, _i64, ctypes.c_int]
_lib.kda_fwd_segments.restype = ctypes.c_int
_lib.kda_decode.argtypes = [_p, _p, _p, _p, _p, ctypes.c_float, _p, _p, _p, ctypes.c_float,
                            _p, ctypes.c_int, _p, ctypes.c_int, _i64, _i64, _i64, _i64, _p]
_lib.kda_decode.restype = ctypes.c_int
_lib.kda_fwd_workspace_bytes.argtypes = [_i64, _i64, _i64, _i64, ctypes.c_int]
_lib.kda_fwd_workspace_bytes.restype = ctypes.c_size_t
_lib.kda_get_last_error.restype = ctypes.c_char_p
_lib.kda_version.restype = ctypes.c_int
_lib.kda_fwd_check_status.argtypes = [_p, _p, ctypes.POINTER(ctypes.c_int)]
_lib.kda_fwd_check_status.restype = ctypes.c_int
_lib.kda_workspace_layout.argtypes = [_i64, _i64, _i64, _i64, ctypes.c_int, ctypes.c_int,
                                      ctypes.POINTER(ctypes.c_int64)]
_lib.kda_workspace_layout.restype = ctypes.c_int
_lib.kda_debug_prep.argtypes = [_p, _p, _p, _p, ctypes.c_float, _p, _p, ctypes.c_float, _p, _i64, _i64,
                                _i64, _i64, _i64, _p, ctypes.c_size_t, _p, ctypes.c_int]
_lib.kda_debug_prep.restype = ctypes.c_int
_lib.kda_fwd_fused_noalloc.argtypes = _lib.kda_fwd.argtypes[:21] + [_p]
_lib.kda_fwd_fused_noalloc.restype = ctypes.c_int
_lib.kda_debug_set_spin_limit.argtypes = [ctypes.c_int]
_lib.kda_debug_set_spin_limit.restype = ctypes.c_int


class KDAError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__("%s (code %d)" % (msg, code))
        self.code = code


class KDAValueError(KDAError, ValueError):
    pass


def lib() -> ctypes.CDLL:
    return _lib


def last_error() -> str:
    return _lib.kda_get_last_error().decode()


def version() -> int:
    return _lib.kda_version()


def _raise(code: int):
    msg = last_error()
    if code in (KDA_EINVAL, KDA_EDTYPE):
        raise KDAValueError(code, msg)
    raise KDAError(code, msg)


def _path_code(path) -> int:
    if path not in PATHS:
        raise KDAValueError(KDA_EINVAL, "path must be None, 'auto', 'split' or 'fused', got %r" % (path,))
    return PATHS[path]


def workspace_bytes(B: int, T: int, H: int, num_seqs: int = 0, has_cu_seqlens: bool = False, chunk=None,
                    parts=None, path=None) -> int:
    """Workspace bytes: with no chunk / parts / path, a size that suits every
    path (kda_fwd_workspace_bytes); otherwise what that configuration needs
    (kda_fwd_workspace_bytes_ex)."""
    if chunk is None and parts is None and path is None:
        return int(_lib.kda_fwd_workspace_bytes(B, T, H, num_seqs, int(has_cu_seqlens)))
    return int(_lib.kda_fwd_workspace_bytes_ex(B, T, H, num_seqs, int(has_cu_seqlens), int(chunk or 0),
                                               int(parts or 0), _path_code(path)))


_PATH_NAMES = {KDA_PATH_AUTO: "auto", KDA_PATH_SPLIT: "split", KDA_PATH_FUSED: "fused"}


def path_used(chunk=None, parts=None, path=None) -> str:
    """'split', 'fused' or 'auto' (chosen on the device by the scheduler
    kernel): the path kda_fwd_ex takes for these requests."""
    p = _lib.kda_fwd_path(int(chunk or 0), int(parts or 0), _path_code(path))
    if p < 0:
        raise KDAValueError(KDA_EINVAL, "invalid chunk / parts / path combination")
    return _PATH_NAMES[p]


def path_taken(workspace: torch.Tensor) -> str:
    """'split' or 'fused': the path the last call using this workspace ran
    (synchronises the current stream)."""
    p = ctypes.c_int(-1)
    with torch.cuda.device(workspace.device):
        rc = _lib.kda_fwd_path_taken(_ptr(workspace), _stream(workspace.device), ctypes.byref(p))
    if rc != KDA_OK:
        _raise(rc)
    return _PATH_NAMES.get(p.value, "unknown")


def num_events(B: int, T: int, chunk=None, parts=None, path=None) -> int:
    """Events kda_fwd_ex records for these sizes and requests."""
    return int(_lib.kda_fwd_num_events(B, T, int(chunk or 0), int(parts or 0), _path_code(path)))


def workspace_layout(B: int, T: int, H: int, num_seqs: int = 0, has_cu_seqlens: bool = False,
                     chunk: int = CHUNK) -> dict:
    off = (ctypes.c_int64 * 7)()
    rc = _lib.kda_workspace_layout(B, T, H, num_seqs, int(has_cu_seqlens), chunk, off)
    if rc != KDA_OK:
        _raise(rc)
    keys = ("chunk_table", "seq_table", "order", "records", "rec_bytes", "max_chunks", "total")
    return dict(zip(keys, [int(x) for x in off]))


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _state_code(t: Optional[torch.Tensor]) -> int:
    if t is None:
        return KDA_DTYPE_NONE
    if t.dtype == torch.bfloat16:
        return KDA_DTYPE_BF16
    if t.dtype == torch.float32:
        return KDA_DTYPE_FP32
    raise KDAValueError(KDA_EDTYPE, "state tensors must be bfloat16 or float32, got %s" % t.dtype)


def _check(name, t, dtype, shape=None):
    if t.dtype != dtype:
        raise KDAValueError(KDA_EDTYPE, "%s must be %s, got %s" % (name, dtype, t.dtype))
    if not t.is_contiguous():
        raise KDAValueError(KDA_EINVAL, "%s must be contiguous" % name)
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise KDAValueError(KDA_EINVAL, "%s must have shape %s, got %s" % (name, tuple(shape), tuple(t.shape)))


def _stream(device: torch.device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def alloc_workspace(B: int, T: int, H: int, num_seqs: int, has_cu: bool, device, chunk=None, parts=None,
                    path=None) -> torch.Tensor:
    n = workspace_bytes(B, T, H, num_seqs, has_cu, chunk, parts, path)
    if n == 0:
        raise KDAValueError(KDA_EINVAL, "bad sizes for the workspace: B=%d T=%d H=%d" % (B, T, H))
    return torch.empty(n, dtype=torch.uint8, device=device)


def segmented_workspace_bytes(B: int, T: int, H: int, num_seqs: int, has_cu_seqlens: bool, segments: int) -> int:
    """Bytes of workspace kda_fwd_segmented needs (0 on bad sizes)."""
    return _lib.kda_fwd_segmented_workspace_bytes(B, T, H, num_seqs, int(bool(has_cu_seqlens)), int(segments))


def segments_for(B: int, T: int, H: int, num_seqs: int = 0, has_cu_seqlens: bool = False) -> int:
    """The segment count kda_fwd_segmented chooses for segments = 0."""
    return _lib.kda_fwd_segments(B, T, H, num_seqs, int(bool(has_cu_seqlens)))


def parts(B: int, T: int, requested: int = 0) -> int:
    """Parts (overlapped prep / recurrence ranges) a call uses; see kda_fwd_ex."""
    return _lib.kda_fwd_parts(B, T, requested)


def _fwd_shapes(q, k, v, g, beta, out, A_log, dt_bias, initial_state, final_state, cu_seqlens):
    """Shape, dtype and device checks of the forward entry points; returns
    (B, T, H, K, V, N, device)."""
    if q.dim() != 4:
        raise KDAValueError(KDA_EINVAL, "q must be [B, T, H, K]")
    B, T, H, K = q.shape
    V = v.shape[-1]
    dev = q.device
    _check("q", q, torch.bfloat16)
    _check("k", k, torch.bfloat16, (B, T, H, K))
    _check("g", g, torch.bfloat16, (B, T, H, K))
    _check("v", v, torch.bfloat16, (B, T, H, V))
    _check("beta", beta, torch.bfloat16, (B, T, H))
    _check("out", out, torch.bfloat16, (B, T, H, V))
    _check("A_log", A_log, torch.float32, (H,))
    _check("dt_bias", dt_bias, torch.float32, (H, K))
    if cu_seqlens is not None:
        _check("cu_seqlens", cu_seqlens, torch.int64)
        if cu_seqlens.dim() != 1 or cu_seqlens.numel() < 2:
            raise KDAValueError(KDA_EINVAL, "cu_seqlens must be a 1-D int64 tensor of N + 1 >= 2 entries")
        N = cu_seqlens.numel() - 1
    else:
        N = B
    for name, t in (("initial_state", initial_state), ("final_state", final_state)):
        if t is not None:
            _state_code(t)
            _check(name, t, t.dtype, (N, H, V, K))
    tensors = [q, k, v, g, beta, out, A_log, dt_bias, initial_state, final_state, cu_seqlens]
    for t in tensors:
        if t is not None and t.device != dev:
            raise KDAValueError(KDA_EINVAL, "all tensors must be on %s" % dev)
    if dev.type != "cuda":
        raise KDAValueError(KDA_EINVAL, "tensors must be on a HIP device, got %s" % dev)
    return B, T, H, K, V, N, dev


def fwd(q, k, v, g, beta, scale, out, A_log, dt_bias, lower_bound, initial_state=None, final_state=None,
        cu_seqlens=None, workspace: Optional[torch.Tensor] = None, events=None, parts: Optional[int] = None,
        chunk: Optional[int] = None, path=None, segments: Optional[int] = None, precision: Optional[int] = None):
    """Chunked KDA forward into the caller's ``out`` (and ``final_state``).

    Shapes and dtypes as in include/kda.h.  Runs on the current stream of the
    tensors' device.  Returns ``out``.  ``path``: None / 'auto' for the
    library's choice, 'split' or 'fused' (kda_fwd_ex).  ``chunk``: None for
    the library's choice, or 16 / 32 / 64 tokens per chunk (32, 64: split path
    only).
    ``parts``: None for one, or the number of overlapped ranges (split path).
    ``events``: optional torch.cuda.Event list (enable_timing=True): with no
    chunk / parts / path, four go through kda_fwd_profiled; otherwise
    ``num_events(B, T, chunk, parts, path)`` go through kda_fwd_ex, which
    records them around every kernel.  ``segments``: cut every sequence into
    that many pieces run side by side (kda_fwd_segmented; 0 or 'auto' for the
    library's choice); it takes none of events / parts / chunk / path.
    ``precision``: a KDA_PREC_* combination for the precision study entry
    point kda_fwd_precision (split path, 16-token chunks); it takes none of
    events / parts / chunk / path / segments.
    """
    B, T, H, K, V, N, dev = _fwd_shapes(q, k, v, g, beta, out, A_log, dt_bias, initial_state, final_state,
                                        cu_seqlens)
    path_c = _path_code(path)
    if segments == "auto":
        segments = 0
    if precision is not None:
        if events is not None or parts is not None or chunk is not None or path is not None or segments is not None:
            raise KDAValueError(KDA_EINVAL, "precision takes none of events, parts, chunk, path, segments")
        if workspace is None:
            workspace = alloc_workspace(B, T, H, N, cu_seqlens is not None, dev, 16, 1, "split")
    if segments is not None:
        if events is not None or parts is not None or chunk is not None or path is not None:
            raise KDAValueError(KDA_EINVAL, "segments takes none of events, parts, chunk, path")
        if workspace is None:
            n = segmented_workspace_bytes(B, T, H, N, cu_seqlens is not None, segments)
            if n == 0:
                raise KDAValueError(KDA_EINVAL, "bad sizes for the workspace: B=%d T=%d H=%d segments=%d" % (
                    B, T, H, segments))
            workspace = torch.empty(n, dtype=torch.uint8, device=dev)
    elif workspace is None:   # what this call's path needs (kda_fwd: every form it may take)
        workspace = alloc_workspace(B, T, H, N, cu_seqlens is not None, dev, chunk, parts, path)
    args = (_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), float(scale), _ptr(out),
            _ptr(A_log), _ptr(dt_bias), float(lower_bound), _ptr(initial_state),
            _state_code(initial_state), _ptr(final_state), _state_code(final_state),
            _ptr(cu_seqlens), N, B, T, H, K, V, _ptr(workspace), workspace.numel())
    with torch.cuda.device(dev):
        plain = parts is None and chunk is None and path is None
        if precision is not None:
            rc = _lib.kda_fwd_precision(*args, _stream(dev), int(precision))
        elif segments is not None:
            rc = _lib.kda_fwd_segmented(*args[:21], int(segments), *args[21:], _stream(dev))
        elif events is None and plain:
            rc = _lib.kda_fwd(*args, _stream(dev))
        elif plain and len(events) == 4:
            ev = (ctypes.c_void_p * 4)(*[e.cuda_event for e in events])
            rc = _lib.kda_fwd_profiled(*args, _stream(dev), ev)
        else:
            n = 0 if events is None else len(events)
            ev = None if events is None else (ctypes.c_void_p * n)(*[e.cuda_event for e in events])
            rc = _lib.kda_fwd_ex(*args, _stream(dev), int(chunk or 0), int(parts or 0), path_c, ev, n)
    if rc != KDA_OK:
        _raise(rc)
    return out


def fwd_fused_noalloc(q, k, v, g, beta, scale, out, A_log, dt_bias, lower_bound, initial_state=None,
                      final_state=None, cu_seqlens=None):
    """kda_fwd_fused_noalloc: the fused path with the library's static
    per-GPU scratch instead of a workspace (at most 16384 sequences; calls
    that overlap on one GPU race).  Same arguments and results as ``fwd(...,
    path='fused')``.  Returns ``out``."""
    B, T, H, K, V, N, dev = _fwd_shapes(q, k, v, g, beta, out, A_log, dt_bias, initial_state, final_state,
                                        cu_seqlens)
    args = (_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), float(scale), _ptr(out),
            _ptr(A_log), _ptr(dt_bias), float(lower_bound), _ptr(initial_state),
            _state_code(initial_state), _ptr(final_state), _state_code(final_state),
            _ptr(cu_seqlens), N, B, T, H, K, V)
    with torch.cuda.device(dev):
        rc = _lib.kda_fwd_fused_noalloc(*args, _stream(dev))
    if rc != KDA_OK:
        _raise(rc)
    return out


def decode(q, k, v, g, beta, scale, out, A_log, dt_bias, lower_bound, initial_state=None, final_state=None):
    """One recurrent step, one token per sequence (kda_decode), into ``out``.

    q, k, g, v: bf16 [N, H, 128] or [N, 1, H, 128]; beta: bf16 [N, H] or
    [N, 1, H]; out like v; states [N, H, V, K] (bf16 / fp32, may be the same
    tensor).  Runs on the current stream of the tensors' device.  Returns out.
    """
    if q.dim() == 4:
        if q.shape[1] != 1:
            raise KDAValueError(KDA_EINVAL, "decode takes one token per sequence: q must be [N, 1, H, K]")
        N, _, H, K = q.shape
    elif q.dim() == 3:
        N, H, K = q.shape
    else:
        raise KDAValueError(KDA_EINVAL, "q must be [N, H, K] or [N, 1, H, K]")
    V = v.shape[-1]
    dev = q.device
    for name, t, last in (("q", q, K), ("k", k, K), ("g", g, K), ("v", v, V), ("out", out, V), ("beta", beta, 1)):
        _check(name, t, torch.bfloat16)
        if t.numel() != N * H * last:
            raise KDAValueError(KDA_EINVAL, "%s has %d elements, expected %d (N=%d, H=%d)"
                                % (name, t.numel(), N * H * last, N, H))
    _check("A_log", A_log, torch.float32, (H,))
    _check("dt_bias", dt_bias, torch.float32, (H, K))
    for name, t in (("initial_state", initial_state), ("final_state", final_state)):
        if t is not None:
            _state_code(t)
            _check(name, t, t.dtype, (N, H, V, K))
    for t in (q, k, v, g, beta, out, A_log, dt_bias, initial_state, final_state):
        if t is not None and t.device != dev:
            raise KDAValueError(KDA_EINVAL, "all tensors must be on %s" % dev)
    if dev.type != "cuda":
        raise KDAValueError(KDA_EINVAL, "tensors must be on a HIP device, got %s" % dev)
    with torch.cuda.device(dev):
        rc = _lib.kda_decode(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), float(scale), _ptr(out),
                             _ptr(A_log), _ptr(dt_bias), float(lower_bound), _ptr(initial_state),
                             _state_code(initial_state), _ptr(final_state), _state_code(final_state),
                             N, H, K, V, _stream(dev))
    if rc != KDA_OK:
        _raise(rc)
    return out


def check_status(workspace: torch.Tensor) -> int:
    st = ctypes.c_int(-1)
    with torch.cuda.device(workspace.device):
        rc = _lib.kda_fwd_check_status(_ptr(workspace), _stream(workspace.device), ctypes.byref(st))
    if rc != KDA_OK:
        _raise(rc)
    return st.value


def debug_set_spin_limit(polls: int) -> None:
    """Test-only: the waits between waves (recurrence, fused kernel) give up after `polls`
    polls (0: at once) in the launches that follow; negative restores the default."""
    _lib.kda_debug_set_spin_limit(int(polls))


def debug_prep(q, k, g, beta, scale, A_log, dt_bias, lower_bound, cu_seqlens=None, workspace=None,
               chunk: int = CHUNK):
    """Test-only: run the scheduler and prep kernels; returns the workspace tensor."""
    B, T, H, K = q.shape
    N = B if cu_seqlens is None else cu_seqlens.numel() - 1
    if workspace is None:
        workspace = alloc_workspace(B, T, H, N, cu_seqlens is not None, q.device, chunk, 1, "split")
    with torch.cuda.device(q.device):
        rc = _lib.kda_debug_prep(_ptr(q), _ptr(k), _ptr(g), _ptr(beta), float(scale), _ptr(A_log),
                                 _ptr(dt_bias), float(lower_bound), _ptr(cu_seqlens), N, B, T, H, K,
                                 _ptr(workspace), workspace.numel(), _stream(q.device), chunk)
    if rc != KDA_OK:
        _raise(rc)
    return workspace
