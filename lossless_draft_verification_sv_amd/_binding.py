"""ctypes binding of libsv.so: argument marshalling only.

Every step of verification runs in the HIP kernels behind the C ABI (include/sv.h). This module
turns torch tensors into device pointers, allocates outputs and the workspace with torch on the
tensors' device, and passes torch's current HIP stream. If the library is missing it raises;
there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os
import threading
from typing import NamedTuple, Optional

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIBRARY_PATH = os.path.join(_PKG, "libsv.so")

SV_OK = 0
SV_ERR_INVALID_ARG = -1
SV_ERR_UNSUPPORTED = -2
SV_ERR_WORKSPACE = -3
SV_ERR_HIP = -4
SV_DTYPE_F32 = 0
SV_DTYPE_BF16 = 1

_lock = threading.Lock()
_lib = None


class SVError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"sv status {status}: {message}")
        self.status = status


def load_library(path: str = LIBRARY_PATH) -> ctypes.CDLL:
    """Load libsv.so once and declare the C signatures. Raises if it has not been built."""
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(path):
            raise RuntimeError(
                f"{path} is missing: build it with `python -m "
                "lossless_draft_verification_sv_amd.build` (hipcc, gfx950)")
        lib = ctypes.CDLL(path)
        vp, i32, f32, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
        lib.sv_workspace_bytes.argtypes = [i32, i32, i32]
        lib.sv_workspace_bytes.restype = sz
        lib.sv_status_string.argtypes = [i32]
        lib.sv_status_string.restype = ctypes.c_char_p
        lib.sv_last_error.argtypes = []
        lib.sv_last_error.restype = ctypes.c_char_p
        lib.sv_verify_batch.argtypes = [vp, vp, i32, i32, i32, i32, f32, vp, vp, vp, vp, vp, vp,
                                        vp, vp, vp, sz, vp]
        lib.sv_verify_batch.restype = i32
        lib.sv_verify_batch_noalloc.argtypes = [vp, vp, i32, i32, i32, i32, f32, vp, vp, vp, vp,
                                                vp, vp, vp, vp, vp]
        lib.sv_verify_batch_noalloc.restype = i32
        lib.sv_verify_greedy.argtypes = [vp, i32, i32, i32, i32, vp, vp, vp, vp, vp, sz, vp]
        lib.sv_verify_greedy.restype = i32
        i64 = ctypes.c_int64
        lib.sv_verify_ragged.argtypes = [vp, vp, i32, i32, i32, i32, i64, i64, vp, vp, vp, vp,
                                         vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
        lib.sv_verify_ragged.restype = i32
        lib.sv_schedule_prefix.argtypes = [vp, i32, i32, vp, i32, f32, vp, vp, vp, vp, vp, sz,
                                           vp]
        lib.sv_schedule_prefix.restype = i32
        lib.sv_schedule_workspace_bytes.argtypes = [i32, i32]
        lib.sv_schedule_workspace_bytes.restype = sz
        lib.sv_markov_workspace_bytes.argtypes = [i32, i32]
        lib.sv_markov_workspace_bytes.restype = sz
        lib.sv_markov_draft.argtypes = [vp, i32, i32, i32, i32, vp, vp, i32, vp, vp, vp, vp, sz,
                                        vp]
        lib.sv_markov_draft.restype = i32
        lib.sv_markov_draft_sampled.argtypes = [vp, i32, i32, i32, i32, vp, vp, i32, vp, vp, vp,
                                                vp, vp, vp, sz, vp]
        lib.sv_markov_draft_sampled.restype = i32
        lib.sv_markov_topk_workspace_bytes.argtypes = [i32, i32, i32]
        lib.sv_markov_topk_workspace_bytes.restype = sz
        lib.sv_markov_topk.argtypes = [vp, i32, i32, i32, i32, vp, vp, i32, i32, vp, vp, vp, vp,
                                       vp, sz, vp]
        lib.sv_markov_topk.restype = i32
        lib.sv_read_probe.argtypes = [vp, sz, vp, i32, vp]
        lib.sv_read_probe.restype = i32
        lib.sv_set_call_counter.argtypes = [ctypes.c_uint64]
        lib.sv_set_call_counter.restype = None
        _lib = lib
        return lib


def sv_workspace_bytes(B: int, K: int, V: int) -> int:
    return int(load_library().sv_workspace_bytes(B, K, V))


def sv_status_string(status: int) -> str:
    return load_library().sv_status_string(status).decode()


def sv_last_error() -> str:
    return load_library().sv_last_error().decode()


def _check(status: int) -> None:
    if status != SV_OK:
        raise SVError(status, f"{sv_status_string(status)}: {sv_last_error()}")


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return SV_DTYPE_F32
    if t.dtype == torch.bfloat16:
        return SV_DTYPE_BF16
    raise TypeError(f"logits must be float32 or bfloat16, got {t.dtype}")


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _need(t: torch.Tensor, name: str, dtype, shape, device) -> None:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


_ws_cache = {}


def _workspace(device: torch.device, stream: int, nbytes: int,
               kind: str = "verify") -> torch.Tensor:
    """One cached workspace per (device, stream, kind), zero-filled when allocated: calls on one
    stream never overlap, and a workspace needs no clearing between calls (the library stamps
    every word it hands between work-groups with a fresh call number, and zero-fills a workspace
    itself after its call counter wraps). Kinds that leave untagged words behind get their own
    workspace: "markov" (the per-position form's tile argmaxes) and "markov_topk" (candidate
    tables), so that no function reads another's untagged words as tagged ones."""
    key = (device, stream, kind)
    ws = _ws_cache.get(key)
    if ws is None or ws.numel() < nbytes:
        ws = torch.zeros(max(nbytes, 256), dtype=torch.uint8, device=device)
        _ws_cache[key] = ws
    return ws


class VerifyOutput(NamedTuple):
    accepted_len: torch.Tensor  # [B] int32
    committed: torch.Tensor  # [B, K+1] int32
    target_prob: Optional[torch.Tensor]  # [B, K] float32 (sampling mode)
    draft_prob: Optional[torch.Tensor]  # [B, K] float32 (sampling mode, on request)


def sv_verify_batch(target: torch.Tensor, draft: torch.Tensor, draft_tokens: torch.Tensor,
                    uniforms: torch.Tensor, residual_uniform: torch.Tensor,
                    temperature: float = 1.0, num_draft: Optional[torch.Tensor] = None,
                    return_draft_prob: bool = False) -> VerifyOutput:
    """Sampling-mode verification on the tensors' GPU (see sv_verify_batch in include/sv.h).

    target [B, K+1, V] and draft [B, K, V]: float32 or bfloat16 logits; draft_tokens [B, K]
    int32; uniforms [B, K] float32; residual_uniform [B] float32; num_draft [B] int32 or None.
    """
    lib = load_library()
    if target.dim() != 3:
        raise ValueError("target must be [B, K+1, V]")
    B, K1, V = target.shape
    K = K1 - 1
    dev = target.device
    if dev.type != "cuda":
        raise ValueError("target must be a GPU tensor")
    _need(draft, "draft", target.dtype, (B, K, V), dev)
    _need(target, "target", target.dtype, (B, K + 1, V), dev)
    _need(draft_tokens, "draft_tokens", torch.int32, (B, K), dev)
    _need(uniforms, "uniforms", torch.float32, (B, K), dev)
    _need(residual_uniform, "residual_uniform", torch.float32, (B,), dev)
    if num_draft is not None:
        _need(num_draft, "num_draft", torch.int32, (B,), dev)
    acc = torch.empty(B, dtype=torch.int32, device=dev)
    com = torch.empty(B, K + 1, dtype=torch.int32, device=dev)
    tp = torch.empty(B, K, dtype=torch.float32, device=dev)
    dp = torch.empty(B, K, dtype=torch.float32, device=dev) if return_draft_prob else None
    stream = torch.cuda.current_stream(dev).cuda_stream
    nbytes = int(lib.sv_workspace_bytes(B, K, V))
    ws = _workspace(dev, stream, nbytes)
    _check(lib.sv_verify_batch(
        _ptr(target), _ptr(draft), _dtype_code(target), B, K, V, float(temperature),
        _ptr(draft_tokens), _ptr(num_draft), _ptr(uniforms), _ptr(residual_uniform), _ptr(acc),
        _ptr(com), _ptr(tp), _ptr(dp), _ptr(ws), ws.numel(), stream))
    return VerifyOutput(acc, com, tp, dp)


def sv_verify_greedy(target: torch.Tensor, draft_tokens: torch.Tensor,
                     num_draft: Optional[torch.Tensor] = None) -> VerifyOutput:
    """Greedy-mode verification on the tensors' GPU (see sv_verify_greedy in include/sv.h)."""
    lib = load_library()
    if target.dim() != 3:
        raise ValueError("target must be [B, K+1, V]")
    B, K1, V = target.shape
    K = K1 - 1
    dev = target.device
    if dev.type != "cuda":
        raise ValueError("target must be a GPU tensor")
    _need(target, "target", target.dtype, (B, K + 1, V), dev)
    _need(draft_tokens, "draft_tokens", torch.int32, (B, K), dev)
    if num_draft is not None:
        _need(num_draft, "num_draft", torch.int32, (B,), dev)
    acc = torch.empty(B, dtype=torch.int32, device=dev)
    com = torch.empty(B, K + 1, dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream(dev).cuda_stream
    nbytes = int(lib.sv_workspace_bytes(B, K, V))
    ws = _workspace(dev, stream, nbytes)
    _check(lib.sv_verify_greedy(
        _ptr(target), _dtype_code(target), B, K, V, _ptr(draft_tokens), _ptr(num_draft),
        _ptr(acc), _ptr(com), _ptr(ws), ws.numel(), stream))
    return VerifyOutput(acc, com, None, None)


def sv_verify_ragged(target: torch.Tensor, draft: Optional[torch.Tensor],
                     draft_tokens: torch.Tensor, uniforms: torch.Tensor,
                     residual_uniform: torch.Tensor, temperature: torch.Tensor,
                     num_draft: torch.Tensor, target_row_start: torch.Tensor,
                     draft_row_start: torch.Tensor,
                     return_draft_prob: bool = False) -> VerifyOutput:
    """Flattened, mixed-mode verification on the tensors' GPU (see sv_verify_ragged in
    include/sv.h).

    target [rows_t, V] and draft [rows_d, V] (or None when no request samples): float32 or
    bfloat16 logit rows; draft_tokens [B, K] int32; uniforms [B, K] float32; residual_uniform
    [B] float32; temperature [B] float32 (0 = greedy request); num_draft, target_row_start,
    draft_row_start [B] int32.
    """
    lib = load_library()
    if target.dim() != 2:
        raise ValueError("target must be [rows, V]")
    rows_t, V = target.shape
    dev = target.device
    if dev.type != "cuda":
        raise ValueError("target must be a GPU tensor")
    _need(target, "target", target.dtype, (rows_t, V), dev)
    if draft is not None:
        if draft.dim() != 2:
            raise ValueError("draft must be [rows, V]")
        _need(draft, "draft", target.dtype, (draft.shape[0], V), dev)
    rows_d = 0 if draft is None else draft.shape[0]
    if draft_tokens.dim() != 2:
        raise ValueError("draft_tokens must be [B, K]")
    B, K = draft_tokens.shape
    _need(draft_tokens, "draft_tokens", torch.int32, (B, K), dev)
    _need(uniforms, "uniforms", torch.float32, (B, K), dev)
    _need(residual_uniform, "residual_uniform", torch.float32, (B,), dev)
    _need(temperature, "temperature", torch.float32, (B,), dev)
    for t, n in ((num_draft, "num_draft"), (target_row_start, "target_row_start"),
                 (draft_row_start, "draft_row_start")):
        _need(t, n, torch.int32, (B,), dev)
    acc = torch.empty(B, dtype=torch.int32, device=dev)
    com = torch.empty(B, K + 1, dtype=torch.int32, device=dev)
    tp = torch.empty(B, K, dtype=torch.float32, device=dev)
    dp = torch.empty(B, K, dtype=torch.float32, device=dev) if return_draft_prob else None
    stream = torch.cuda.current_stream(dev).cuda_stream
    nbytes = int(lib.sv_workspace_bytes(B, K, V))
    ws = _workspace(dev, stream, nbytes)
    _check(lib.sv_verify_ragged(
        _ptr(target), _ptr(draft), _dtype_code(target), B, K, V, rows_t, rows_d,
        _ptr(target_row_start), _ptr(draft_row_start), _ptr(num_draft), _ptr(temperature),
        _ptr(draft_tokens), _ptr(uniforms), _ptr(residual_uniform), _ptr(acc), _ptr(com),
        _ptr(tp), _ptr(dp), _ptr(ws), ws.numel(), stream))
    return VerifyOutput(acc, com, tp, dp)


class ScheduleOutput(NamedTuple):
    num_draft: torch.Tensor  # [B] int32
    target_row_start: torch.Tensor  # [B] int32
    draft_row_start: torch.Tensor  # [B] int32
    summary: torch.Tensor  # [2] float32: N chosen, expected tokens per unit time


def sv_schedule_prefix(confidence: torch.Tensor, step_time: Optional[torch.Tensor] = None,
                       threshold: float = 0.5) -> ScheduleOutput:
    """Confidence-scheduled prefix selection on the tensor's GPU (see sv_schedule_prefix in
    include/sv.h). confidence [B, K] float32; step_time [T] float32 (hardware-aware mode) or
    None (threshold mode)."""
    lib = load_library()
    if confidence.dim() != 2:
        raise ValueError("confidence must be [B, K]")
    B, K = confidence.shape
    dev = confidence.device
    if dev.type != "cuda":
        raise ValueError("confidence must be a GPU tensor")
    _need(confidence, "confidence", torch.float32, (B, K), dev)
    T = 0
    if step_time is not None:
        if step_time.dim() != 1:
            raise ValueError("step_time must be [T]")
        T = step_time.shape[0]
        _need(step_time, "step_time", torch.float32, (T,), dev)
    num = torch.empty(B, dtype=torch.int32, device=dev)
    ts = torch.empty(B, dtype=torch.int32, device=dev)
    ds = torch.empty(B, dtype=torch.int32, device=dev)
    summ = torch.empty(2, dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev).cuda_stream
    ws, nbytes = None, 0
    if step_time is not None:
        nbytes = int(lib.sv_schedule_workspace_bytes(B, K))
        ws = _workspace(dev, stream, nbytes)
    _check(lib.sv_schedule_prefix(_ptr(confidence), B, K, _ptr(step_time), T, float(threshold),
                                  _ptr(num), _ptr(ts), _ptr(ds), _ptr(summ), _ptr(ws), nbytes,
                                  stream))
    return ScheduleOutput(num, ts, ds, summ)


def sv_markov_draft(base: torch.Tensor, left_factor: torch.Tensor, right_factor: torch.Tensor,
                    anchor: Optional[torch.Tensor] = None, return_logits: bool = True):
    """Markov-head correction of a draft block on the tensors' GPU (see sv_markov_draft in
    include/sv.h). base [B, K, V] float32 or bfloat16; left_factor, right_factor [V, R]
    bfloat16; anchor [B] int32 or None. Returns (tokens [B, K] int32, corrected logits
    [B, K, V] of base's dtype or None)."""
    lib = load_library()
    if base.dim() != 3:
        raise ValueError("base must be [B, K, V]")
    B, K, V = base.shape
    dev = base.device
    if dev.type != "cuda":
        raise ValueError("base must be a GPU tensor")
    _need(base, "base", base.dtype, (B, K, V), dev)
    if left_factor.dim() != 2:
        raise ValueError("left_factor must be [V, R]")
    R = left_factor.shape[1]
    _need(left_factor, "left_factor", torch.bfloat16, (V, R), dev)
    _need(right_factor, "right_factor", torch.bfloat16, (V, R), dev)
    if anchor is not None:
        _need(anchor, "anchor", torch.int32, (B,), dev)
    tokens = torch.empty(B, K, dtype=torch.int32, device=dev)
    out = torch.empty_like(base) if return_logits else None
    stream = torch.cuda.current_stream(dev).cuda_stream
    nbytes = int(lib.sv_markov_workspace_bytes(B, V))
    ws = _workspace(dev, stream, nbytes, "markov")
    _check(lib.sv_markov_draft(_ptr(base), _dtype_code(base), B, K, V, _ptr(left_factor),
                               _ptr(right_factor), R, _ptr(anchor), _ptr(tokens), _ptr(out),
                               _ptr(ws), ws.numel(), stream))
    return tokens, out


def sv_markov_draft_sampled(base: torch.Tensor, left_factor: torch.Tensor,
                            right_factor: torch.Tensor, temperature: torch.Tensor,
                            uniforms: torch.Tensor, anchor: Optional[torch.Tensor] = None):
    """Sampled Markov-head drafting on the tensors' GPU (see sv_markov_draft_sampled in
    include/sv.h). base [B, K, V] float32 or bfloat16; left_factor, right_factor [V, R]
    bfloat16; temperature [B] float32 (0: argmax); uniforms [B, K] float32; anchor [B] int32 or
    None. Returns (tokens [B, K] int32, draft logits [B, K, V] of base's dtype)."""
    lib = load_library()
    if base.dim() != 3:
        raise ValueError("base must be [B, K, V]")
    B, K, V = base.shape
    dev = base.device
    if dev.type != "cuda":
        raise ValueError("base must be a GPU tensor")
    _need(base, "base", base.dtype, (B, K, V), dev)
    if left_factor.dim() != 2:
        raise ValueError("left_factor must be [V, R]")
    R = left_factor.shape[1]
    _need(left_factor, "left_factor", torch.bfloat16, (V, R), dev)
    _need(right_factor, "right_factor", torch.bfloat16, (V, R), dev)
    _need(temperature, "temperature", torch.float32, (B,), dev)
    _need(uniforms, "uniforms", torch.float32, (B, K), dev)
    if anchor is not None:
        _need(anchor, "anchor", torch.int32, (B,), dev)
    tokens = torch.empty(B, K, dtype=torch.int32, device=dev)
    out = torch.empty_like(base)
    stream = torch.cuda.current_stream(dev).cuda_stream
    nbytes = int(lib.sv_markov_workspace_bytes(B, V))
    ws = _workspace(dev, stream, nbytes, "markov")
    _check(lib.sv_markov_draft_sampled(_ptr(base), _dtype_code(base), B, K, V, _ptr(left_factor),
                                       _ptr(right_factor), R, _ptr(anchor), _ptr(temperature),
                                       _ptr(uniforms), _ptr(tokens), _ptr(out), _ptr(ws),
                                       ws.numel(), stream))
    return tokens, out


class TopkOutput(NamedTuple):
    tokens: torch.Tensor  # [B, K] int32
    candidates: Optional[torch.Tensor]  # [B, K, kc] int32, ascending vocabulary index
    cand_logits: Optional[torch.Tensor]  # [B, K, kc] float32 corrected logits


def sv_markov_topk(base: torch.Tensor, left_factor: torch.Tensor, right_factor: torch.Tensor,
                   kc: int, anchor: Optional[torch.Tensor] = None,
                   return_candidates: bool = True) -> TopkOutput:
    """Top-K Markov drafting on the tensors' GPU (see sv_markov_topk in include/sv.h)."""
    lib = load_library()
    if base.dim() != 3:
        raise ValueError("base must be [B, K, V]")
    B, K, V = base.shape
    dev = base.device
    if dev.type != "cuda":
        raise ValueError("base must be a GPU tensor")
    _need(base, "base", base.dtype, (B, K, V), dev)
    if left_factor.dim() != 2:
        raise ValueError("left_factor must be [V, R]")
    R = left_factor.shape[1]
    _need(left_factor, "left_factor", torch.bfloat16, (V, R), dev)
    _need(right_factor, "right_factor", torch.bfloat16, (V, R), dev)
    if anchor is not None:
        _need(anchor, "anchor", torch.int32, (B,), dev)
    kc = int(kc)
    tokens = torch.empty(B, K, dtype=torch.int32, device=dev)
    cands = torch.empty(B, K, kc, dtype=torch.int32, device=dev) if return_candidates else None
    logits = torch.empty(B, K, kc, dtype=torch.float32, device=dev) if return_candidates else None
    stream = torch.cuda.current_stream(dev).cuda_stream
    nbytes = int(lib.sv_markov_topk_workspace_bytes(B, K, V))
    ws = _workspace(dev, stream, nbytes, "markov_topk")
    _check(lib.sv_markov_topk(_ptr(base), _dtype_code(base), B, K, V, _ptr(left_factor),
                              _ptr(right_factor), R, kc, _ptr(anchor), _ptr(tokens), _ptr(cands),
                              _ptr(logits), _ptr(ws), ws.numel(), stream))
    return TopkOutput(tokens, cands, logits)


def sv_read_probe(data: torch.Tensor, groups: int = 2048) -> torch.Tensor:
    """Read probe over a contiguous GPU tensor (see sv_read_probe in include/sv.h): every
    16-byte word read once with non-temporal loads. Returns the [groups] uint32 partial sums
    (as int32). Asynchronous on the current stream."""
    lib = load_library()
    if data.device.type != "cuda" or not data.is_contiguous():
        raise ValueError("data must be a contiguous GPU tensor")
    nbytes = data.numel() * data.element_size()
    out = torch.empty(groups, dtype=torch.int32, device=data.device)
    stream = torch.cuda.current_stream(data.device).cuda_stream
    _check(lib.sv_read_probe(_ptr(data), nbytes - nbytes % 16, _ptr(out), groups, stream))
    return out
