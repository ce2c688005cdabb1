"""Exact IO-aware attention for MI355X (gfx950): Python binding.

The functions here carry the names of the C ABI (include/fa.h) and only
marshal arguments: they check tensor dtype/device/shape, allocate outputs with
torch (device memory is plumbing), take the current HIP stream, and call the
library.  Every step of the computation runs in the library's HIP kernels;
there is no other implementation, and importing this package fails if the
library has not been built.

Tensors are contiguous [B, H, N, d] on a GPU; ``lse`` is [B, H, N] float32.
"""

from __future__ import annotations

import contextlib
import math
from typing import Optional, Tuple

import numpy as np
import torch

from ._lib import LIB, FAError, FA_OK, FA_BWD_NOALLOC_MAX_ROWS, status_str  # noqa: F401

__all__ = [
    "fa_fwd", "fa_fwd_split_max", "fa_fwd_split", "fa_merge", "fa_bwd", "fa_bwd_noalloc", "fa_bwd_workspace_bytes", "fa_bwd_preprocess", "fa_bwd_dkdv",
    "fa_bwd_dq", "fa_f32_key_block", "fa_fwd_f32", "fa_bwd_f32", "fa_bwd_f32_workspace_bytes",
    "default_scale", "FAError", "status_str", "forward", "backward",
]


def default_scale(d: int) -> float:
    """1/sqrt(d) rounded once to fp32."""
    return float(np.float32(1.0 / math.sqrt(d)))


def _check(status: int, where: str) -> None:
    if status != FA_OK:
        raise FAError(status, where)


def _shape4(x: torch.Tensor, name: str, dtype: torch.dtype):
    if not isinstance(x, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if x.device.type != "cuda":
        raise ValueError(f"{name} must be on a GPU (got {x.device})")
    if x.dtype != dtype:
        raise TypeError(f"{name} must be {dtype} (got {x.dtype})")
    if x.dim() != 4:
        raise ValueError(f"{name} must be [B, H, N, d] (got {tuple(x.shape)})")
    if not x.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return tuple(x.shape)


def _same(shape, x: torch.Tensor, name: str, dtype: torch.dtype, dev: torch.device):
    if _shape4(x, name, dtype) != shape:
        raise ValueError(f"{name} has shape {tuple(x.shape)}, expected {shape}")
    if x.device != dev:
        raise ValueError(f"{name} is on {x.device}, the other tensors on {dev}")


def _rows(x: torch.Tensor, name: str, shape, dev: torch.device) -> None:
    B, H, N, _ = shape
    if not isinstance(x, torch.Tensor) or x.device != dev or x.dtype != torch.float32 \
            or tuple(x.shape) != (B, H, N) or not x.is_contiguous():
        raise ValueError(f"{name} must be a contiguous float32 [B, H, N] tensor on {dev}")


def _on(dev: torch.device):
    """Device context of a call.  The default stream's handle (0) means the
    null stream of the current device, so a call on another device's tensors
    makes that device current for the call."""
    if dev.index is None or dev.index == torch.cuda.current_device():
        return contextlib.nullcontext()
    return torch.cuda.device(dev)


def _stream(dev: torch.device, stream) -> int:
    if stream is None:
        stream = torch.cuda.current_stream(dev)
    return int(stream.cuda_stream) if hasattr(stream, "cuda_stream") else int(stream)


def _ptr(x: Optional[torch.Tensor]) -> int:
    return 0 if x is None else int(x.data_ptr())


def _fwd(fn, where, dtype, q, k, v, scale, o, lse, stream):
    shape = _shape4(q, "q", dtype)
    dev = q.device
    _same(shape, k, "k", dtype, dev)
    _same(shape, v, "v", dtype, dev)
    B, H, N, d = shape
    if scale is None:
        scale = default_scale(d)
    if o is None:
        o = torch.empty_like(q)
    else:
        _same(shape, o, "o", dtype, dev)
    if lse is None:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    else:
        _rows(lse, "lse", shape, dev)
    with _on(dev):
        _check(fn(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, H, N, d, float(scale),
                  _stream(q.device, stream)), where)
    return o, lse


def fa_fwd(q, k, v, scale: Optional[float] = None, o=None, lse=None, stream=None
           ) -> Tuple[torch.Tensor, torch.Tensor]:
    """bf16 forward.  Returns (o, lse); o bf16 [B,H,N,d], lse fp32 [B,H,N]."""
    return _fwd(LIB.fa_fwd, "fa_fwd", torch.bfloat16, q, k, v, scale, o, lse, stream)


def fa_fwd_split_max(B: int, H: int, N: int, d: int) -> int:
    """Largest key-range count fa_fwd_split accepts (-1 for an invalid shape)."""
    return int(LIB.fa_fwd_split_max(B, H, N, d))


def fa_fwd_split(q, k, v, n_split: int, scale: Optional[float] = None, o_part=None,
                 lse_part=None, stream=None) -> Tuple[torch.Tensor, torch.Tensor]:
    """Split-KV forward.  Returns (o_part fp32 [n_split,B,H,N,d], lse_part fp32
    [n_split,B,H,N]): each key range's own normalised output and LSE."""
    shape = _shape4(q, "q", torch.bfloat16)
    dev = q.device
    _same(shape, k, "k", torch.bfloat16, dev)
    _same(shape, v, "v", torch.bfloat16, dev)
    B, H, N, d = shape
    if scale is None:
        scale = default_scale(d)
    n = int(n_split)
    if o_part is None:
        o_part = torch.empty((max(n, 0), B, H, N, d), dtype=torch.float32, device=q.device)
    if lse_part is None:
        lse_part = torch.empty((max(n, 0), B, H, N), dtype=torch.float32, device=q.device)
    _parts(o_part, lse_part, n, shape, dev)
    with _on(dev):
        _check(LIB.fa_fwd_split(_ptr(q), _ptr(k), _ptr(v), _ptr(o_part), _ptr(lse_part),
                                B, H, N, d, float(scale), n, _stream(q.device, stream)),
               "fa_fwd_split")
    return o_part, lse_part


def fa_merge(o_part, lse_part, o=None, lse=None, stream=None
             ) -> Tuple[torch.Tensor, torch.Tensor]:
    """Merge of partial results.  o_part fp32 [P,B,H,N,d], lse_part fp32
    [P,B,H,N]; returns (o bf16 [B,H,N,d], lse fp32 [B,H,N])."""
    if not isinstance(o_part, torch.Tensor) or o_part.dim() != 5:
        raise ValueError("o_part must be a [P, B, H, N, d] tensor")
    n = int(o_part.shape[0])
    shape = tuple(o_part.shape[1:])
    dev = o_part.device
    _parts(o_part, lse_part, n, shape, dev)
    B, H, N, d = shape
    if o is None:
        o = torch.empty(shape, dtype=torch.bfloat16, device=o_part.device)
    else:
        _same(shape, o, "o", torch.bfloat16, dev)
    if lse is None:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=o_part.device)
    else:
        _rows(lse, "lse", shape, dev)
    with _on(dev):
        _check(LIB.fa_merge(_ptr(o_part), _ptr(lse_part), n, _ptr(o), _ptr(lse), B, H, N, d,
                            _stream(o_part.device, stream)), "fa_merge")
    return o, lse


def _parts(o_part, lse_part, n: int, shape, dev: torch.device) -> None:
    for x, name, tail in ((o_part, "o_part", tuple(shape)), (lse_part, "lse_part", tuple(shape[:3]))):
        if not isinstance(x, torch.Tensor) or x.device.type != "cuda":
            raise ValueError(f"{name} must be a GPU tensor")
        if x.device != dev:
            raise ValueError(f"{name} is on {x.device}, the other tensors on {dev}")
        if x.dtype != torch.float32 or not x.is_contiguous():
            raise ValueError(f"{name} must be contiguous float32")
        if tuple(x.shape) != (max(n, 0),) + tail:
            raise ValueError(f"{name} has shape {tuple(x.shape)}, expected {(n,) + tail}")


def fa_fwd_f32(q, k, v, scale: Optional[float] = None, o=None, lse=None, stream=None
               ) -> Tuple[torch.Tensor, torch.Tensor]:
    """fp32 forward.  Returns (o, lse).  Keys per rescale step:
    fa_f32_key_block(N, d)."""
    return _fwd(LIB.fa_fwd_f32, "fa_fwd_f32", torch.float32, q, k, v, scale, o, lse, stream)


def fa_f32_key_block(N: int, d: int) -> int:
    """Keys per rescale step of the fp32 calls at this shape (8 or 32; -1
    for an invalid shape)."""
    return int(LIB.fa_f32_key_block(N, d))


def fa_bwd_workspace_bytes(B: int, H: int, N: int, d: int) -> int:
    return int(LIB.fa_bwd_workspace_bytes(B, H, N, d))


def fa_bwd_f32_workspace_bytes(B: int, H: int, N: int, d: int) -> int:
    return int(LIB.fa_bwd_f32_workspace_bytes(B, H, N, d))


def _bwd(fn, wsfn, where, dtype, q, k, v, o, lse, dO, scale, dq, dk, dv, workspace, stream):
    shape = _shape4(q, "q", dtype)
    dev = q.device
    for x, name in ((k, "k"), (v, "v"), (o, "o"), (dO, "dO")):
        _same(shape, x, name, dtype, dev)
    _rows(lse, "lse", shape, dev)
    B, H, N, d = shape
    if scale is None:
        scale = default_scale(d)
    outs = []
    for x, name in ((dq, "dq"), (dk, "dk"), (dv, "dv")):
        if x is None:
            x = torch.empty_like(q)
        else:
            _same(shape, x, name, dtype, dev)
        outs.append(x)
    dq, dk, dv = outs
    need = int(wsfn(B, H, N, d))
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    elif not isinstance(workspace, torch.Tensor) or workspace.device != dev \
            or not workspace.is_contiguous():
        raise ValueError(f"workspace must be a contiguous tensor on {dev}")
    ws_bytes = workspace.numel() * workspace.element_size()
    with _on(dev):
        _check(fn(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(dO), _ptr(dq), _ptr(dk),
                  _ptr(dv), _ptr(workspace), ws_bytes, B, H, N, d, float(scale),
                  _stream(q.device, stream)), where)
    return dq, dk, dv


def fa_bwd(q, k, v, o, lse, dO, scale: Optional[float] = None, dq=None, dk=None, dv=None,
           workspace=None, stream=None):
    """bf16 backward with recomputation.  Returns (dq, dk, dv)."""
    return _bwd(LIB.fa_bwd, LIB.fa_bwd_workspace_bytes, "fa_bwd", torch.bfloat16, q, k, v, o,
                lse, dO, scale, dq, dk, dv, workspace, stream)


def fa_bwd_noalloc(q, k, v, o, lse, dO, scale: Optional[float] = None, dq=None, dk=None,
                   dv=None, stream=None):
    """bf16 backward whose workspace is the library's fixed device array
    (B*H*N <= FA_BWD_NOALLOC_MAX_ROWS); the C call allocates nothing.  Pass
    dq, dk, dv to make this call allocate nothing either.  Calls that overlap
    in time on one GPU race.  Returns (dq, dk, dv)."""
    shape = _shape4(q, "q", torch.bfloat16)
    dev = q.device
    for x, name in ((k, "k"), (v, "v"), (o, "o"), (dO, "dO")):
        _same(shape, x, name, torch.bfloat16, dev)
    _rows(lse, "lse", shape, dev)
    B, H, N, d = shape
    if scale is None:
        scale = default_scale(d)
    outs = []
    for x, name in ((dq, "dq"), (dk, "dk"), (dv, "dv")):
        if x is None:
            x = torch.empty_like(q)
        else:
            _same(shape, x, name, torch.bfloat16, dev)
        outs.append(x)
    dq, dk, dv = outs
    with _on(dev):
        _check(LIB.fa_bwd_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(dO),
                                  _ptr(dq), _ptr(dk), _ptr(dv), B, H, N, d, float(scale),
                                  _stream(q.device, stream)), "fa_bwd_noalloc")
    return dq, dk, dv


def fa_bwd_f32(q, k, v, o, lse, dO, scale: Optional[float] = None, dq=None, dk=None, dv=None,
               workspace=None, stream=None):
    """fp32 backward.  Returns (dq, dk, dv)."""
    return _bwd(LIB.fa_bwd_f32, LIB.fa_bwd_f32_workspace_bytes, "fa_bwd_f32", torch.float32,
                q, k, v, o, lse, dO, scale, dq, dk, dv, workspace, stream)


def fa_bwd_preprocess(o, dO, delta=None, stream=None):
    """Stage 1 of fa_bwd: delta = rowsum(dO * o), fp32 [B,H,N]."""
    shape = _shape4(o, "o", torch.bfloat16)
    dev = o.device
    _same(shape, dO, "dO", torch.bfloat16, dev)
    B, H, N, d = shape
    if delta is None:
        delta = torch.empty((B, H, N), dtype=torch.float32, device=o.device)
    else:
        _rows(delta, "delta", shape, dev)
    with _on(dev):
        _check(LIB.fa_bwd_preprocess(_ptr(o), _ptr(dO), _ptr(delta), B, H, N, d,
                                     _stream(o.device, stream)), "fa_bwd_preprocess")
    return delta


def fa_bwd_dkdv(q, k, v, lse, dO, delta, scale: Optional[float] = None, dk=None, dv=None,
                stream=None):
    """Stage 2 of fa_bwd.  Returns (dk, dv)."""
    shape = _shape4(q, "q", torch.bfloat16)
    dev = q.device
    for x, name in ((k, "k"), (v, "v"), (dO, "dO")):
        _same(shape, x, name, torch.bfloat16, dev)
    _rows(lse, "lse", shape, dev)
    _rows(delta, "delta", shape, dev)
    B, H, N, d = shape
    if scale is None:
        scale = default_scale(d)
    dk = torch.empty_like(q) if dk is None else dk
    dv = torch.empty_like(q) if dv is None else dv
    _same(shape, dk, "dk", torch.bfloat16, dev)
    _same(shape, dv, "dv", torch.bfloat16, dev)
    with _on(dev):
        _check(LIB.fa_bwd_dkdv(_ptr(q), _ptr(k), _ptr(v), _ptr(lse), _ptr(dO), _ptr(delta),
                               _ptr(dk), _ptr(dv), B, H, N, d, float(scale),
                               _stream(q.device, stream)), "fa_bwd_dkdv")
    return dk, dv


def fa_bwd_dq(q, k, v, lse, dO, delta, scale: Optional[float] = None, dq=None, stream=None):
    """Stage 3 of fa_bwd.  Returns dq."""
    shape = _shape4(q, "q", torch.bfloat16)
    dev = q.device
    for x, name in ((k, "k"), (v, "v"), (dO, "dO")):
        _same(shape, x, name, torch.bfloat16, dev)
    _rows(lse, "lse", shape, dev)
    _rows(delta, "delta", shape, dev)
    B, H, N, d = shape
    if scale is None:
        scale = default_scale(d)
    dq = torch.empty_like(q) if dq is None else dq
    _same(shape, dq, "dq", torch.bfloat16, dev)
    with _on(dev):
        _check(LIB.fa_bwd_dq(_ptr(q), _ptr(k), _ptr(v), _ptr(lse), _ptr(dO), _ptr(delta),
                             _ptr(dq), B, H, N, d, float(scale), _stream(q.device, stream)),
               "fa_bwd_dq")
    return dq


# Short names for the two calls of the hot path: forward(q, k, v, scale=None)
# -> (o, lse) and backward(q, k, v, o, lse, dO, scale=None) -> (dq, dk, dv),
# bf16; a non-OK status raises FAError (a RuntimeError).
forward = fa_fwd
backward = fa_bwd
