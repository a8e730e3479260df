"""Exact IO-aware attention for MI355X (gfx950): Python binding of ``libfa.so``.

The functions here carry the names of the C entry points in ``include/fa.h``
and only marshal arguments: they read shapes and strides off torch tensors,
allocate outputs with torch (device memory and streams are the only things
torch provides), and call the HIP library on the current torch stream. Every
step of the computation runs in the library's kernels; there is no CPU or
PyTorch fallback, and a missing library raises.

Tensor layout: [batch, heads, seqlen, head_dim] with unit stride along
head_dim (any other strides that are multiples of 16 bytes work).
"""
from __future__ import annotations

import ctypes
import math
from typing import Optional, Sequence

import torch

from . import _abi
from ._abi import FA_BF16, FA_FP32, FA_MASK_BLOCK, Params, Strides  # noqa: F401

__all__ = ["fa_fwd", "fa_bwd", "fa_bwd_noalloc", "fa_decode", "fa_bwd_workspace_size",
           "fa_decode_workspace_size",
           "fa_tile_log_words", "fa_strerror",
           "FAError", "make_params", "library"]


class FAError(RuntimeError):
    def __init__(self, status: int, where: str):
        lib = _abi.load()
        self.status = status
        detail = lib.fa_last_error_detail().decode()
        super().__init__(f"{where}: {lib.fa_strerror(status).decode()} (status {status})"
                         + (f": {detail}" if detail else ""))


def library() -> ctypes.CDLL:
    """The loaded HIP library (raises if it has not been built)."""
    return _abi.load()


def fa_strerror(status: int) -> str:
    return _abi.load().fa_strerror(status).decode()


_DT = {torch.bfloat16: FA_BF16, torch.float32: FA_FP32, torch.float8_e4m3fn: _abi.FA_FP8_E4M3}


def _strides(t: torch.Tensor) -> Strides:
    if t.dim() != 4:
        raise ValueError("tensors must be 4-D [batch, heads, seqlen, head_dim]")
    if t.stride(3) != 1:
        raise ValueError("head_dim must have unit stride")
    return Strides(t.stride(0), t.stride(1), t.stride(2))


def make_params(*, dtype=FA_BF16, o_dtype=None, batch, heads_q, heads_kv, seqlen, head_dim,
                scale=None, causal=False, seqlens_k=0, block_mask=0, block_mask_ld=0,
                window=None, dropout_p=0.0, dropout_seed=0, dropout_offset=0,
                descale=(1.0, 1.0, 1.0)) -> Params:
    """fa_params from plain values (device pointers as ints); ``window`` is
    None or a (left, right) sliding-window band; ``dropout_p`` (stored as
    float32), ``dropout_seed`` (uint64) and ``dropout_offset`` (uint32) select
    the in-kernel dropout; ``descale`` the (q, k, v) factors of FP8 inputs."""
    wl, wr = (0, 0) if window is None else (int(window[0]), int(window[1]))
    return Params(dtype, dtype if o_dtype is None else o_dtype, batch, heads_q, heads_kv, seqlen,
                  head_dim, 1.0 / math.sqrt(head_dim) if scale is None else scale, int(bool(causal)),
                  seqlens_k or None, block_mask or None, block_mask_ld,
                  int(window is not None), wl, wr, float(dropout_p), int(dropout_offset),
                  int(dropout_seed), float(descale[0]), float(descale[1]), float(descale[2]))


def _params_from(q, k, *, scale, causal, seqlens_k, block_mask, o_dtype, window,
                 dropout_p=0.0, dropout_seed=0, dropout_offset=0,
                 descale=(1.0, 1.0, 1.0)) -> Params:
    if q.dtype not in _DT:
        raise ValueError(f"unsupported dtype {q.dtype}")
    if k.dtype != q.dtype:
        raise ValueError("q, k, v must share a dtype")
    B, Hq, N, d = q.shape
    if k.shape[0] != B or k.shape[2] != N or k.shape[3] != d:
        raise ValueError("k/v shape does not match q")
    bm_ptr, bm_ld = 0, 0
    if block_mask is not None:
        if block_mask.dtype != torch.uint8 or block_mask.dim() != 2 or block_mask.stride(1) != 1:
            raise ValueError("block_mask must be a 2-D uint8 tensor with unit column stride")
        if block_mask.shape[0] < -(-N // FA_MASK_BLOCK):
            raise ValueError("block_mask has too few rows")
        bm_ptr, bm_ld = block_mask.data_ptr(), block_mask.stride(0)
    sl_ptr = 0
    if seqlens_k is not None:
        if seqlens_k.dtype != torch.int32 or seqlens_k.numel() < B or not seqlens_k.is_contiguous():
            raise ValueError("seqlens_k must be a contiguous int32 tensor of length >= batch")
        sl_ptr = seqlens_k.data_ptr()
    odt = _DT[q.dtype] if o_dtype is None else _DT[o_dtype]
    return make_params(dtype=_DT[q.dtype], o_dtype=odt, batch=B, heads_q=Hq, heads_kv=k.shape[1],
                       seqlen=N, head_dim=d, scale=scale, causal=causal, seqlens_k=sl_ptr,
                       block_mask=bm_ptr, block_mask_ld=bm_ld, window=window,
                       dropout_p=dropout_p, dropout_seed=dropout_seed,
                       dropout_offset=dropout_offset, descale=descale)


def _stream() -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _ptr(t: Optional[torch.Tensor]) -> ctypes.c_void_p:
    return ctypes.c_void_p(0 if t is None else t.data_ptr())


def fa_tile_log_words(params: Params) -> int:
    return _abi.load().fa_tile_log_words(ctypes.byref(params))


def fa_bwd_workspace_size(params: Params) -> int:
    return _abi.load().fa_bwd_workspace_size(ctypes.byref(params))


def fa_fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, *, scale: Optional[float] = None,
           causal: bool = False, seqlens_k: Optional[torch.Tensor] = None,
           block_mask: Optional[torch.Tensor] = None, o_dtype: Optional[torch.dtype] = None,
           out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
           tile_log: bool = False, window: Optional[tuple] = None, dropout_p: float = 0.0,
           dropout_seed: int = 0, dropout_offset: int = 0, descale=(1.0, 1.0, 1.0)):
    """Forward pass. Returns (O, LSE, tile_log or None).

    float8_e4m3fn q, k, v select the FP8 forward: ``descale`` gives the
    per-tensor (q, k, v) factors, and O defaults to bfloat16.
    """
    lib = _abi.load()
    fp8 = q.dtype == torch.float8_e4m3fn
    if fp8 and o_dtype is None:
        o_dtype = torch.bfloat16
    p = _params_from(q, k, scale=scale, causal=causal, seqlens_k=seqlens_k,
                     block_mask=block_mask, o_dtype=o_dtype, window=window,
                     dropout_p=dropout_p, dropout_seed=dropout_seed,
                     dropout_offset=dropout_offset, descale=descale)
    B, Hq, N, d = q.shape
    if out is None:
        out = torch.empty((B, Hq, N, d), dtype=o_dtype or q.dtype, device=q.device)
    if lse is None:
        lse = torch.empty((B, Hq, N), dtype=torch.float32, device=q.device)
    if not lse.is_contiguous() or lse.dtype != torch.float32 or lse.numel() != B * Hq * N:
        raise ValueError("lse must be a contiguous float32 [B, Hq, N] tensor")
    log = None
    if tile_log:
        log = torch.zeros(lib.fa_tile_log_words(ctypes.byref(p)), dtype=torch.int32,
                          device=q.device)
    st = lib.fa_fwd(ctypes.byref(p), _ptr(q), _strides(q), _ptr(k), _strides(k), _ptr(v),
                    _strides(v), _ptr(out), _strides(out), _ptr(lse), _ptr(log), _stream())
    if st != 0:
        raise FAError(st, "fa_fwd")
    return out, lse, log


def fa_bwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, o: torch.Tensor, lse: torch.Tensor,
           dout: torch.Tensor, *, scale: Optional[float] = None, causal: bool = False,
           seqlens_k: Optional[torch.Tensor] = None, block_mask: Optional[torch.Tensor] = None,
           dq: Optional[torch.Tensor] = None, dk: Optional[torch.Tensor] = None,
           dv: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
           tile_log: bool = False, stage_events: Optional[Sequence] = None,
           window: Optional[tuple] = None, dropout_p: float = 0.0, dropout_seed: int = 0,
           dropout_offset: int = 0):
    """Backward pass. Returns (dQ, dK, dV, tile_log or None).

    ``stage_events``: optional 3 ``torch.cuda.Event`` objects, recorded by
    the library before its dQ kernel, between it and the dK/dV kernel, and
    after that (for per-kernel timing). The
    dropout arguments must be those of the forward that produced ``o``.
    """
    lib = _abi.load()
    p = _params_from(q, k, scale=scale, causal=causal, seqlens_k=seqlens_k,
                     block_mask=block_mask, o_dtype=o.dtype, window=window,
                     dropout_p=dropout_p, dropout_seed=dropout_seed,
                     dropout_offset=dropout_offset)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    need = lib.fa_bwd_workspace_size(ctypes.byref(p))
    if workspace is None:
        workspace = torch.empty(need // 4 + 4, dtype=torch.float32, device=q.device)
    log = None
    if tile_log:
        log = torch.zeros(2 * lib.fa_tile_log_words(ctypes.byref(p)), dtype=torch.int32,
                          device=q.device)
    ev_arr = None
    if stage_events is not None:
        handles = []
        for ev in stage_events:
            if ev.cuda_event == 0:
                ev.record()  # materialise the underlying hipEvent_t
            handles.append(ev.cuda_event)
        if len(handles) != 3:
            raise ValueError("stage_events takes 3 events")
        ev_arr = (ctypes.c_void_p * 3)(*handles)
    st = lib.fa_bwd(ctypes.byref(p), _ptr(q), _strides(q), _ptr(k), _strides(k), _ptr(v),
                    _strides(v), _ptr(o), _strides(o), _ptr(dout), _strides(dout), _ptr(lse),
                    _ptr(dq), _strides(dq), _ptr(dk), _strides(dk), _ptr(dv), _strides(dv),
                    _ptr(workspace), workspace.numel() * workspace.element_size(), _ptr(log),
                    ctypes.cast(ev_arr, ctypes.c_void_p) if ev_arr is not None else None,
                    _stream())
    if st != 0:
        raise FAError(st, "fa_bwd")
    return dq, dk, dv, log


def fa_bwd_noalloc(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, o: torch.Tensor,
                   lse: torch.Tensor, dout: torch.Tensor, dq: torch.Tensor, dk: torch.Tensor,
                   dv: torch.Tensor, *, scale: Optional[float] = None, causal: bool = False,
                   seqlens_k: Optional[torch.Tensor] = None,
                   block_mask: Optional[torch.Tensor] = None,
                   tile_log: Optional[torch.Tensor] = None, window: Optional[tuple] = None,
                   dropout_p: float = 0.0, dropout_seed: int = 0, dropout_offset: int = 0):
    """Backward pass that allocates nothing: the caller passes the outputs
    (and, optionally, a caller-zeroed int32 tile log of
    2 * fa_tile_log_words words), and the library's fixed device array
    serves as workspace (up to FA_NOALLOC_WORKSPACE_BYTES). Calls that can
    overlap on one GPU share that array and race."""
    lib = _abi.load()
    p = _params_from(q, k, scale=scale, causal=causal, seqlens_k=seqlens_k,
                     block_mask=block_mask, o_dtype=o.dtype, window=window,
                     dropout_p=dropout_p, dropout_seed=dropout_seed,
                     dropout_offset=dropout_offset)
    st = lib.fa_bwd_noalloc(ctypes.byref(p), _ptr(q), _strides(q), _ptr(k), _strides(k), _ptr(v),
                            _strides(v), _ptr(o), _strides(o), _ptr(dout), _strides(dout),
                            _ptr(lse), _ptr(dq), _strides(dq), _ptr(dk), _strides(dk), _ptr(dv),
                            _strides(dv), _ptr(tile_log), None, _stream())
    if st != 0:
        raise FAError(st, "fa_bwd_noalloc")
    return dq, dk, dv


def fa_decode_workspace_size(params: Params) -> int:
    return _abi.load().fa_decode_workspace_size(ctypes.byref(params))


def fa_decode(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, *, scale: Optional[float] = None,
              seqlens_k: Optional[torch.Tensor] = None, o_dtype: Optional[torch.dtype] = None,
              out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
              workspace: Optional[torch.Tensor] = None):
    """Decode attention: q [B, Hq, 1, d] (one new row per head) against the
    cache k, v [B, Hkv, N, d]. Returns (O [B, Hq, 1, d], LSE [B, Hq])."""
    lib = _abi.load()
    if q.dim() != 4 or q.shape[2] != 1:
        raise ValueError("q must be [batch, heads_q, 1, head_dim]")
    if q.dtype != torch.bfloat16 or k.dtype != q.dtype or v.dtype != q.dtype:
        raise ValueError("decode takes bf16 q, k, v")
    B, Hq, _, d = q.shape
    if k.dim() != 4 or k.shape[0] != B or k.shape[3] != d or v.shape != k.shape:
        raise ValueError("k/v must be [batch, heads_kv, seqlen, head_dim] matching q")
    sl_ptr = 0
    if seqlens_k is not None:
        if seqlens_k.dtype != torch.int32 or seqlens_k.numel() < B or not seqlens_k.is_contiguous():
            raise ValueError("seqlens_k must be a contiguous int32 tensor of length >= batch")
        sl_ptr = seqlens_k.data_ptr()
    odt = FA_BF16 if o_dtype is None else _DT[o_dtype]
    p = make_params(dtype=FA_BF16, o_dtype=odt, batch=B, heads_q=Hq, heads_kv=k.shape[1],
                    seqlen=k.shape[2], head_dim=d, scale=scale, seqlens_k=sl_ptr)
    if out is None:
        out = torch.empty((B, Hq, 1, d), dtype=o_dtype or q.dtype, device=q.device)
    if lse is None:
        lse = torch.empty((B, Hq), dtype=torch.float32, device=q.device)
    if not lse.is_contiguous() or lse.dtype != torch.float32 or lse.numel() != B * Hq:
        raise ValueError("lse must be a contiguous float32 [B, Hq] tensor")
    need = lib.fa_decode_workspace_size(ctypes.byref(p))
    if need and workspace is None:
        workspace = torch.empty(need // 4 + 4, dtype=torch.float32, device=q.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib.fa_decode(ctypes.byref(p), _ptr(q), _strides(q), _ptr(k), _strides(k), _ptr(v),
                       _strides(v), _ptr(out), _strides(out), _ptr(lse), _ptr(workspace),
                       ws_bytes, _stream())
    if st != 0:
        raise FAError(st, "fa_decode")
    return out, lse
