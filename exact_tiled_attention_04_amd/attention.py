"""torch-facing wrapper over the C ABI: torch supplies device memory and the
current stream; every step of the computation runs in libfa's HIP kernels."""
from __future__ import annotations

import math
from typing import Optional, Tuple

import torch

from . import _lib

_DTYPES = {torch.float32: _lib.FA_DTYPE_F32, torch.float16: _lib.FA_DTYPE_F16,
           torch.bfloat16: _lib.FA_DTYPE_BF16}


def fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, causal: bool = False,
        window_left: int = -1, scale: Optional[float] = None, out: Optional[torch.Tensor] = None,
        lse: Optional[torch.Tensor] = None, want_lse: bool = True,
        stream: Optional[torch.cuda.Stream] = None) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """Exact attention forward on the GPU.

    q: [B, Hq, N, d]; k, v: [B, Hkv, N, d]; contiguous, one dtype (float32,
    float16 or bfloat16), on one GPU.  Returns (o, lse): o like q, lse float32
    [B, Hq, N] (None when want_lse is False and no lse buffer is given).
    The call is asynchronous on ``stream`` (default: the current stream).
    Raises _lib.FaError when the library rejects the arguments.
    """
    if q.dim() != 4 or k.dim() != 4 or v.dim() != 4:
        raise ValueError("q, k, v must be [B, H, N, d]")
    if q.dtype not in _DTYPES or k.dtype != q.dtype or v.dtype != q.dtype:
        raise ValueError(f"q, k, v must share one dtype of {list(_DTYPES)}")
    if not (q.is_cuda and k.device == q.device and v.device == q.device):
        raise ValueError("q, k, v must be on one GPU")
    if not (q.is_contiguous() and k.is_contiguous() and v.is_contiguous()):
        raise ValueError("q, k, v must be contiguous")
    B, Hq, N, d = q.shape
    if tuple(k.shape) != (B, k.shape[1], N, d) or k.shape != v.shape:
        raise ValueError("k and v must be [B, Hkv, N, d] with q's B, N, d")
    Hkv = k.shape[1]
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    o = out if out is not None else torch.empty_like(q)
    if o.shape != q.shape or o.dtype != q.dtype or not o.is_contiguous() or o.device != q.device:
        raise ValueError("out must be a contiguous tensor like q")
    if lse is None and want_lse:
        lse = torch.empty((B, Hq, N), dtype=torch.float32, device=q.device)
    if lse is not None and (lse.shape != (B, Hq, N) or lse.dtype != torch.float32
                            or not lse.is_contiguous() or lse.device != q.device):
        raise ValueError("lse must be a contiguous float32 [B, Hq, N] tensor")
    s = stream if stream is not None else torch.cuda.current_stream(q.device)
    with torch.cuda.device(q.device):
        status = _lib.fa_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                             lse.data_ptr() if lse is not None else None,
                             B, Hq, Hkv, N, d, causal, window_left, float(scale), s.cuda_stream,
                             _DTYPES[q.dtype])
    if status != _lib.FA_OK:
        raise _lib.FaError(status, _lib.fa_last_error())
    return o, lse


def fwd_varlen(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, cu_seqlens_q: torch.Tensor,
               cu_seqlens_k: torch.Tensor, max_seqlen_q: int, max_seqlen_k: int, causal: bool = False,
               window_left: int = -1, scale: Optional[float] = None, out: Optional[torch.Tensor] = None,
               lse: Optional[torch.Tensor] = None, want_lse: bool = True,
               stream: Optional[torch.cuda.Stream] = None) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """Attention over packed sequences of different lengths: q [total_q, Hq,
    d], k, v [total_k, Hkv, d] (float16 or bfloat16, contiguous), cu_seqlens_q
    and cu_seqlens_k int32 [B+1] offsets on the GPU, max_seqlen_q and
    max_seqlen_k the longest lengths.  Each sequence's query rows stand at the
    end of its keys.  Returns (o like q, lse float32 [Hq, total_q]).
    Asynchronous on ``stream``.  The library writes only the rows it
    computes; when this function allocates o and lse, the rows no sequence
    owns (and rows beyond max_seqlen_q) hold o = 0 and lse = -inf."""
    if q.dim() != 3 or k.dim() != 3 or k.shape != v.shape or k.shape[2] != q.shape[2]:
        raise ValueError("q must be [total_q, Hq, d] and k, v [total_k, Hkv, d]")
    if q.dtype not in (torch.float16, torch.bfloat16) or k.dtype != q.dtype or v.dtype != q.dtype:
        raise ValueError("q, k, v must share one dtype, float16 or bfloat16")
    if not (q.is_cuda and k.device == q.device and v.device == q.device):
        raise ValueError("q, k, v must be on one GPU")
    if not (q.is_contiguous() and k.is_contiguous() and v.is_contiguous()):
        raise ValueError("q, k, v must be contiguous")
    cq = _int32_dev(cu_seqlens_q, q.device, "cu_seqlens_q")
    ck = _int32_dev(cu_seqlens_k, q.device, "cu_seqlens_k")
    if cq is None or ck is None or cq.dim() != 1 or cq.shape != ck.shape or cq.numel() < 1:
        raise ValueError("cu_seqlens_q and cu_seqlens_k must be int32 [B+1]")
    total_q, Hq, d = q.shape
    total_k, Hkv, _ = k.shape
    B = cq.numel() - 1
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    s = stream if stream is not None else torch.cuda.current_stream(q.device)
    with torch.cuda.stream(s):
        # rows the library does not compute must not read as uninitialised memory
        o = out if out is not None else torch.zeros_like(q)
        if lse is None and want_lse:
            lse = torch.full((Hq, total_q), float("-inf"), dtype=torch.float32, device=q.device)
    if o.shape != q.shape or o.dtype != q.dtype or not o.is_contiguous() or o.device != q.device:
        raise ValueError("out must be a contiguous tensor like q")
    if lse is not None and (lse.shape != (Hq, total_q) or lse.dtype != torch.float32
                            or not lse.is_contiguous() or lse.device != q.device):
        raise ValueError("lse must be a contiguous float32 [Hq, total_q] tensor")
    with torch.cuda.device(q.device):
        status = _lib.fa_fwd_varlen(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                                    lse.data_ptr() if lse is not None else None, cq.data_ptr(), ck.data_ptr(),
                                    B, Hq, Hkv, total_q, total_k, int(max_seqlen_q), int(max_seqlen_k), d, causal,
                                    window_left, float(scale), s.cuda_stream, _DTYPES[q.dtype])
    if status != _lib.FA_OK:
        raise _lib.FaError(status, _lib.fa_last_error())
    return o, lse


_BYTE_TYPES = (torch.uint8, torch.float8_e4m3fn)


def fwd_fp8(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, q_scale: float, k_scale: float, v_scale: float,
            causal: bool = False, window_left: int = -1, scale: Optional[float] = None,
            out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None, want_lse: bool = True,
            stream: Optional[torch.cuda.Stream] = None) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """Exact attention forward on FP8 (E4M3) inputs with per-tensor scales.

    q: [B, Hq, N, d]; k, v: [B, Hkv, N, d]; contiguous torch.float8_e4m3fn
    (or uint8 holding the same bytes) on one GPU; element x stands for
    e4m3(x) * x_scale.  Returns (o, lse): o bfloat16 shaped like q, lse
    float32 [B, Hq, N] (None when want_lse is False and no lse is given).
    Asynchronous on ``stream`` (default: the current stream).  Raises
    _lib.FaError when the library rejects the arguments.
    """
    if q.dim() != 4 or k.dim() != 4 or v.dim() != 4:
        raise ValueError("q, k, v must be [B, H, N, d]")
    if any(t.dtype not in _BYTE_TYPES for t in (q, k, v)):
        raise ValueError("q, k, v must be float8_e4m3fn (or uint8 bytes)")
    if not (q.is_cuda and k.device == q.device and v.device == q.device):
        raise ValueError("q, k, v must be on one GPU")
    if not (q.is_contiguous() and k.is_contiguous() and v.is_contiguous()):
        raise ValueError("q, k, v must be contiguous")
    B, Hq, N, d = q.shape
    if tuple(k.shape) != (B, k.shape[1], N, d) or k.shape != v.shape:
        raise ValueError("k and v must be [B, Hkv, N, d] with q's B, N, d")
    Hkv = k.shape[1]
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    o = out if out is not None else torch.empty(q.shape, dtype=torch.bfloat16, device=q.device)
    if o.shape != q.shape or o.dtype != torch.bfloat16 or not o.is_contiguous() or o.device != q.device:
        raise ValueError("out must be a contiguous bfloat16 tensor shaped like q")
    if lse is None and want_lse:
        lse = torch.empty((B, Hq, N), dtype=torch.float32, device=q.device)
    if lse is not None and (lse.shape != (B, Hq, N) or lse.dtype != torch.float32
                            or not lse.is_contiguous() or lse.device != q.device):
        raise ValueError("lse must be a contiguous float32 [B, Hq, N] tensor")
    s = stream if stream is not None else torch.cuda.current_stream(q.device)
    with torch.cuda.device(q.device):
        status = _lib.fa_fwd_fp8(q.data_ptr(), k.data_ptr(), v.data_ptr(), float(q_scale), float(k_scale),
                                 float(v_scale), o.data_ptr(), lse.data_ptr() if lse is not None else None,
                                 B, Hq, Hkv, N, d, causal, window_left, float(scale), s.cuda_stream)
    if status != _lib.FA_OK:
        raise _lib.FaError(status, _lib.fa_last_error())
    return o, lse


def _kv_common(q, k, v, out, lse, want_lse, workspace, B, Hq, Hkv, Nq, Nk, d, num_splits, stream):
    if q.dtype not in (torch.float16, torch.bfloat16) or k.dtype != q.dtype or v.dtype != q.dtype:
        raise ValueError("q, k, v must share one dtype, float16 or bfloat16")
    if not (q.is_cuda and k.device == q.device and v.device == q.device):
        raise ValueError("q, k, v must be on one GPU")
    if not (q.is_contiguous() and k.is_contiguous() and v.is_contiguous()):
        raise ValueError("q, k, v must be contiguous")
    o = out if out is not None else torch.empty_like(q)
    if o.shape != q.shape or o.dtype != q.dtype or not o.is_contiguous() or o.device != q.device:
        raise ValueError("out must be a contiguous tensor like q")
    if lse is None and want_lse:
        lse = torch.empty((B, Hq, Nq), dtype=torch.float32, device=q.device)
    if lse is not None and (lse.shape != (B, Hq, Nq) or lse.dtype != torch.float32
                            or not lse.is_contiguous() or lse.device != q.device):
        raise ValueError("lse must be a contiguous float32 [B, Hq, Nq] tensor")
    nbytes = _lib.fa_fwd_kvcache_workspace_size(B, Hq, Hkv, Nq, Nk, d, num_splits)
    if workspace is None and nbytes > 0:
        workspace = torch.empty(nbytes // 4, dtype=torch.float32, device=q.device)
    if workspace is not None and (workspace.dtype != torch.float32 or workspace.numel() * 4 < nbytes
                                  or not workspace.is_contiguous()):
        raise ValueError(f"workspace must be a contiguous float32 tensor of at least {nbytes} bytes")
    s = stream if stream is not None else torch.cuda.current_stream(q.device)
    return o, lse, workspace, s


def kvcache_num_splits(cache_seqlens, Hq: int, Hkv: int, Nq: int, Nk: int, causal: bool = False,
                       window_left: int = -1) -> int:
    """The split count ``fa_fwd_kvcache_num_splits_for_lengths`` picks for
    caches of these lengths (a host sequence or CPU tensor of B ints; Nk is
    the capacity, page_size * pages per sequence for a paged cache)."""
    import numpy as np
    lens = np.ascontiguousarray(np.asarray(cache_seqlens.cpu() if isinstance(cache_seqlens, torch.Tensor)
                                           else cache_seqlens, dtype=np.int32).reshape(-1))
    return _lib.fa_fwd_kvcache_num_splits_for_lengths(len(lens), Hq, Hkv, Nq, Nk, int(causal), window_left,
                                                      lens.ctypes.data)


def _int32_dev(x, device, name):
    if x is None:
        return None
    if not (isinstance(x, torch.Tensor) and x.dtype == torch.int32 and x.device == device and x.is_contiguous()):
        raise ValueError(f"{name} must be a contiguous int32 tensor on the GPU of q")
    return x


def fwd_kvcache(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                cache_seqlens: Optional[torch.Tensor] = None, causal: bool = False, window_left: int = -1,
                scale: Optional[float] = None, num_splits: int = 0, out: Optional[torch.Tensor] = None,
                lse: Optional[torch.Tensor] = None, want_lse: bool = True,
                workspace: Optional[torch.Tensor] = None,
                stream: Optional[torch.cuda.Stream] = None) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """Attention of q [B, Hq, Nq, d] against a contiguous cache k_cache,
    v_cache [B, Hkv, Nk, d] whose batch b holds cache_seqlens[b] keys (int32
    on the GPU; None: all Nk).  Query rows stand at the end of the cache.
    Returns (o like q, lse float32 [B, Hq, Nq]); rows that see no key get
    o = 0, lse = -inf.  num_splits = 0 lets the library choose.  The split
    workspace is allocated here unless given.  Asynchronous on ``stream``.
    """
    if q.dim() != 4 or k_cache.dim() != 4 or v_cache.dim() != 4 or k_cache.shape != v_cache.shape:
        raise ValueError("q must be [B, Hq, Nq, d] and k_cache, v_cache [B, Hkv, Nk, d]")
    B, Hq, Nq, d = q.shape
    _, Hkv, Nk, dk = k_cache.shape
    if k_cache.shape[0] != B or dk != d:
        raise ValueError("k_cache, v_cache must be [B, Hkv, Nk, d] with q's B and d")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    seq = _int32_dev(cache_seqlens, q.device, "cache_seqlens")
    o, lse, ws, s = _kv_common(q, k_cache, v_cache, out, lse, want_lse, workspace, B, Hq, Hkv, Nq, Nk, d,
                               num_splits, stream)
    with torch.cuda.device(q.device):
        status = _lib.fa_fwd_kvcache(q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(),
                                     seq.data_ptr() if seq is not None else None, o.data_ptr(),
                                     lse.data_ptr() if lse is not None else None,
                                     ws.data_ptr() if ws is not None else None, B, Hq, Hkv, Nq, Nk, d, causal,
                                     window_left, float(scale), num_splits, s.cuda_stream, _DTYPES[q.dtype])
    if status != _lib.FA_OK:
        raise _lib.FaError(status, _lib.fa_last_error())
    return o, lse


def fwd_kvcache_paged(q: torch.Tensor, k_pages: torch.Tensor, v_pages: torch.Tensor, block_table: torch.Tensor,
                      cache_seqlens: torch.Tensor, causal: bool = False, window_left: int = -1,
                      scale: Optional[float] = None, num_splits: int = 0, out: Optional[torch.Tensor] = None,
                      lse: Optional[torch.Tensor] = None, want_lse: bool = True,
                      workspace: Optional[torch.Tensor] = None,
                      stream: Optional[torch.cuda.Stream] = None) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """As ``fwd_kvcache`` on a paged cache: k_pages, v_pages [num_pages,
    page_size, Hkv, d]; block_table int32 [B, max_pages_per_seq] of page
    indices; cache_seqlens int32 [B] (required)."""
    if q.dim() != 4 or k_pages.dim() != 4 or k_pages.shape != v_pages.shape:
        raise ValueError("q must be [B, Hq, Nq, d] and k_pages, v_pages [num_pages, page_size, Hkv, d]")
    B, Hq, Nq, d = q.shape
    num_pages, page_size, Hkv, dk = k_pages.shape
    if dk != d:
        raise ValueError("pages must have q's head dimension")
    if block_table is None or block_table.dim() != 2 or block_table.shape[0] != B:
        raise ValueError("block_table must be int32 [B, max_pages_per_seq]")
    if cache_seqlens is None or cache_seqlens.shape != (B,):
        raise ValueError("cache_seqlens must be int32 [B]")
    bt = _int32_dev(block_table, q.device, "block_table")
    seq = _int32_dev(cache_seqlens, q.device, "cache_seqlens")
    max_pages = bt.shape[1]
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    o, lse, ws, s = _kv_common(q, k_pages, v_pages, out, lse, want_lse, workspace, B, Hq, Hkv, Nq,
                               page_size * max_pages, d, num_splits, stream)
    with torch.cuda.device(q.device):
        status = _lib.fa_fwd_kvcache_paged(q.data_ptr(), k_pages.data_ptr(), v_pages.data_ptr(), bt.data_ptr(),
                                           seq.data_ptr(), o.data_ptr(), lse.data_ptr() if lse is not None else None,
                                           ws.data_ptr() if ws is not None else None, B, Hq, Hkv, Nq, d, num_pages,
                                           page_size, max_pages, causal, window_left, float(scale), num_splits,
                                           s.cuda_stream, _DTYPES[q.dtype])
    if status != _lib.FA_OK:
        raise _lib.FaError(status, _lib.fa_last_error())
    return o, lse


def bwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, o: torch.Tensor, lse: torch.Tensor,
        dout: torch.Tensor, causal: bool = False, window_left: int = -1, scale: Optional[float] = None,
        dq: Optional[torch.Tensor] = None, dk: Optional[torch.Tensor] = None, dv: Optional[torch.Tensor] = None,
        workspace: Optional[torch.Tensor] = None,
        stream: Optional[torch.cuda.Stream] = None) -> Tuple[torch.Tensor, torch.Tensor, torch.Tensor]:
    """Gradients of ``fwd``'s output with respect to q, k and v on the GPU.

    q, k, v, causal, window_left, scale: as passed to ``fwd``; o, lse: what
    ``fwd`` returned for them; dout: upstream gradient like o.  Only float16
    and bfloat16 are supported.  Returns (dq, dk, dv) like (q, k, v).  The
    float32 workspace (``_lib.fa_bwd_workspace_size`` bytes) is allocated here
    unless given.  Asynchronous on ``stream`` (default: the current stream).
    Raises _lib.FaError when the library rejects the arguments.
    """
    ts = (q, k, v, o, dout)
    if any(t.dim() != 4 for t in ts):
        raise ValueError("q, k, v, o, dout must be [B, H, N, d]")
    if q.dtype not in (torch.float16, torch.bfloat16) or any(t.dtype != q.dtype for t in ts):
        raise ValueError("q, k, v, o, dout must share one dtype, float16 or bfloat16")
    if not q.is_cuda or any(t.device != q.device for t in ts + (lse,)):
        raise ValueError("all tensors must be on one GPU")
    if not all(t.is_contiguous() for t in ts + (lse,)):
        raise ValueError("all tensors must be contiguous")
    B, Hq, N, d = q.shape
    if tuple(k.shape) != (B, k.shape[1], N, d) or k.shape != v.shape:
        raise ValueError("k and v must be [B, Hkv, N, d] with q's B, N, d")
    if o.shape != q.shape or dout.shape != q.shape:
        raise ValueError("o and dout must be shaped like q")
    if lse.shape != (B, Hq, N) or lse.dtype != torch.float32:
        raise ValueError("lse must be float32 [B, Hq, N]")
    Hkv = k.shape[1]
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    dq = dq if dq is not None else torch.empty_like(q)
    dk = dk if dk is not None else torch.empty_like(k)
    dv = dv if dv is not None else torch.empty_like(v)
    for name, g, ref in (("dq", dq, q), ("dk", dk, k), ("dv", dv, v)):
        if g.shape != ref.shape or g.dtype != ref.dtype or not g.is_contiguous() or g.device != q.device:
            raise ValueError(f"{name} must be a contiguous tensor like its input")
    nbytes = _lib.fa_bwd_workspace_size(B, Hq, N)
    if workspace is None:
        workspace = torch.empty(max(1, nbytes // 4), dtype=torch.float32, device=q.device)
    if workspace.dtype != torch.float32 or workspace.numel() * 4 < nbytes or not workspace.is_contiguous():
        raise ValueError(f"workspace must be a contiguous float32 tensor of at least {nbytes} bytes")
    s = stream if stream is not None else torch.cuda.current_stream(q.device)
    with torch.cuda.device(q.device):
        status = _lib.fa_bwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                             dout.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), workspace.data_ptr(),
                             B, Hq, Hkv, N, d, causal, window_left, float(scale), s.cuda_stream, _DTYPES[q.dtype])
    if status != _lib.FA_OK:
        raise _lib.FaError(status, _lib.fa_last_error())
    return dq, dk, dv


def bwd_varlen(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, o: torch.Tensor, lse: torch.Tensor,
               dout: torch.Tensor, cu_seqlens_q: torch.Tensor, cu_seqlens_k: torch.Tensor, max_seqlen_q: int,
               max_seqlen_k: int, causal: bool = False, window_left: int = -1, scale: Optional[float] = None,
               dq: Optional[torch.Tensor] = None, dk: Optional[torch.Tensor] = None,
               dv: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
               stream: Optional[torch.cuda.Stream] = None) -> Tuple[torch.Tensor, torch.Tensor, torch.Tensor]:
    """Gradients of ``fwd_varlen``'s output with respect to q, k and v.

    q, k, v, cu_seqlens_q/k, max_seqlen_q/k, causal, window_left, scale: as
    passed to ``fwd_varlen``; o, lse: what it returned; dout: upstream
    gradient like o.  Returns (dq, dk, dv) like (q, k, v); rows outside
    every sequence are left as the given (or freshly allocated) tensors hold
    them.  Asynchronous on ``stream``; raises _lib.FaError when the library
    rejects the arguments."""
    ts = (q, k, v, o, dout)
    if q.dim() != 3 or k.dim() != 3 or k.shape != v.shape or k.shape[2] != q.shape[2]:
        raise ValueError("q must be [total_q, Hq, d] and k, v [total_k, Hkv, d]")
    if o.shape != q.shape or dout.shape != q.shape:
        raise ValueError("o and dout must be shaped like q")
    if q.dtype not in (torch.float16, torch.bfloat16) or any(t.dtype != q.dtype for t in ts):
        raise ValueError("q, k, v, o, dout must share one dtype, float16 or bfloat16")
    if not q.is_cuda or any(t.device != q.device for t in ts + (lse,)):
        raise ValueError("all tensors must be on one GPU")
    if not all(t.is_contiguous() for t in ts + (lse,)):
        raise ValueError("all tensors must be contiguous")
    cq = _int32_dev(cu_seqlens_q, q.device, "cu_seqlens_q")
    ck = _int32_dev(cu_seqlens_k, q.device, "cu_seqlens_k")
    if cq is None or ck is None or cq.dim() != 1 or cq.shape != ck.shape or cq.numel() < 1:
        raise ValueError("cu_seqlens_q and cu_seqlens_k must be int32 [B+1]")
    total_q, Hq, d = q.shape
    total_k, Hkv, _ = k.shape
    if lse.shape != (Hq, total_q) or lse.dtype != torch.float32:
        raise ValueError("lse must be float32 [Hq, total_q]")
    B = cq.numel() - 1
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    dq = dq if dq is not None else torch.zeros_like(q)
    dk = dk if dk is not None else torch.zeros_like(k)
    dv = dv if dv is not None else torch.zeros_like(v)
    for name, g, ref in (("dq", dq, q), ("dk", dk, k), ("dv", dv, v)):
        if g.shape != ref.shape or g.dtype != ref.dtype or not g.is_contiguous() or g.device != q.device:
            raise ValueError(f"{name} must be a contiguous tensor like its input")
    nbytes = _lib.fa_bwd_workspace_size(1, Hq, total_q)
    if workspace is None:
        workspace = torch.empty(max(1, nbytes // 4), dtype=torch.float32, device=q.device)
    if workspace.dtype != torch.float32 or workspace.numel() * 4 < nbytes or not workspace.is_contiguous():
        raise ValueError(f"workspace must be a contiguous float32 tensor of at least {nbytes} bytes")
    s = stream if stream is not None else torch.cuda.current_stream(q.device)
    with torch.cuda.device(q.device):
        status = _lib.fa_bwd_varlen(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                                    dout.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(),
                                    workspace.data_ptr(), cq.data_ptr(), ck.data_ptr(), B, Hq, Hkv, total_q,
                                    total_k, int(max_seqlen_q), int(max_seqlen_k), d, causal, window_left,
                                    float(scale), s.cuda_stream, _DTYPES[q.dtype])
    if status != _lib.FA_OK:
        raise _lib.FaError(status, _lib.fa_last_error())
    return dq, dk, dv


class _Attention(torch.autograd.Function):
    """``fwd`` as a differentiable torch operation: the forward saves q, k, v,
    o and lse, the backward calls ``bwd`` with them."""

    @staticmethod
    def forward(ctx, q, k, v, causal, window_left, scale):
        o, lse = fwd(q, k, v, causal=causal, window_left=window_left, scale=scale)
        ctx.save_for_backward(q, k, v, o, lse)
        ctx.args = (causal, window_left, scale)
        ctx.mark_non_differentiable(lse)
        return o, lse

    @staticmethod
    def backward(ctx, dout, _dlse):
        q, k, v, o, lse = ctx.saved_tensors
        causal, window_left, scale = ctx.args
        dq, dk, dv = bwd(q, k, v, o, lse, dout.contiguous(), causal=causal, window_left=window_left, scale=scale)
        return dq, dk, dv, None, None, None


def attend(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, causal: bool = False, window_left: int = -1,
           scale: Optional[float] = None) -> torch.Tensor:
    """Differentiable exact attention: returns o like ``fwd`` and, when a loss
    built on it is backpropagated, the gradients of q, k and v from ``bwd``
    (float16/bfloat16; the logsumexp the backward needs is kept internally).
    """
    o, _ = _Attention.apply(q, k, v, causal, window_left, scale)
    return o


class _AttentionVarlen(torch.autograd.Function):
    """``fwd_varlen`` as a differentiable torch operation: the forward saves
    q, k, v, o, lse and the offsets, the backward calls ``bwd_varlen``."""

    @staticmethod
    def forward(ctx, q, k, v, cu_seqlens_q, cu_seqlens_k, max_seqlen_q, max_seqlen_k, causal, window_left, scale):
        o, lse = fwd_varlen(q, k, v, cu_seqlens_q, cu_seqlens_k, max_seqlen_q, max_seqlen_k, causal=causal,
                            window_left=window_left, scale=scale)
        ctx.save_for_backward(q, k, v, o, lse, cu_seqlens_q, cu_seqlens_k)
        ctx.args = (max_seqlen_q, max_seqlen_k, causal, window_left, scale)
        ctx.mark_non_differentiable(lse)
        return o, lse

    @staticmethod
    def backward(ctx, dout, _dlse):
        q, k, v, o, lse, cq, ck = ctx.saved_tensors
        max_q, max_k, causal, window_left, scale = ctx.args
        dq, dk, dv = bwd_varlen(q, k, v, o, lse, dout.contiguous(), cq, ck, max_q, max_k, causal=causal,
                                window_left=window_left, scale=scale)
        return dq, dk, dv, None, None, None, None, None, None, None


def attend_varlen(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, cu_seqlens_q: torch.Tensor,
                  cu_seqlens_k: torch.Tensor, max_seqlen_q: int, max_seqlen_k: int, causal: bool = False,
                  window_left: int = -1, scale: Optional[float] = None) -> torch.Tensor:
    """Differentiable attention over packed sequences: returns o like
    ``fwd_varlen`` and, under backpropagation, the gradients of q, k and v
    from ``bwd_varlen`` (rows outside every sequence get zero gradients).
    cu_seqlens_q/k must be int32 tensors on q's GPU."""
    o, _ = _AttentionVarlen.apply(q, k, v, cu_seqlens_q, cu_seqlens_k, int(max_seqlen_q), int(max_seqlen_k), causal,
                                  window_left, scale)
    return o
