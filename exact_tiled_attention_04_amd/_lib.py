"""ctypes binding of libfa.so: the C entry points of include/fa.h under the
same names, taking raw device addresses (ints) and sizes.

Nothing here computes: each function marshals its arguments and calls the
library.  If libfa.so has not been built, the first call raises; there is no
fallback implementation.
"""
from __future__ import annotations

import ctypes
import os
import threading

# FA_LIB_PATH names another build of the same library (the host-sanitizer
# build the CPU tests run the C-ABI checks against); by default the in-tree one.
LIB_PATH = os.environ.get("FA_LIB_PATH") or os.path.join(os.path.dirname(os.path.abspath(__file__)), "libfa.so")

FA_DTYPE_F32, FA_DTYPE_F16, FA_DTYPE_BF16 = 0, 1, 2
DTYPE_CODES = {"f32": FA_DTYPE_F32, "f16": FA_DTYPE_F16, "bf16": FA_DTYPE_BF16}

FA_OK = 0
FA_ERR_INVALID_ARG = -1
FA_ERR_UNSUPPORTED = -2
FA_ERR_MISALIGNED = -3
FA_ERR_HIP = -4

EXPORTED = ["fa_fwd", "fa_fwd_bf16", "fa_fwd_f16", "fa_fwd_f32", "fa_fwd_varlen", "fa_fwd_fp8", "fa_fwd_kvcache",
            "fa_fwd_kvcache_paged", "fa_fwd_kvcache_paged_noalloc", "fa_fwd_kvcache_num_splits", "fa_fwd_kvcache_num_splits_for_lengths",
            "fa_fwd_kvcache_workspace_size", "fa_bwd", "fa_bwd_varlen",
            "fa_bwd_bf16", "fa_bwd_f16", "fa_bwd_workspace_size", "fa_status_string", "fa_last_error", "fa_version"]

_lock = threading.Lock()
_lib = None


class FaError(RuntimeError):
    """A libfa call returned a negative status."""

    def __init__(self, status: int, detail: str):
        self.status = status
        super().__init__(f"{fa_status_string(status)} ({status}): {detail}")


def load() -> ctypes.CDLL:
    global _lib
    if _lib is not None:
        return _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built: run `python -m exact_tiled_attention_04_amd.build`")
        lib = ctypes.CDLL(LIB_PATH)
        P, I, F = ctypes.c_void_p, ctypes.c_int, ctypes.c_float
        fwd_args = [P, P, P, P, P, I, I, I, I, I, I, I, F, P]
        for name in ("fa_fwd_bf16", "fa_fwd_f16", "fa_fwd_f32"):
            fn = getattr(lib, name)
            fn.argtypes = fwd_args
            fn.restype = I
        lib.fa_fwd.argtypes = fwd_args + [I]
        lib.fa_fwd.restype = I
        lib.fa_fwd_varlen.argtypes = [P, P, P, P, P, P, P, I, I, I, I, I, I, I, I, I, I, F, P, I]
        lib.fa_fwd_varlen.restype = I
        lib.fa_fwd_fp8.argtypes = [P, P, P, F, F, F, P, P, I, I, I, I, I, I, I, F, P]
        lib.fa_fwd_fp8.restype = I
        lib.fa_fwd_kvcache.argtypes = [P, P, P, P, P, P, P, I, I, I, I, I, I, I, I, F, I, P, I]
        lib.fa_fwd_kvcache.restype = I
        lib.fa_fwd_kvcache_paged.argtypes = [P, P, P, P, P, P, P, P, I, I, I, I, I, I, I, I, I, I, F, I, P, I]
        lib.fa_fwd_kvcache_paged_noalloc.restype = I
        lib.fa_fwd_kvcache_paged_noalloc.argtypes = [P, P, P, P, P, P, P, I, I, I, I, I, I, I, I, I, I, F, I, P, I]
        lib.fa_fwd_kvcache_paged.restype = I
        lib.fa_fwd_kvcache_num_splits.argtypes = [I, I, I, I, I]
        lib.fa_fwd_kvcache_num_splits.restype = I
        lib.fa_fwd_kvcache_num_splits_for_lengths.argtypes = [I, I, I, I, I, I, I, P]
        lib.fa_fwd_kvcache_num_splits_for_lengths.restype = I
        lib.fa_fwd_kvcache_workspace_size.argtypes = [I, I, I, I, I, I, I]
        lib.fa_fwd_kvcache_workspace_size.restype = ctypes.c_size_t
        bwd_args = [P, P, P, P, P, P, P, P, P, P, I, I, I, I, I, I, I, F, P]
        for name in ("fa_bwd_bf16", "fa_bwd_f16"):
            fn = getattr(lib, name)
            fn.argtypes = bwd_args
            fn.restype = I
        lib.fa_bwd.argtypes = bwd_args + [I]
        lib.fa_bwd.restype = I
        lib.fa_bwd_varlen.argtypes = [P] * 12 + [I] * 10 + [F, P, I]
        lib.fa_bwd_varlen.restype = I
        lib.fa_bwd_workspace_size.argtypes = [I, I, I]
        lib.fa_bwd_workspace_size.restype = ctypes.c_size_t
        lib.fa_status_string.argtypes = [I]
        lib.fa_status_string.restype = ctypes.c_char_p
        lib.fa_last_error.argtypes = []
        lib.fa_last_error.restype = ctypes.c_char_p
        lib.fa_version.argtypes = []
        lib.fa_version.restype = I
        _lib = lib
    return _lib


def _ptr(x):
    return None if x is None or x == 0 else ctypes.c_void_p(int(x))


def fa_fwd(q, k, v, o, lse, B, Hq, Hkv, N, d, causal, window_left, scale, stream, dtype) -> int:
    return load().fa_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, Hq, Hkv, N, d,
                         int(bool(causal)), window_left, scale, _ptr(stream), dtype)


def fa_fwd_bf16(q, k, v, o, lse, B, Hq, Hkv, N, d, causal, window_left, scale, stream) -> int:
    return load().fa_fwd_bf16(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, Hq, Hkv, N, d,
                              int(bool(causal)), window_left, scale, _ptr(stream))


def fa_fwd_f16(q, k, v, o, lse, B, Hq, Hkv, N, d, causal, window_left, scale, stream) -> int:
    return load().fa_fwd_f16(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, Hq, Hkv, N, d,
                             int(bool(causal)), window_left, scale, _ptr(stream))


def fa_fwd_f32(q, k, v, o, lse, B, Hq, Hkv, N, d, causal, window_left, scale, stream) -> int:
    return load().fa_fwd_f32(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, Hq, Hkv, N, d,
                             int(bool(causal)), window_left, scale, _ptr(stream))


def fa_fwd_varlen(q, k, v, o, lse, cu_seqlens_q, cu_seqlens_k, B, Hq, Hkv, total_q, total_k, max_seqlen_q,
                  max_seqlen_k, d, causal, window_left, scale, stream, dtype) -> int:
    return load().fa_fwd_varlen(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(cu_seqlens_q),
                                _ptr(cu_seqlens_k), B, Hq, Hkv, total_q, total_k, max_seqlen_q, max_seqlen_k, d,
                                int(bool(causal)), window_left, scale, _ptr(stream), dtype)


def fa_fwd_fp8(q, k, v, q_scale, k_scale, v_scale, o, lse, B, Hq, Hkv, N, d, causal, window_left, scale,
               stream) -> int:
    return load().fa_fwd_fp8(_ptr(q), _ptr(k), _ptr(v), q_scale, k_scale, v_scale, _ptr(o), _ptr(lse), B, Hq, Hkv,
                             N, d, int(bool(causal)), window_left, scale, _ptr(stream))


def fa_fwd_kvcache(q, k_cache, v_cache, cache_seqlens, o, lse, workspace, B, Hq, Hkv, Nq, Nk, d, causal,
                   window_left, scale, num_splits, stream, dtype) -> int:
    return load().fa_fwd_kvcache(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(cache_seqlens), _ptr(o), _ptr(lse),
                                 _ptr(workspace), B, Hq, Hkv, Nq, Nk, d, int(bool(causal)), window_left, scale,
                                 num_splits, _ptr(stream), dtype)


def fa_fwd_kvcache_paged(q, k_pages, v_pages, block_table, cache_seqlens, o, lse, workspace, B, Hq, Hkv, Nq, d,
                         num_pages, page_size, max_pages_per_seq, causal, window_left, scale, num_splits, stream,
                         dtype) -> int:
    return load().fa_fwd_kvcache_paged(_ptr(q), _ptr(k_pages), _ptr(v_pages), _ptr(block_table),
                                       _ptr(cache_seqlens), _ptr(o), _ptr(lse), _ptr(workspace), B, Hq, Hkv, Nq, d,
                                       num_pages, page_size, max_pages_per_seq, int(bool(causal)), window_left,
                                       scale, num_splits, _ptr(stream), dtype)


def fa_fwd_kvcache_paged_noalloc(q, k_pages, v_pages, block_table, cache_seqlens, o, lse, B, Hq, Hkv, Nq, d,
                                 num_pages, page_size, max_pages_per_seq, causal, window_left, scale, num_splits,
                                 stream, dtype) -> int:
    return load().fa_fwd_kvcache_paged_noalloc(_ptr(q), _ptr(k_pages), _ptr(v_pages), _ptr(block_table),
                                               _ptr(cache_seqlens), _ptr(o), _ptr(lse), B, Hq, Hkv, Nq, d, num_pages,
                                               page_size, max_pages_per_seq, int(bool(causal)), window_left, scale,
                                               num_splits, _ptr(stream), dtype)


def fa_fwd_kvcache_num_splits(B: int, Hq: int, Hkv: int, Nq: int, Nk: int) -> int:
    return load().fa_fwd_kvcache_num_splits(B, Hq, Hkv, Nq, Nk)


def fa_fwd_kvcache_num_splits_for_lengths(B: int, Hq: int, Hkv: int, Nq: int, Nk: int, causal: int,
                                          window_left: int, seqlens_host_addr: int) -> int:
    return load().fa_fwd_kvcache_num_splits_for_lengths(B, Hq, Hkv, Nq, Nk, causal, window_left, seqlens_host_addr)


def fa_fwd_kvcache_workspace_size(B: int, Hq: int, Hkv: int, Nq: int, Nk: int, d: int, num_splits: int) -> int:
    return load().fa_fwd_kvcache_workspace_size(B, Hq, Hkv, Nq, Nk, d, num_splits)


def fa_bwd(q, k, v, o, lse, dout, dq, dk, dv, workspace, B, Hq, Hkv, N, d, causal, window_left, scale, stream,
           dtype) -> int:
    return load().fa_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(dout), _ptr(dq), _ptr(dk), _ptr(dv),
                         _ptr(workspace), B, Hq, Hkv, N, d, int(bool(causal)), window_left, scale, _ptr(stream),
                         dtype)


def fa_bwd_varlen(q, k, v, o, lse, dout, dq, dk, dv, workspace, cu_seqlens_q, cu_seqlens_k, B, Hq, Hkv, total_q,
                  total_k, max_seqlen_q, max_seqlen_k, d, causal, window_left, scale, stream, dtype) -> int:
    return load().fa_bwd_varlen(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(dout), _ptr(dq), _ptr(dk),
                                _ptr(dv), _ptr(workspace), _ptr(cu_seqlens_q), _ptr(cu_seqlens_k), B, Hq, Hkv,
                                total_q, total_k, max_seqlen_q, max_seqlen_k, d, int(bool(causal)), window_left,
                                scale, _ptr(stream), dtype)


def fa_bwd_bf16(q, k, v, o, lse, dout, dq, dk, dv, workspace, B, Hq, Hkv, N, d, causal, window_left, scale,
                stream) -> int:
    return load().fa_bwd_bf16(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(dout), _ptr(dq), _ptr(dk),
                              _ptr(dv), _ptr(workspace), B, Hq, Hkv, N, d, int(bool(causal)), window_left, scale,
                              _ptr(stream))


def fa_bwd_f16(q, k, v, o, lse, dout, dq, dk, dv, workspace, B, Hq, Hkv, N, d, causal, window_left, scale,
               stream) -> int:
    return load().fa_bwd_f16(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(dout), _ptr(dq), _ptr(dk),
                             _ptr(dv), _ptr(workspace), B, Hq, Hkv, N, d, int(bool(causal)), window_left, scale,
                             _ptr(stream))


def fa_bwd_workspace_size(B: int, Hq: int, N: int) -> int:
    return load().fa_bwd_workspace_size(B, Hq, N)


def fa_status_string(status: int) -> str:
    return load().fa_status_string(status).decode()


def fa_last_error() -> str:
    return load().fa_last_error().decode()


def fa_version() -> int:
    return load().fa_version()
