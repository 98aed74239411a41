"""Exact attention forward and backward (IO-aware, tiled, online softmax) for
AMD MI355X.

The computation lives in ``libfa.so`` (HIP kernels for gfx950 behind the C ABI
of ``include/fa.h``).  This package is a thin binding:

    _lib        the C entry points under their C names (raw addresses, sizes)
    attention   ``fwd(q, k, v, causal, window_left, scale)``,
                ``fwd_varlen(q, k, v, cu_seqlens_q, cu_seqlens_k, ...)``,
                ``fwd_fp8(q8, k8, v8, q_scale, k_scale, v_scale, ...)``,
                ``fwd_kvcache(q, k_cache, v_cache, cache_seqlens, ...)``,
                ``fwd_kvcache_paged(q, k_pages, v_pages, block_table, ...)`` and
                ``bwd(q, k, v, o, lse, dout, ...)``,
                ``bwd_varlen(q, k, v, o, lse, dout, cu_seqlens_q, ...)`` on
                torch tensors, and
                ``attend(q, k, v, ...)`` / ``attend_varlen(...)``, the
                forwards as differentiable torch operations whose backwards
                are ``bwd`` / ``bwd_varlen``
    build       compiles libfa.so in-tree with hipcc
"""
from ._lib import FaError, LIB_PATH, load  # noqa: F401


def fwd(*args, **kwargs):
    from .attention import fwd as _fwd
    return _fwd(*args, **kwargs)


def fwd_varlen(*args, **kwargs):
    from .attention import fwd_varlen as _f
    return _f(*args, **kwargs)


def fwd_fp8(*args, **kwargs):
    from .attention import fwd_fp8 as _fwd_fp8
    return _fwd_fp8(*args, **kwargs)


def fwd_kvcache(*args, **kwargs):
    from .attention import fwd_kvcache as _f
    return _f(*args, **kwargs)


def fwd_kvcache_paged(*args, **kwargs):
    from .attention import fwd_kvcache_paged as _f
    return _f(*args, **kwargs)


def kvcache_num_splits(*args, **kwargs):
    from .attention import kvcache_num_splits as _f
    return _f(*args, **kwargs)


def bwd(*args, **kwargs):
    from .attention import bwd as _bwd
    return _bwd(*args, **kwargs)


def bwd_varlen(*args, **kwargs):
    from .attention import bwd_varlen as _f
    return _f(*args, **kwargs)


def attend_varlen(*args, **kwargs):
    from .attention import attend_varlen as _a
    return _a(*args, **kwargs)


def attend(*args, **kwargs):
    from .attention import attend as _a
    return _a(*args, **kwargs)


__all__ = ["fwd", "fwd_varlen", "fwd_fp8", "fwd_kvcache", "fwd_kvcache_paged", "kvcache_num_splits", "bwd", "bwd_varlen",
           "attend", "attend_varlen", "FaError",
           "LIB_PATH", "load"]
