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

# The torch-facing calls live in ``attention``, which imports torch; they are
# resolved on first use so that ``_lib`` (and the ABI checks built on it)
# works without importing torch.
_TORCH_API = ("fwd", "fwd_varlen", "fwd_fp8", "fwd_kvcache", "fwd_kvcache_paged", "kvcache_num_splits",
              "bwd", "bwd_varlen", "attend", "attend_varlen")


def __getattr__(name):
    if name in _TORCH_API:
        from . import attention
        return getattr(attention, name)
    raise AttributeError(f"module {__name__!r} has no attribute {name!r}")


__all__ = list(_TORCH_API) + ["FaError", "LIB_PATH", "load"]
