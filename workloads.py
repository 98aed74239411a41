"""Seeded synthetic inputs for exact attention, shared by the tests, the bench
and the smoke check.

This module draws random numbers and rounds them to the storage type; it holds
none of the attention arithmetic (no scores, no softmax, no products), so both
the CPU oracle's callers and the GPU path's callers can use it without the two
sharing any of the method's code.

Workloads: the five shapes are the ones the attention forward is measured on.
The pages fix no dataset (the FlashAttention-2 (PL) article quotes GPT-style
training, section "Wydajność i efektywność"), so every input is i.i.d. normal
noise of the stated shape, drawn from numpy's PCG64 with a fixed seed.

Draw order, per workload: Q, then K, then V, each ``standard_normal`` in float32
over the contiguous [B][H][N][d] shape; then the workload's transform (a scalar
multiplier, or one K channel scaled by 8 with the channel index drawn next from
the same generator); then round-to-nearest-even to the storage type.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np

DTYPES = ("f32", "f16", "bf16")


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    dtype: str
    B: int
    Hq: int
    Hkv: int
    N: int
    d: int
    causal: bool
    window_left: int  # -1 = no window
    seed: int
    value_mult: float = 1.0       # multiplier applied to Q, K and V before rounding
    k_outlier_mult: float = 0.0   # >0: one K channel (same for every row/head) times this

    @property
    def scale(self) -> float:
        """softmax scale 1/sqrt(d), as the float32 value handed to the kernel."""
        return float(np.float32(1.0 / math.sqrt(self.d)))

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


# The five measured shapes.  "tiny" is small enough for the oracle to finish in
# milliseconds; "causal_8k" is the headline (GPT-style training shape).
WORKLOADS = {
    "tiny_f32": Workload("tiny_f32", "f32", 1, 1, 1, 128, 64, False, -1, 0),
    "bf16_n1k_d64": Workload("bf16_n1k_d64", "bf16", 8, 16, 16, 1024, 64, False, -1, 1),
    "causal_8k": Workload("causal_8k", "bf16", 2, 16, 16, 8192, 128, True, -1, 2, value_mult=0.5),
    "gqa_f16_4k": Workload("gqa_f16_4k", "f16", 4, 32, 8, 4096, 128, True, -1, 3, k_outlier_mult=8.0),
    "swa_32k": Workload("swa_32k", "bf16", 1, 32, 32, 32768, 128, True, 4096, 4),
}
ORDER = ["tiny_f32", "bf16_n1k_d64", "causal_8k", "gqa_f16_4k", "swa_32k"]
HEADLINE = "causal_8k"


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 to the nearest bfloat16 (ties to even); returned as float32.

    NaN stays NaN (quiet); infinities stay infinite.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = (u + 0x7FFF + lsb) >> 16
    r = (r << 16).astype(np.uint32)
    nan = np.isnan(x)
    if nan.any():
        r[nan] = (x.view(np.uint32)[nan] | 0x00400000) & 0xFFFF0000
    return r.view(np.float32)


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """The 16-bit bfloat16 patterns of float32 values that are already bf16-exact."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    return (u >> 16).astype(np.uint16)


def round_to_f16(x: np.ndarray) -> np.ndarray:
    """Round float32 to the nearest float16 (numpy's conversion is ties-to-even)."""
    return np.asarray(x, dtype=np.float32).astype(np.float16).astype(np.float32)


def round_to(dtype: str, x: np.ndarray) -> np.ndarray:
    if dtype == "f32":
        return np.ascontiguousarray(x, dtype=np.float32)
    if dtype == "bf16":
        return round_to_bf16(x)
    if dtype == "f16":
        return round_to_f16(x)
    raise ValueError(dtype)


def make_inputs(w: Workload, *, N: Optional[int] = None, B: Optional[int] = None,
                Hq: Optional[int] = None, Hkv: Optional[int] = None, d: Optional[int] = None):
    """Draw (q, k, v) for workload ``w`` as float32 arrays whose values are exact
    in ``w.dtype``.  Keyword overrides shrink the shape (same seed and recipe)."""
    B = w.B if B is None else B
    Hq = w.Hq if Hq is None else Hq
    Hkv = w.Hkv if Hkv is None else Hkv
    N = w.N if N is None else N
    d = w.d if d is None else d
    rng = np.random.default_rng(w.seed)
    q = rng.standard_normal((B, Hq, N, d), dtype=np.float32)
    k = rng.standard_normal((B, Hkv, N, d), dtype=np.float32)
    v = rng.standard_normal((B, Hkv, N, d), dtype=np.float32)
    if w.value_mult != 1.0:
        m = np.float32(w.value_mult)
        q *= m
        k *= m
        v *= m
    if w.k_outlier_mult > 0.0 and d > 0:
        c = int(rng.integers(d))
        k[..., c] *= np.float32(w.k_outlier_mult)
    return round_to(w.dtype, q), round_to(w.dtype, k), round_to(w.dtype, v)


def random_inputs(seed: int, dtype: str, B: int, Hq: int, Hkv: int, N: int, d: int,
                  mult: float = 1.0):
    """Ad-hoc shapes for edge-case tests, same recipe as ``make_inputs``."""
    w = Workload("adhoc", dtype, B, Hq, Hkv, N, d, False, -1, seed, value_mult=mult)
    return make_inputs(w)


def make_grad(w: Workload, *, N: Optional[int] = None, B: Optional[int] = None,
              Hq: Optional[int] = None, d: Optional[int] = None):
    """Upstream gradient dO for the backward of workload ``w``: standard normal
    draws from the generator seeded with ``w.seed + 1000``, shaped like q,
    exact in ``w.dtype``."""
    B = w.B if B is None else B
    Hq = w.Hq if Hq is None else Hq
    N = w.N if N is None else N
    d = w.d if d is None else d
    rng = np.random.default_rng(w.seed + 1000)
    return round_to(w.dtype, rng.standard_normal((B, Hq, N, d), dtype=np.float32))


def random_grad(seed: int, dtype: str, B: int, Hq: int, N: int, d: int):
    """Ad-hoc upstream gradient, same recipe as ``make_grad``."""
    w = Workload("adhoc", dtype, B, Hq, Hq, N, d, False, -1, seed)
    return make_grad(w)


def bwd_metric_flops(w: Workload) -> float:
    """Algorithmic FLOPs of one backward pass: five products of the forward's
    size per visible pair (recompute S, dV, dP, dQ, dK), i.e. 2.5 x the
    forward's metric FLOPs."""
    return 2.5 * metric_flops(w)


# ---------------------------------------------------------------------------
# FP8 inputs (OCP E4M3: bias 7, 3 mantissa bits, no infinities, largest
# finite 448, subnormals down to 2^-9) with one float32 scale per tensor:
# the value a byte stands for is fp8(byte) * scale.

FP8_MAX = 448.0


def round_to_fp8(x: np.ndarray) -> np.ndarray:
    """Round to the nearest E4M3 value, ties to even (|x| must be <= 448)."""
    a = np.abs(np.asarray(x, dtype=np.float64))
    if (a > FP8_MAX).any():
        raise ValueError("value beyond the E4M3 range (scale the tensor first)")
    with np.errstate(divide="ignore"):
        e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    e = np.maximum(e, -6.0)                 # below 2^-6: subnormal spacing 2^-9
    ulp = np.exp2(e - 3.0)
    r = np.round(a / ulp) * ulp            # numpy rounds half to even
    return np.copysign(r, x)


def fp8_bits(x: np.ndarray) -> np.ndarray:
    """E4M3 byte of values already representable (the output of round_to_fp8)."""
    v = np.asarray(x, dtype=np.float64)
    a = np.abs(v)
    sign = (np.signbit(v)).astype(np.uint8) << 7
    with np.errstate(divide="ignore"):
        e = np.floor(np.log2(np.where(a > 0, a, 1.0))).astype(np.int64)
    normal = a >= 2.0 ** -6
    exp_field = np.where(normal, e + 7, 0)
    mant = np.where(normal, (a / np.exp2(e) - 1.0) * 8.0, a / 2.0 ** -9)
    bits = (exp_field << 3) | np.rint(mant).astype(np.int64)
    bits = np.where(a == 0, 0, bits)
    return (sign | bits.astype(np.uint8)).astype(np.uint8)


def quantize_fp8(x: np.ndarray):
    """Per-tensor quantisation: scale = max|x| / 448 (float32), bytes =
    E4M3(x / scale).  Returns (bytes uint8, scale float, dequantised float64
    values = fp8(bytes) * scale, which are what the method is fed)."""
    x = np.asarray(x, dtype=np.float32)
    amax = float(np.abs(x).max()) if x.size else 0.0
    scale = float(np.float32(amax / FP8_MAX)) if amax > 0 else 1.0
    q = round_to_fp8(np.clip(x.astype(np.float64) / scale, -FP8_MAX, FP8_MAX))
    return fp8_bits(q), scale, q * scale


FP8_WORKLOADS = {
    # the headline shape with FP8 inputs (same seed and recipe, then quantised)
    "causal_8k_fp8": Workload("causal_8k_fp8", "f32", 2, 16, 16, 8192, 128, True, -1, 2, value_mult=0.5),
}


def make_fp8_inputs(w: Workload, **over):
    """(q, k, v) as per-tensor FP8: three (bytes, scale, dequantised) triples,
    drawn with ``make_inputs`` of the float32 recipe, then quantised."""
    q, k, v = make_inputs(w.replace(dtype="f32"), **over)
    return quantize_fp8(q), quantize_fp8(k), quantize_fp8(v)


# ---------------------------------------------------------------------------
# Decoding: Nq query rows per sequence against a key/value cache of per-batch
# length (rows aligned to the end of the cache).  Same generator recipe:
# Q, K, V standard normal in float32 over [B][Hq][Nq][d] and [B][Hkv][Nk][d],
# then, for "uniform" lengths, B lengths drawn from integers(1, Nk + 1), then
# rounding to the storage type.  A paged cache scatters the same keys into
# pages of page_size slots in an order drawn from a generator seeded with
# seed + 2000.

@dataclasses.dataclass(frozen=True)
class DecodeWorkload:
    name: str
    dtype: str
    B: int
    Hq: int
    Hkv: int
    Nq: int
    Nk: int
    d: int
    causal: bool
    window_left: int
    seed: int
    lengths: str = "full"   # "full": every cache holds Nk keys; "uniform": lengths drawn in [1, Nk]
    page_size: int = 0      # 0: contiguous cache [B][Hkv][Nk][d]; else pages [pages][page_size][Hkv][d]

    @property
    def scale(self) -> float:
        return float(np.float32(1.0 / math.sqrt(self.d)))

    def replace(self, **kw) -> "DecodeWorkload":
        return dataclasses.replace(self, **kw)


DECODE_WORKLOADS = {
    # one new token per sequence, GQA 4:1, 32k-token caches
    "decode_gqa_32k": DecodeWorkload("decode_gqa_32k", "bf16", 8, 32, 8, 1, 32768, 128, True, -1, 5),
    # one new token, mixed cache lengths up to 16k, paged in 64-token pages
    "decode_paged_varlen": DecodeWorkload("decode_paged_varlen", "bf16", 16, 32, 8, 1, 16384, 128, True, -1, 6,
                                          lengths="uniform", page_size=64),
    # 16 new tokens per sequence (draft verification / chunked prefill) on 16k caches
    "verify_16_16k": DecodeWorkload("verify_16_16k", "bf16", 4, 32, 8, 16, 16384, 128, True, -1, 7),
}
DECODE_HEADLINE = "decode_gqa_32k"


def make_decode_inputs(w: DecodeWorkload, **over):
    """(q, k, v, seqlens) for a decoding workload: q [B][Hq][Nq][d], k, v
    [B][Hkv][Nk][d] float32 exact in w.dtype, seqlens int32 [B]."""
    w = w.replace(**over) if over else w
    rng = np.random.default_rng(w.seed)
    q = rng.standard_normal((w.B, w.Hq, w.Nq, w.d), dtype=np.float32)
    k = rng.standard_normal((w.B, w.Hkv, w.Nk, w.d), dtype=np.float32)
    v = rng.standard_normal((w.B, w.Hkv, w.Nk, w.d), dtype=np.float32)
    if w.lengths == "uniform":
        seqlens = rng.integers(1, w.Nk + 1, w.B).astype(np.int32)
    else:
        seqlens = np.full(w.B, w.Nk, dtype=np.int32)
    return round_to(w.dtype, q), round_to(w.dtype, k), round_to(w.dtype, v), seqlens


def build_pages(k: np.ndarray, v: np.ndarray, seqlens, page_size: int, seed: int, fill: float = 0.0,
                spare_pages: int = 0):
    """Scatter a contiguous cache k, v [B][Hkv][Nk][d] into token-major pages
    [num_pages][page_size][Hkv][d] in a seeded random page order.  Returns
    (k_pages, v_pages, block_table int32 [B][max_pages]).  Slots past a
    batch's length, pages no sequence uses (``spare_pages``) and table entries
    past the length get ``fill`` (the table: -1), so that a reader that
    touches them shows it."""
    B, Hkv, Nk, d = k.shape
    if page_size <= 0 or Nk % page_size:
        raise ValueError("Nk must be a positive multiple of page_size")
    max_pages = Nk // page_size
    num_pages = B * max_pages + spare_pages
    order = np.random.default_rng(seed + 2000).permutation(num_pages)
    kp = np.full((num_pages, page_size, Hkv, d), fill, dtype=np.float32)
    vp = np.full((num_pages, page_size, Hkv, d), fill, dtype=np.float32)
    table = np.full((B, max_pages), -1, dtype=np.int32)
    for b in range(B):
        L = int(seqlens[b])
        for j in range((L + page_size - 1) // page_size):
            page = int(order[b * max_pages + j])
            table[b, j] = page
            n = min(page_size, L - j * page_size)
            kp[page, :n] = k[b, :, j * page_size:j * page_size + n].transpose(1, 0, 2)
            vp[page, :n] = v[b, :, j * page_size:j * page_size + n].transpose(1, 0, 2)
    return kp, vp, table


def decode_bytes(w: DecodeWorkload, seqlens, elem: int = 2) -> int:
    """Bytes one decoding call must move at least: every visible cached key
    and value row once per key/value head (the union over the group's query
    rows), the query rows, and the output plus its logsumexp."""
    kv = 0
    for L in np.asarray(seqlens, dtype=np.int64):
        L = int(L)
        # union over the rows: the last row sees up to key L - 1 (with or
        # without the causal mask), the first row's window starts lowest
        lo = 0 if w.window_left < 0 else max(0, L - w.Nq - w.window_left)
        kv += max(0, L - lo)
    return (2 * kv * w.Hkv * w.d * elem + w.B * w.Hq * w.Nq * w.d * elem * 2 + w.B * w.Hq * w.Nq * 4)


# ---------------------------------------------------------------------------
# Packed sequences of different lengths (prefill of a mixed batch): B lengths
# drawn from integers(lo, hi + 1) by a generator seeded with the workload's
# seed, then Q, K, V standard normal in float32 over the packed shapes
# [total][H][d] from the same generator, rounded to the storage type.  Query
# and key counts are equal per sequence (self-attention).

@dataclasses.dataclass(frozen=True)
class VarlenWorkload:
    name: str
    dtype: str
    B: int
    Hq: int
    Hkv: int
    lo: int
    hi: int
    d: int
    causal: bool
    window_left: int
    seed: int

    @property
    def scale(self) -> float:
        return float(np.float32(1.0 / math.sqrt(self.d)))

    def replace(self, **kw) -> "VarlenWorkload":
        return dataclasses.replace(self, **kw)


VARLEN_WORKLOADS = {
    # 16 sequences of 512..8192 tokens, causal, MHA d=128 (a mixed training or prefill batch)
    "varlen_causal_16": VarlenWorkload("varlen_causal_16", "bf16", 16, 16, 16, 512, 8192, 128, True, -1, 8),
}


def make_varlen_inputs(w: VarlenWorkload, **over):
    """(q, k, v, cu_seqlens) for a packed workload: q [total][Hq][d], k, v
    [total][Hkv][d] float32 exact in w.dtype, cu_seqlens int32 [B+1]."""
    w = w.replace(**over) if over else w
    rng = np.random.default_rng(w.seed)
    lens = rng.integers(w.lo, w.hi + 1, w.B)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    total = int(cu[-1])
    q = rng.standard_normal((total, w.Hq, w.d), dtype=np.float32)
    k = rng.standard_normal((total, w.Hkv, w.d), dtype=np.float32)
    v = rng.standard_normal((total, w.Hkv, w.d), dtype=np.float32)
    return round_to(w.dtype, q), round_to(w.dtype, k), round_to(w.dtype, v), cu


def varlen_metric_flops(w: VarlenWorkload, cu) -> float:
    """4*d FLOPs per visible (query, key) pair per head, summed over the
    sequences (exact visible pairs: L(L+1)/2 per causal sequence)."""
    total = 0.0
    for a, b in zip(cu[:-1], cu[1:]):
        L = int(b - a)
        total += float(unmasked_pairs(L, w.causal, w.window_left))
    return 4.0 * w.Hq * w.d * total


def unmasked_pairs(N: int, causal: bool, window_left: int) -> int:
    """Number of (query i, key j) pairs that a causal and/or left-window mask
    keeps, per head: key j is kept when j <= i (if causal) and j >= i - wl
    (if wl >= 0)."""
    total = 0
    if not causal and window_left < 0:
        return N * N
    i = np.arange(N, dtype=np.int64)
    hi = i if causal else np.full(N, N - 1, dtype=np.int64)
    lo = np.maximum(0, i - window_left) if window_left >= 0 else np.zeros(N, dtype=np.int64)
    total = int(np.sum(hi - lo + 1))
    return total


def metric_flops(w: Workload) -> float:
    """FLOPs credited to one forward call: 4*d per kept (query, key) pair per
    head (2*d for the score, 2*d for the probability-weighted sum of V).
    Causal without a window counts N^2/2 pairs (the usual convention); a window
    counts the exact kept pairs."""
    if w.causal and w.window_left < 0:
        pairs = w.N * w.N / 2.0
    else:
        pairs = float(unmasked_pairs(w.N, w.causal, w.window_left))
    return 4.0 * w.B * w.Hq * w.d * pairs
