"""CPU tests of the C ABI: the library loads, exports every entry point the
header declares, and rejects bad arguments on the host with the documented
status, before any device work (no call here reaches a kernel launch)."""
from __future__ import annotations

import ctypes
import os
import re

import pytest

from exact_tiled_attention_04_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fa.h")

pytestmark = pytest.mark.skipif(not os.path.exists(_lib.LIB_PATH),
                                reason="libfa.so not built (run __graft_entry__.build())")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(fa_\w+)\s*\(", src)))


def test_header_declares_the_documented_entry_points():
    assert declared_functions() == sorted(_lib.EXPORTED)


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(_lib.LIB_PATH)
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_status_strings_and_version():
    assert _lib.fa_status_string(0) == "FA_OK"
    assert _lib.fa_status_string(-1) == "FA_ERR_INVALID_ARG"
    assert _lib.fa_status_string(-2) == "FA_ERR_UNSUPPORTED"
    assert _lib.fa_status_string(-3) == "FA_ERR_MISALIGNED"
    assert _lib.fa_status_string(-4) == "FA_ERR_HIP"
    assert _lib.fa_status_string(7) == "FA_UNKNOWN_STATUS"
    assert _lib.fa_version() >= 100


# Fake, well-aligned, non-overlapping "device addresses": every case below
# fails validation before the library touches them.
Q, K, V, O, L = 0x100000, 0x200000, 0x300000, 0x400000, 0x500000
GOOD = dict(q=Q, k=K, v=V, o=O, lse=L, B=1, Hq=4, Hkv=2, N=16, d=64, causal=0,
            window_left=-1, scale=0.125, stream=None)


def call(dtype=_lib.FA_DTYPE_BF16, **over):
    a = dict(GOOD, **over)
    return _lib.fa_fwd(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["Hq"], a["Hkv"], a["N"],
                       a["d"], a["causal"], a["window_left"], a["scale"], a["stream"], dtype)


@pytest.mark.parametrize("over,status", [
    (dict(B=-1), _lib.FA_ERR_INVALID_ARG),
    (dict(N=-5), _lib.FA_ERR_INVALID_ARG),
    (dict(Hkv=-1), _lib.FA_ERR_INVALID_ARG),
    (dict(Hkv=3), _lib.FA_ERR_INVALID_ARG),
    (dict(Hkv=0), _lib.FA_ERR_INVALID_ARG),
    (dict(Hkv=8), _lib.FA_ERR_INVALID_ARG),
    (dict(window_left=-2), _lib.FA_ERR_INVALID_ARG),
    (dict(scale=float("nan")), _lib.FA_ERR_INVALID_ARG),
    (dict(scale=float("inf")), _lib.FA_ERR_INVALID_ARG),
    (dict(d=96), _lib.FA_ERR_UNSUPPORTED),
    (dict(d=256), _lib.FA_ERR_UNSUPPORTED),
    (dict(q=0), _lib.FA_ERR_INVALID_ARG),
    (dict(o=0), _lib.FA_ERR_INVALID_ARG),
    (dict(q=Q + 8), _lib.FA_ERR_MISALIGNED),
    (dict(o=O + 2), _lib.FA_ERR_MISALIGNED),
    (dict(lse=L + 2), _lib.FA_ERR_MISALIGNED),
    (dict(o=Q), _lib.FA_ERR_INVALID_ARG),          # output aliases an input
    (dict(lse=O + 64), _lib.FA_ERR_INVALID_ARG),   # lse inside o
])
def test_validation_rejects(over, status):
    assert call(**over) == status
    assert _lib.fa_last_error() != ""


def _nan_floats():
    """NaNs by bit pattern (quiet, signalling, negative, with payloads) and
    the infinities, as float32 objects that reach the C side bit for bit."""
    import struct
    bits = [0x7FC00000, 0x7F800001, 0xFFC00000, 0xFF800001, 0x7FFFFFFF, 0x7FA5A5A5, 0x7F800000, 0xFF800000]
    return [ctypes.c_float.from_buffer_copy(struct.pack("<I", b)) for b in bits]


@pytest.mark.parametrize("x", _nan_floats(), ids=lambda x: f"{ctypes.cast(ctypes.pointer(x), ctypes.POINTER(ctypes.c_uint32)).contents.value:#010x}")
def test_non_finite_scale_by_bit_pattern(x):
    """Every NaN and infinity is rejected whatever its bits: the host check
    must not depend on floating-point semantics the compiler may assume away."""
    assert call(scale=x) == _lib.FA_ERR_INVALID_ARG
    assert call_bwd(scale=x) == _lib.FA_ERR_INVALID_ARG
    assert call_fp8(scale=x) == _lib.FA_ERR_INVALID_ARG
    assert call_fp8(vs=x) == _lib.FA_ERR_INVALID_ARG
    assert call_kv(scale=x) == _lib.FA_ERR_INVALID_ARG


@pytest.mark.parametrize("scale", [0.0, -0.0, -0.5, -1e-30, -3.0e4])
def test_zero_and_negative_scales_pass_validation(scale):
    """Any finite scale is accepted: paired with an unsupported head dimension
    (so nothing is launched), the error reported is the head dimension's."""
    for fn in (lambda: call(scale=scale, d=96), lambda: call_bwd(scale=scale, d=96),
               lambda: call_fp8(scale=scale, d=96), lambda: call_kv(scale=scale, d=96)):
        assert fn() == _lib.FA_ERR_UNSUPPORTED
        assert "head dimension" in _lib.fa_last_error() and "scale" not in _lib.fa_last_error()


def test_unknown_dtype():
    assert call(dtype=7) == _lib.FA_ERR_UNSUPPORTED


@pytest.mark.parametrize("over", [dict(B=0), dict(Hq=0), dict(N=0), dict(B=0, q=0, k=0, v=0, o=0, lse=0)])
def test_empty_problem_is_a_noop(over):
    assert call(**over) == _lib.FA_OK
    assert _lib.fa_last_error() == ""


def test_typed_entry_points_validate_too():
    for fn in (_lib.fa_fwd_bf16, _lib.fa_fwd_f16, _lib.fa_fwd_f32):
        assert fn(Q, K, V, O, L, 1, 4, 3, 16, 64, 0, -1, 0.1, None) == _lib.FA_ERR_INVALID_ARG
        assert fn(Q, K, V, O, L, 1, 4, 2, 16, 80, 0, -1, 0.1, None) == _lib.FA_ERR_UNSUPPORTED
        assert fn(0, 0, 0, 0, 0, 0, 4, 2, 16, 64, 0, -1, 0.1, None) == _lib.FA_OK


def test_missing_library_fails_loudly(tmp_path, monkeypatch):
    monkeypatch.setattr(_lib, "_lib", None)
    monkeypatch.setattr(_lib, "LIB_PATH", str(tmp_path / "absent.so"))
    with pytest.raises(RuntimeError, match="not built"):
        _lib.load()


# backward: fake addresses again; every case fails (or no-ops) before a launch
DO, DQ, DK, DV, W = 0x600000, 0x700000, 0x800000, 0x900000, 0xA00000
GOOD_BWD = dict(q=Q, k=K, v=V, o=O, lse=L, dout=DO, dq=DQ, dk=DK, dv=DV, work=W, B=1, Hq=4, Hkv=2, N=16, d=64,
                causal=0, window_left=-1, scale=0.125, stream=None)


def call_bwd(dtype=_lib.FA_DTYPE_BF16, **over):
    a = dict(GOOD_BWD, **over)
    return _lib.fa_bwd(a["q"], a["k"], a["v"], a["o"], a["lse"], a["dout"], a["dq"], a["dk"], a["dv"], a["work"],
                       a["B"], a["Hq"], a["Hkv"], a["N"], a["d"], a["causal"], a["window_left"], a["scale"],
                       a["stream"], dtype)


@pytest.mark.parametrize("over,status", [
    (dict(B=-1), _lib.FA_ERR_INVALID_ARG),
    (dict(Hkv=3), _lib.FA_ERR_INVALID_ARG),
    (dict(window_left=-2), _lib.FA_ERR_INVALID_ARG),
    (dict(scale=float("nan")), _lib.FA_ERR_INVALID_ARG),
    (dict(d=96), _lib.FA_ERR_UNSUPPORTED),
    (dict(lse=0), _lib.FA_ERR_INVALID_ARG),
    (dict(dout=0), _lib.FA_ERR_INVALID_ARG),
    (dict(work=0), _lib.FA_ERR_INVALID_ARG),
    (dict(dq=DQ + 8), _lib.FA_ERR_MISALIGNED),
    (dict(work=W + 4), _lib.FA_ERR_MISALIGNED),
    (dict(lse=L + 2), _lib.FA_ERR_MISALIGNED),
    (dict(dq=Q), _lib.FA_ERR_INVALID_ARG),            # output aliases an input
    (dict(dk=DO + 64), _lib.FA_ERR_INVALID_ARG),      # output inside dout
    (dict(dv=DK), _lib.FA_ERR_INVALID_ARG),           # two outputs alias
    (dict(work=DV + 128), _lib.FA_ERR_INVALID_ARG),   # workspace inside dv
])
def test_bwd_validation_rejects(over, status):
    assert call_bwd(**over) == status
    assert _lib.fa_last_error() != ""


def test_bwd_rejects_f32_and_unknown_dtype():
    assert call_bwd(dtype=_lib.FA_DTYPE_F32) == _lib.FA_ERR_UNSUPPORTED
    assert call_bwd(dtype=9) == _lib.FA_ERR_UNSUPPORTED


@pytest.mark.parametrize("over", [dict(B=0), dict(N=0), dict(Hq=0, q=0, work=0)])
def test_bwd_empty_problem_is_a_noop(over):
    assert call_bwd(**over) == _lib.FA_OK
    assert _lib.fa_last_error() == ""


def test_bwd_typed_entry_points_and_workspace_size():
    for fn in (_lib.fa_bwd_bf16, _lib.fa_bwd_f16):
        assert fn(Q, K, V, O, L, DO, DQ, DK, DV, W, 1, 4, 3, 16, 64, 0, -1, 0.1, None) == _lib.FA_ERR_INVALID_ARG
        assert fn(Q, K, V, O, L, DO, DQ, DK, DV, W, 1, 4, 2, 16, 80, 0, -1, 0.1, None) == _lib.FA_ERR_UNSUPPORTED
    assert _lib.fa_bwd_workspace_size(2, 16, 8192) == 2 * 2 * 16 * 8192 * 4
    assert _lib.fa_bwd_workspace_size(0, 16, 8192) == 0
    assert _lib.fa_bwd_workspace_size(1, -1, 10) == 0


# FP8 forward: fake addresses; every case fails (or no-ops) before a launch
GOOD_FP8 = dict(q=Q, k=K, v=V, qs=0.01, ks=0.02, vs=0.03, o=O, lse=L, B=1, Hq=4, Hkv=2, N=16, d=64, causal=0,
                window_left=-1, scale=0.125, stream=None)


def call_fp8(**over):
    a = dict(GOOD_FP8, **over)
    return _lib.fa_fwd_fp8(a["q"], a["k"], a["v"], a["qs"], a["ks"], a["vs"], a["o"], a["lse"], a["B"], a["Hq"],
                           a["Hkv"], a["N"], a["d"], a["causal"], a["window_left"], a["scale"], a["stream"])


@pytest.mark.parametrize("over,status", [
    (dict(B=-1), _lib.FA_ERR_INVALID_ARG),
    (dict(Hkv=3), _lib.FA_ERR_INVALID_ARG),
    (dict(window_left=-2), _lib.FA_ERR_INVALID_ARG),
    (dict(scale=float("nan")), _lib.FA_ERR_INVALID_ARG),
    (dict(d=96), _lib.FA_ERR_UNSUPPORTED),
    (dict(qs=0.0), _lib.FA_ERR_INVALID_ARG),
    (dict(ks=-1.0), _lib.FA_ERR_INVALID_ARG),
    (dict(vs=float("inf")), _lib.FA_ERR_INVALID_ARG),
    (dict(vs=float("nan")), _lib.FA_ERR_INVALID_ARG),
    (dict(qs=1e20, ks=1e20), _lib.FA_ERR_INVALID_ARG),   # scale * q_scale * k_scale overflows
    (dict(v=0), _lib.FA_ERR_INVALID_ARG),
    (dict(k=K + 8), _lib.FA_ERR_MISALIGNED),
    (dict(lse=L + 1), _lib.FA_ERR_MISALIGNED),
    (dict(o=K - 1024), _lib.FA_ERR_INVALID_ARG),   # o (2 bytes per element) runs into k
    (dict(lse=O + 2048 - 4), _lib.FA_ERR_INVALID_ARG),   # lse inside o's 2-byte span
])
def test_fp8_validation_rejects(over, status):
    assert call_fp8(**over) == status
    assert _lib.fa_last_error() != ""


# Size limits: fake addresses 16 TiB apart, so that no span overlaps another and
# only the size rules (32-bit offsets within one head, one launch's grid) can
# reject the call.
FAR = 1 << 44
FAR_FWD = dict(q=1 * FAR, k=2 * FAR, v=3 * FAR, o=4 * FAR, lse=5 * FAR)
FAR_BWD = dict(FAR_FWD, dout=6 * FAR, dq=7 * FAR, dk=8 * FAR, dv=9 * FAR, work=10 * FAR)


@pytest.mark.parametrize("dtype,over,what", [
    (_lib.FA_DTYPE_BF16, dict(N=2 ** 24, d=64), "too long"),        # 2^24 * 64 * 2 B = 2 GiB per head
    (_lib.FA_DTYPE_F16, dict(N=2 ** 23, d=128), "too long"),        # 2^23 * 128 * 2 B = 2 GiB
    (_lib.FA_DTYPE_F32, dict(N=2 ** 22, d=128), "too long"),        # 2^22 * 128 * 4 B = 2 GiB
    (_lib.FA_DTYPE_BF16, dict(N=2 ** 23 - 2 ** 12, d=128), "too long"),   # within 1 MiB of the limit
    (_lib.FA_DTYPE_BF16, dict(B=2 ** 20, Hq=2 ** 12, Hkv=2 ** 12, N=1), "launch"),   # 2^32 row blocks
    (_lib.FA_DTYPE_F32, dict(B=2 ** 19, Hq=2 ** 12, Hkv=2 ** 12, N=1), "launch"),    # 2^31 row blocks
])
def test_size_limits_forward(dtype, over, what):
    assert call(dtype=dtype, **dict(FAR_FWD, **over)) == _lib.FA_ERR_UNSUPPORTED
    assert what in _lib.fa_last_error()


@pytest.mark.parametrize("over", [
    dict(N=2 ** 24, d=64),
    dict(N=2 ** 23, d=128),
    dict(B=2 ** 20, Hq=2 ** 12, Hkv=2 ** 12, N=1),
])
def test_size_limits_backward(over):
    assert call_bwd(**dict(FAR_BWD, **over)) == _lib.FA_ERR_UNSUPPORTED
    assert _lib.fa_last_error() != ""


@pytest.mark.parametrize("over", [
    dict(N=2 ** 24, d=128),                          # 2^24 * 128 * 1 B = 2 GiB per head
    dict(N=2 ** 25, d=64),
    dict(B=2 ** 20, Hq=2 ** 12, Hkv=2 ** 12, N=1),
])
def test_size_limits_fp8(over):
    assert call_fp8(**dict(FAR_FWD, **over)) == _lib.FA_ERR_UNSUPPORTED
    assert _lib.fa_last_error() != ""


def test_fp8_empty_problem_is_a_noop():
    assert call_fp8(B=0, q=0, k=0, v=0, o=0, lse=0) == _lib.FA_OK
    assert call_fp8(N=0) == _lib.FA_OK


# key/value cache: fake addresses; every case fails (or no-ops) before a launch
SQ, BT, WS = 0xB00000, 0xC00000, 0xD00000
GOOD_KV = dict(q=Q, k=K, v=V, seq=SQ, o=O, lse=L, ws=WS, B=1, Hq=4, Hkv=2, Nq=2, Nk=64, d=64, causal=1,
               window_left=-1, scale=0.125, splits=2, stream=None)


def call_kv(dtype=_lib.FA_DTYPE_BF16, **over):
    a = dict(GOOD_KV, **over)
    return _lib.fa_fwd_kvcache(a["q"], a["k"], a["v"], a["seq"], a["o"], a["lse"], a["ws"], a["B"], a["Hq"],
                               a["Hkv"], a["Nq"], a["Nk"], a["d"], a["causal"], a["window_left"], a["scale"],
                               a["splits"], a["stream"], dtype)


@pytest.mark.parametrize("over,status", [
    (dict(B=-1), _lib.FA_ERR_INVALID_ARG),
    (dict(Nk=-1), _lib.FA_ERR_INVALID_ARG),
    (dict(splits=-1), _lib.FA_ERR_INVALID_ARG),
    (dict(Hkv=3), _lib.FA_ERR_INVALID_ARG),
    (dict(window_left=-2), _lib.FA_ERR_INVALID_ARG),
    (dict(scale=float("nan")), _lib.FA_ERR_INVALID_ARG),
    (dict(d=96), _lib.FA_ERR_UNSUPPORTED),
    (dict(q=0), _lib.FA_ERR_INVALID_ARG),
    (dict(ws=0), _lib.FA_ERR_INVALID_ARG),                # two splits need a workspace
    (dict(ws=WS + 4), _lib.FA_ERR_MISALIGNED),
    (dict(seq=SQ + 2), _lib.FA_ERR_MISALIGNED),
    (dict(o=Q), _lib.FA_ERR_INVALID_ARG),                 # output aliases q
    (dict(ws=O + 64), _lib.FA_ERR_INVALID_ARG),           # workspace inside o
    (dict(Nk=2 ** 30), _lib.FA_ERR_UNSUPPORTED),          # one head's cache beyond 2 GiB
])
def test_kvcache_validation_rejects(over, status):
    assert call_kv(**over) == status
    assert _lib.fa_last_error() != ""


def test_kvcache_f32_and_empty():
    assert call_kv(dtype=_lib.FA_DTYPE_F32) == _lib.FA_ERR_UNSUPPORTED
    assert call_kv(B=0, q=0, k=0, v=0, o=0, lse=0, ws=0) == _lib.FA_OK
    assert call_kv(Nq=0) == _lib.FA_OK


def test_kvcache_paged_validation():
    def call(**over):
        a = dict(q=Q, k=K, v=V, bt=BT, seq=SQ, o=O, lse=L, ws=WS, B=1, Hq=4, Hkv=2, Nq=1, d=64, pages=8, ps=64,
                 maxp=4, causal=1, wl=-1, scale=0.125, splits=2)
        a.update(over)
        return _lib.fa_fwd_kvcache_paged(a["q"], a["k"], a["v"], a["bt"], a["seq"], a["o"], a["lse"], a["ws"],
                                         a["B"], a["Hq"], a["Hkv"], a["Nq"], a["d"], a["pages"], a["ps"], a["maxp"],
                                         a["causal"], a["wl"], a["scale"], a["splits"], None, _lib.FA_DTYPE_BF16)
    assert call(ps=48) == _lib.FA_ERR_UNSUPPORTED         # page size neither 16 nor a multiple of 32
    assert call(ps=8) == _lib.FA_ERR_UNSUPPORTED
    assert call(ps=0) == _lib.FA_ERR_INVALID_ARG
    assert call(pages=0) == _lib.FA_ERR_INVALID_ARG
    assert call(bt=0) == _lib.FA_ERR_INVALID_ARG          # a paged cache needs its table
    assert call(seq=0) == _lib.FA_ERR_INVALID_ARG         # and its lengths
    assert call(bt=BT + 2) == _lib.FA_ERR_MISALIGNED
    assert call(B=0) == _lib.FA_OK


def test_kvcache_workspace_size():
    ws = _lib.fa_fwd_kvcache_workspace_size
    assert ws(2, 8, 2, 3, 1000, 128, 1) == 0
    assert ws(2, 8, 2, 3, 1000, 128, 4) == 4 * 2 * 8 * 3 * 129 * 4
    assert ws(0, 8, 2, 3, 1000, 128, 4) == 0
    s = _lib.fa_fwd_kvcache_num_splits(2, 8, 2, 3, 1000)
    assert 1 <= s <= 128
    assert ws(2, 8, 2, 3, 1000, 128, 0) == (0 if s == 1 else s * 2 * 8 * 3 * 129 * 4)
    # a short cache is never cut below four 32-key tiles per split
    assert _lib.fa_fwd_kvcache_num_splits(1, 8, 8, 1, 100) == 1
    assert _lib.fa_fwd_kvcache_num_splits(1, 8, 8, 1, 32768) >= 8


def _splits_for(lens, Hq, Hkv, Nq, Nk, causal=1, wl=-1):
    import numpy as np
    a = np.ascontiguousarray(np.asarray(lens, dtype=np.int32))
    return _lib.fa_fwd_kvcache_num_splits_for_lengths(len(a), Hq, Hkv, Nq, Nk, causal, wl, a.ctypes.data)


def _active(lens, Hkv, Nq, Nk, S, wl=-1):
    """Splits that read keys, as the launch cuts them (each split a fixed
    share of the capacity), and the work items they make."""
    need = (Nk + 31) // 32
    if wl >= 0:
        need = min(need, (wl + Nq + 31) // 32 + 1)
    per = max(1, -(-need // S))
    chunks = 0
    for L in lens:
        L = min(max(L, 0), Nk)
        if L:
            lo = max(0, L - Nq - wl) if wl >= 0 else 0
            chunks += -(-((L - 1) // 32 + 1 - lo // 32) // per)
    return chunks * Hkv


def test_kvcache_splits_for_lengths():
    # no device here: the library assumes 256 compute units
    rows = lambda Hq, Hkv, Nq: -(-(Hq // Hkv) * Nq // 32)
    # equal full caches: three streaming wavefronts per unit are enough
    assert _splits_for([32768] * 8, 32, 8, 1, 32768) == 12
    # 16 query rows per sequence make two row blocks, one work item each:
    # four items per unit (64 per split) cap the splits at 16 before three
    # streams per unit are reached
    assert _splits_for([16384] * 4, 32, 8, 16, 16384) == 16
    # three blocks, three items per stream: the cap of 1024 items allows 21
    # splits (48 items each)
    assert _splits_for([16384] * 4, 32, 4, 12, 16384) == 21
    # four blocks: one wavefront takes two, two items per stream; the target
    # is four streams per unit, and the cap stops it at 32 splits
    assert _splits_for([16384] * 4, 32, 4, 16, 16384) == 32
    # caches of varied lengths leave splits empty: more splits than for full ones
    import numpy as np
    lens = np.random.default_rng(6).integers(1, 16385, 16)
    s = _splits_for(lens, 32, 8, 1, 16384)
    assert s > _splits_for([16384] * 16, 32, 8, 1, 16384)
    # the choice is the fewest splits meeting the rule, within the limits
    assert _active(lens, 8, 1, 16384, s) >= 3 * 256 and _active(lens, 8, 1, 16384, s) <= 4 * 256
    assert _active(lens, 8, 1, 16384, s - 1) < 3 * 256
    # nothing to read, or no lengths: one split
    assert _splits_for([0, 0, 0], 32, 8, 1, 16384) == 1
    assert _lib.fa_fwd_kvcache_num_splits_for_lengths(3, 32, 8, 1, 16384, 1, -1, None) == 1
    assert _lib.fa_fwd_kvcache_num_splits_for_lengths(3, 30, 8, 1, 16384, 1, -1, None) == 1
    # short caches keep at least four tiles per split; never above 128
    assert _splits_for([100], 8, 8, 1, 100) == 1
    assert 1 <= _splits_for([1 << 20] * 1, 8, 1, 1, 1 << 20) <= 128
    # a window bounds the keys a split can cover
    assert _splits_for([32768] * 8, 32, 8, 1, 32768, wl=1000) >= 1


# packed variable-length forward: fake addresses
CQ, CK = 0xE00000, 0xF00000
GOOD_VL = dict(q=Q, k=K, v=V, o=O, lse=L, cq=CQ, ck=CK, B=2, Hq=4, Hkv=2, tq=40, tk=50, mq=30, mk=30, d=64,
               causal=1, window_left=-1, scale=0.125, stream=None)


def call_vl(dtype=_lib.FA_DTYPE_BF16, **over):
    a = dict(GOOD_VL, **over)
    return _lib.fa_fwd_varlen(a["q"], a["k"], a["v"], a["o"], a["lse"], a["cq"], a["ck"], a["B"], a["Hq"],
                              a["Hkv"], a["tq"], a["tk"], a["mq"], a["mk"], a["d"], a["causal"], a["window_left"],
                              a["scale"], a["stream"], dtype)


@pytest.mark.parametrize("over,status", [
    (dict(B=-1), _lib.FA_ERR_INVALID_ARG),
    (dict(tk=-1), _lib.FA_ERR_INVALID_ARG),
    (dict(Hkv=3), _lib.FA_ERR_INVALID_ARG),
    (dict(window_left=-2), _lib.FA_ERR_INVALID_ARG),
    (dict(scale=float("nan")), _lib.FA_ERR_INVALID_ARG),
    (dict(scale=0.0, d=80), _lib.FA_ERR_UNSUPPORTED),     # a zero scale passes; the head dimension does not
    (dict(scale=-2.0, d=80), _lib.FA_ERR_UNSUPPORTED),
    (dict(d=80), _lib.FA_ERR_UNSUPPORTED),
    (dict(cq=0), _lib.FA_ERR_INVALID_ARG),
    (dict(ck=0), _lib.FA_ERR_INVALID_ARG),
    (dict(cq=CQ + 2), _lib.FA_ERR_MISALIGNED),
    (dict(o=O + 8), _lib.FA_ERR_MISALIGNED),
    (dict(o=Q), _lib.FA_ERR_INVALID_ARG),
    (dict(lse=O + 16), _lib.FA_ERR_INVALID_ARG),
    (dict(mk=2 ** 24), _lib.FA_ERR_UNSUPPORTED),
])
def test_varlen_validation_rejects(over, status):
    assert call_vl(**over) == status
    assert _lib.fa_last_error() != ""


def test_varlen_f32_and_empty():
    assert call_vl(dtype=_lib.FA_DTYPE_F32) == _lib.FA_ERR_UNSUPPORTED
    assert call_vl(B=0, q=0, k=0, v=0, o=0, lse=0, cq=0, ck=0) == _lib.FA_OK
    assert call_vl(tq=0) == _lib.FA_OK
    assert call_vl(mq=0) == _lib.FA_OK


# packed variable-length backward: fake addresses (1 MiB apart; the sizes
# below keep every buffer inside its MiB)
GOOD_BVL = dict(q=Q, k=K, v=V, o=O, lse=L, dout=DO, dq=DQ, dk=DK, dv=DV, work=W, cq=CQ, ck=CK, B=2, Hq=4, Hkv=2,
                tq=40, tk=50, mq=30, mk=30, d=64, causal=1, window_left=-1, scale=0.125, stream=None)


def call_bvl(dtype=_lib.FA_DTYPE_BF16, **over):
    a = dict(GOOD_BVL, **over)
    return _lib.fa_bwd_varlen(a["q"], a["k"], a["v"], a["o"], a["lse"], a["dout"], a["dq"], a["dk"], a["dv"],
                              a["work"], a["cq"], a["ck"], a["B"], a["Hq"], a["Hkv"], a["tq"], a["tk"], a["mq"],
                              a["mk"], a["d"], a["causal"], a["window_left"], a["scale"], a["stream"], dtype)


@pytest.mark.parametrize("over,status", [
    (dict(B=-1), _lib.FA_ERR_INVALID_ARG),
    (dict(tk=-1), _lib.FA_ERR_INVALID_ARG),
    (dict(Hkv=3), _lib.FA_ERR_INVALID_ARG),
    (dict(window_left=-2), _lib.FA_ERR_INVALID_ARG),
    (dict(scale=float("inf")), _lib.FA_ERR_INVALID_ARG),
    (dict(scale=-1.0, d=96), _lib.FA_ERR_UNSUPPORTED),    # a negative scale passes; the head dimension does not
    (dict(d=96), _lib.FA_ERR_UNSUPPORTED),
    (dict(lse=0), _lib.FA_ERR_INVALID_ARG),
    (dict(work=0), _lib.FA_ERR_INVALID_ARG),
    (dict(cq=0), _lib.FA_ERR_INVALID_ARG),
    (dict(ck=CK + 2), _lib.FA_ERR_MISALIGNED),
    (dict(dq=DQ + 8), _lib.FA_ERR_MISALIGNED),
    (dict(dk=DV), _lib.FA_ERR_INVALID_ARG),
    (dict(dq=Q), _lib.FA_ERR_INVALID_ARG),
    (dict(work=L), _lib.FA_ERR_INVALID_ARG),
    (dict(mk=2 ** 24), _lib.FA_ERR_UNSUPPORTED),
    (dict(mq=2 ** 23), _lib.FA_ERR_UNSUPPORTED),
])
def test_bwd_varlen_validation_rejects(over, status):
    assert call_bvl(**over) == status
    assert _lib.fa_last_error() != ""


def test_bwd_varlen_f32_and_empty():
    assert call_bvl(dtype=_lib.FA_DTYPE_F32) == _lib.FA_ERR_UNSUPPORTED
    assert call_bvl(B=0, q=0, k=0, v=0, o=0, lse=0, dout=0, dq=0, dk=0, dv=0, work=0, cq=0, ck=0) == _lib.FA_OK
    assert call_bvl(tq=0) == _lib.FA_OK
    assert call_bvl(mq=0) == _lib.FA_OK


# allocation-free paged decoding: validation as for the paged entry point, and
# a request beyond the library's scratch rejected before anything is enqueued
def call_noalloc(**over):
    a = dict(q=Q, k=K, v=V, bt=BT, seq=SQ, o=O, lse=L, B=1, Hq=4, Hkv=2, Nq=1, d=64, pages=8, ps=64, maxp=4,
             causal=1, wl=-1, scale=0.125, splits=2, dtype=_lib.FA_DTYPE_BF16)
    a.update(over)
    return _lib.fa_fwd_kvcache_paged_noalloc(a["q"], a["k"], a["v"], a["bt"], a["seq"], a["o"], a["lse"], a["B"],
                                             a["Hq"], a["Hkv"], a["Nq"], a["d"], a["pages"], a["ps"], a["maxp"],
                                             a["causal"], a["wl"], a["scale"], a["splits"], None, a["dtype"])


@pytest.mark.parametrize("over,status", [
    (dict(B=-1), _lib.FA_ERR_INVALID_ARG),
    (dict(splits=-1), _lib.FA_ERR_INVALID_ARG),
    (dict(Hkv=3), _lib.FA_ERR_INVALID_ARG),
    (dict(scale=float("nan")), _lib.FA_ERR_INVALID_ARG),
    (dict(d=96), _lib.FA_ERR_UNSUPPORTED),
    (dict(ps=48), _lib.FA_ERR_UNSUPPORTED),
    (dict(pages=0), _lib.FA_ERR_INVALID_ARG),
    (dict(bt=0), _lib.FA_ERR_INVALID_ARG),
    (dict(q=Q + 8), _lib.FA_ERR_MISALIGNED),
    (dict(o=Q), _lib.FA_ERR_INVALID_ARG),
    (dict(dtype=_lib.FA_DTYPE_F32), _lib.FA_ERR_UNSUPPORTED),
    (dict(splits=129), _lib.FA_ERR_UNSUPPORTED),
])
def test_kvcache_paged_noalloc_validation_rejects(over, status):
    assert call_noalloc(**over) == status
    assert _lib.fa_last_error() != ""


def test_kvcache_paged_noalloc_rejects_more_than_its_scratch():
    # 8 splits * 64 * 64 rows * (128 + 1) floats = 16.9 MB > 16 MiB
    st = call_noalloc(B=64, Hq=64, Hkv=2, d=128, pages=64 * 64, maxp=64, splits=8)
    assert st == _lib.FA_ERR_UNSUPPORTED
    assert "scratch" in _lib.fa_last_error()
    # the same request against the workspace form is only short of its workspace
    st = _lib.fa_fwd_kvcache_paged(Q, K, V, BT, SQ, O, L, None, 64, 64, 2, 1, 128, 64 * 64, 64, 64, 1, -1, 0.125, 8,
                                   None, _lib.FA_DTYPE_BF16)
    assert st == _lib.FA_ERR_INVALID_ARG and "workspace" in _lib.fa_last_error()


def test_kvcache_paged_noalloc_empty_is_a_noop():
    assert call_noalloc(B=0, q=0, k=0, v=0, o=0, lse=0) == _lib.FA_OK
    assert call_noalloc(Nq=0) == _lib.FA_OK
