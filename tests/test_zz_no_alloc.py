"""GPU test of the allocation-free paged decoding entry point
(fa_fwd_kvcache_paged_noalloc), through the C ABI: two calls in a row, the
second with a smaller input, each against the workspace form
(fa_fwd_kvcache_paged) on the same inputs -- the same kernels, so the same
bits -- and against the fp64 cache oracle at the decoding tolerance."""
from __future__ import annotations

import numpy as np
import pytest
import torch

from exact_tiled_attention_04_amd import _lib
from oracle import attention_fwd_kvcache
from tests.gpu_util import announce, compare, to_dev
from workloads import build_pages, round_to

pytestmark = pytest.mark.gpu

DT = {"bf16": _lib.FA_DTYPE_BF16, "f16": _lib.FA_DTYPE_F16}


def _case(seed, dtype, B, Hq, Hkv, Nq, cap, d, lens, page_size):
    rng = np.random.default_rng(seed)
    q = round_to(dtype, rng.standard_normal((B, Hq, Nq, d), dtype=np.float32))
    k = round_to(dtype, rng.standard_normal((B, Hkv, cap, d), dtype=np.float32))
    v = round_to(dtype, rng.standard_normal((B, Hkv, cap, d), dtype=np.float32))
    lens = np.asarray(lens, dtype=np.int32)
    kp, vp, table = build_pages(k, v, lens, page_size, seed, fill=np.nan, spare_pages=2)
    dev = dict(q=to_dev(q, dtype), kp=to_dev(kp, dtype), vp=to_dev(vp, dtype),
               table=torch.from_numpy(table).cuda(), lens=torch.from_numpy(lens).cuda())
    shape = dict(B=B, Hq=Hq, Hkv=Hkv, Nq=Nq, d=d, num_pages=kp.shape[0], page_size=page_size,
                 max_pages=table.shape[1])
    return (q, k, v, lens), dev, shape


def _outputs(dev, shape):
    o = torch.full_like(dev["q"], float("nan"))
    lse = torch.full(tuple(dev["q"].shape[:3]), float("nan"), dtype=torch.float32, device="cuda")
    return o, lse


def _run(dev, shape, dtype, causal, wl, scale, splits, noalloc, stream):
    o, lse = _outputs(dev, shape)
    s = shape
    args_head = (dev["q"].data_ptr(), dev["kp"].data_ptr(), dev["vp"].data_ptr(), dev["table"].data_ptr(),
                 dev["lens"].data_ptr(), o.data_ptr(), lse.data_ptr())
    tail = (s["num_pages"], s["page_size"], s["max_pages"], int(causal), wl, scale, splits, stream.cuda_stream,
            DT[dtype])
    if noalloc:
        st = _lib.fa_fwd_kvcache_paged_noalloc(*args_head, s["B"], s["Hq"], s["Hkv"], s["Nq"], s["d"], *tail)
    else:
        nk = s["page_size"] * s["max_pages"]
        nbytes = _lib.fa_fwd_kvcache_workspace_size(s["B"], s["Hq"], s["Hkv"], s["Nq"], nk, s["d"], splits)
        ws = torch.empty(max(1, nbytes // 4), dtype=torch.float32, device="cuda")
        st = _lib.fa_fwd_kvcache_paged(*args_head, ws.data_ptr(), s["B"], s["Hq"], s["Hkv"], s["Nq"], s["d"], *tail)
    assert st == _lib.FA_OK, _lib.fa_last_error()
    return o, lse


# (seed, dtype, B, Hq, Hkv, Nq, capacity, d, lengths, page size, causal, window, splits): the second call of each
# pair is smaller than the first
CASES = [
    [(3100, "bf16", 4, 16, 4, 2, 512, 128, [500, 77, 1, 256], 32, True, -1, 7),
     (3101, "bf16", 2, 8, 2, 1, 128, 64, [100, 33], 16, True, -1, 3)],
    [(3110, "f16", 3, 32, 8, 4, 1024, 128, [1024, 0, 640], 64, True, 100, 12),
     (3111, "f16", 1, 4, 4, 1, 256, 128, [200], 32, False, -1, 2)],
]


@pytest.mark.parametrize("pair", range(len(CASES)))
def test_noalloc_matches_workspace_form_two_calls(pair):
    stream = torch.cuda.current_stream()
    for seed, dtype, B, Hq, Hkv, Nq, cap, d, lens, ps, causal, wl, splits in CASES[pair]:
        host, dev, shape = _case(seed, dtype, B, Hq, Hkv, Nq, cap, d, lens, ps)
        label = f"noalloc B={B} H={Hq}/{Hkv} Nq={Nq} d={d} lens={lens} page={ps} splits={splits}"
        announce(label)
        o_ref, l_ref = _run(dev, shape, dtype, causal, wl, d ** -0.5, splits, False, stream)
        o_na, l_na = _run(dev, shape, dtype, causal, wl, d ** -0.5, splits, True, stream)
        torch.cuda.synchronize()
        # same kernels, same split count: the same bits
        assert torch.equal(o_na.view(torch.int16), o_ref.view(torch.int16)), label
        assert torch.equal(l_na.view(torch.int32), l_ref.view(torch.int32)), label
        q, k, v, lv = host
        ro, rl = attention_fwd_kvcache(q, k, v, lv, causal, wl, d ** -0.5)
        o, lse = o_na.double().cpu().numpy(), l_na.double().cpu().numpy()
        empty = np.isneginf(rl)
        assert (o[empty] == 0).all() and np.isneginf(lse[empty]).all(), label
        if (~empty).any():
            compare(o[~empty], lse[~empty], ro[~empty], rl[~empty], dtype, label=label, scaled=True)


def test_noalloc_request_beyond_scratch_is_refused_untouched():
    """More partial results than the scratch holds: an error, nothing
    enqueued, the caller's outputs as they were.  The buffers are of the
    request's real size."""
    B, Hq, Hkv, d, splits = 64, 64, 2, 128, 8
    assert splits * B * Hq * (d + 1) * 4 > 16 << 20
    _, dev, s = _case(3120, "bf16", B, Hq, Hkv, 1, 64, d, [64] * B, 32)
    o, lse = _outputs(dev, s)
    announce("noalloc beyond scratch")
    st = _lib.fa_fwd_kvcache_paged_noalloc(dev["q"].data_ptr(), dev["kp"].data_ptr(), dev["vp"].data_ptr(),
                                           dev["table"].data_ptr(), dev["lens"].data_ptr(), o.data_ptr(),
                                           lse.data_ptr(), B, Hq, Hkv, 1, d, s["num_pages"], s["page_size"],
                                           s["max_pages"], 1, -1, 0.1, splits, None, _lib.FA_DTYPE_BF16)
    torch.cuda.synchronize()
    assert st == _lib.FA_ERR_UNSUPPORTED and "scratch" in _lib.fa_last_error()
    assert torch.isnan(o).all() and torch.isnan(lse).all()
    # the same request with 2 splits fits, and equals the workspace form
    o_na, l_na = _run(dev, s, "bf16", True, -1, 0.1, 2, True, torch.cuda.current_stream())
    o_ref, l_ref = _run(dev, s, "bf16", True, -1, 0.1, 2, False, torch.cuda.current_stream())
    torch.cuda.synchronize()
    assert torch.equal(o_na.view(torch.int16), o_ref.view(torch.int16))
    assert torch.equal(l_na.view(torch.int32), l_ref.view(torch.int32))
