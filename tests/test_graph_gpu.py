"""The library's calls under HIP graph capture (torch.cuda.CUDAGraph).

Every entry point enqueues kernels only (no allocation, no memset, no
synchronisation), so a caller can capture a call once and replay it.  Each
test captures a call on preallocated buffers, then replays the graph several
times with the program's own eager work in between (the outputs refilled
with NaN, new values copied into the inputs, synchronisations), and checks
every replay bit for bit against the same call run eagerly on the same
values: the kernels are deterministic, so a replay that read stale inputs or
skipped work would differ.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import exact_tiled_attention_04_amd as fa
from tests.gpu_util import announce, to_dev
from workloads import build_pages, quantize_fp8, random_grad, random_inputs, round_to

pytestmark = pytest.mark.gpu

REPLAYS = 3


def _capture(fn):
    """Capture fn() into a graph (after one warm-up call on a side stream,
    as torch recommends)."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def _same(a, b, label):
    assert a.shape == b.shape and a.dtype == b.dtype, label
    assert torch.equal(a, b), f"{label}: replay differs from the eager call"


def _replay_and_check(g, inputs, draws, outputs, eager, label):
    """For each replay: copy draw r into the captured input tensors, poison
    the outputs, replay, and compare with eager(draw r)."""
    for r in range(REPLAYS):
        announce(f"graph {label} replay {r}")
        for t, x in zip(inputs, draws[r]):
            t.copy_(x)
        for o in outputs:
            o.fill_(float("nan")) if o.is_floating_point() else o.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        want = eager(*draws[r])
        for i, (o, w) in enumerate(zip(outputs, want)):
            _same(o, w, f"{label} replay {r} output {i}")


def test_forward_graph():
    B, Hq, Hkv, N, d = 1, 4, 2, 700, 128
    draws = [tuple(to_dev(x, "bf16") for x in random_inputs(8000 + r, "bf16", B, Hq, Hkv, N, d))
             for r in range(REPLAYS)]
    q, k, v = (x.clone() for x in draws[0])
    o = torch.empty_like(q)
    lse = torch.empty((B, Hq, N), dtype=torch.float32, device="cuda")
    g = _capture(lambda: fa.fwd(q, k, v, causal=True, window_left=300, out=o, lse=lse))

    def eager(q_, k_, v_):
        return fa.fwd(q_, k_, v_, causal=True, window_left=300)

    _replay_and_check(g, (q, k, v), draws, (o, lse), eager, "forward")


def test_backward_graph():
    B, Hq, Hkv, N, d = 1, 4, 2, 300, 64
    draws = []
    for r in range(REPLAYS):
        q, k, v = (to_dev(x, "f16") for x in random_inputs(8100 + r, "f16", B, Hq, Hkv, N, d))
        do = to_dev(random_grad(8150 + r, "f16", B, Hq, N, d), "f16")
        o, lse = fa.fwd(q, k, v, causal=True)
        draws.append((q, k, v, o, lse, do))
    q, k, v, o, lse, do = (x.clone() for x in draws[0])
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws = torch.empty(max(1, fa._lib.fa_bwd_workspace_size(B, Hq, N) // 4), dtype=torch.float32, device="cuda")
    g = _capture(lambda: fa.bwd(q, k, v, o, lse, do, causal=True, dq=dq, dk=dk, dv=dv, workspace=ws))

    def eager(*a):
        return fa.bwd(*a, causal=True)

    _replay_and_check(g, (q, k, v, o, lse, do), draws, (dq, dk, dv), eager, "backward")


def test_fp8_graph():
    B, Hq, Hkv, N, d = 1, 2, 1, 500, 128
    # one set of per-tensor scales (they are call arguments, fixed at capture);
    # the bytes change between replays
    scales = None
    draws = []
    for r in range(REPLAYS):
        q, k, v = random_inputs(8200 + r, "f32", B, Hq, Hkv, N, d)
        qq = [quantize_fp8(x) for x in (q, k, v)]
        if scales is None:
            scales = tuple(x[1] for x in qq)
        draws.append(tuple(torch.from_numpy(np.ascontiguousarray(x[0])).cuda() for x in qq))
    q, k, v = (x.clone() for x in draws[0])
    o = torch.empty((B, Hq, N, d), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((B, Hq, N), dtype=torch.float32, device="cuda")
    g = _capture(lambda: fa.fwd_fp8(q, k, v, *scales, causal=True, out=o, lse=lse))

    def eager(q_, k_, v_):
        return fa.fwd_fp8(q_, k_, v_, *scales, causal=True)

    _replay_and_check(g, (q, k, v), draws, (o, lse), eager, "fp8")


def test_packed_forward_graph():
    lens = [300, 0, 129, 64]
    Hq, Hkv, d = 4, 2, 128
    cu = torch.from_numpy(np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)).cuda()
    T = sum(lens)
    draws = []
    for r in range(REPLAYS):
        rng = np.random.default_rng(8300 + r)
        draws.append(tuple(to_dev(round_to("bf16", rng.standard_normal((T, H, d), dtype=np.float32)), "bf16")
                           for H in (Hq, Hkv, Hkv)))
    q, k, v = (x.clone() for x in draws[0])
    o = torch.empty_like(q)
    lse = torch.empty((Hq, T), dtype=torch.float32, device="cuda")
    mx = max(lens)
    g = _capture(lambda: fa.fwd_varlen(q, k, v, cu, cu, mx, mx, causal=True, out=o, lse=lse))

    def eager(q_, k_, v_):
        return fa.fwd_varlen(q_, k_, v_, cu, cu, mx, mx, causal=True)

    _replay_and_check(g, (q, k, v), draws, (o, lse), eager, "packed forward")


@pytest.mark.parametrize("paged", [False, True])
def test_kvcache_graph(paged):
    """Split-KV decoding with four splits: the split kernel, the workspace
    and the merge all inside the graph; the cache lengths change between
    replays through the captured length tensor."""
    B, Hq, Hkv, Nq, Nk, d, page = 3, 8, 2, 2, 512, 128, 64
    splits = 4
    rng = np.random.default_rng(8400 + paged)
    draws = []
    for r in range(REPLAYS):
        q = round_to("bf16", rng.standard_normal((B, Hq, Nq, d), dtype=np.float32))
        k = round_to("bf16", rng.standard_normal((B, Hkv, Nk, d), dtype=np.float32))
        v = round_to("bf16", rng.standard_normal((B, Hkv, Nk, d), dtype=np.float32))
        lens = rng.integers(1, Nk + 1, size=B).astype(np.int32)
        if paged:
            kp, vp, table = build_pages(k, v, lens, page, 8450, fill=0.0)
            draws.append((to_dev(q, "bf16"), to_dev(kp, "bf16"), to_dev(vp, "bf16"),
                          torch.from_numpy(table).cuda(), torch.from_numpy(lens).cuda()))
        else:
            draws.append((to_dev(q, "bf16"), to_dev(k, "bf16"), to_dev(v, "bf16"), torch.from_numpy(lens).cuda()))
    cur = [x.clone() for x in draws[0]]
    o = torch.empty_like(cur[0])
    lse = torch.empty((B, Hq, Nq), dtype=torch.float32, device="cuda")
    cap = page * draws[0][3].shape[1] if paged else Nk
    ws = torch.empty(max(1, fa._lib.fa_fwd_kvcache_workspace_size(B, Hq, Hkv, Nq, cap, d, splits) // 4),
                     dtype=torch.float32, device="cuda")
    if paged:
        def call(q_, kp_, vp_, t_, l_, **kw):
            return fa.fwd_kvcache_paged(q_, kp_, vp_, t_, l_, causal=True, num_splits=splits, **kw)
    else:
        def call(q_, k_, v_, l_, **kw):
            return fa.fwd_kvcache(q_, k_, v_, l_, causal=True, num_splits=splits, **kw)
    g = _capture(lambda: call(*cur, out=o, lse=lse, workspace=ws))
    _replay_and_check(g, cur, draws, (o, lse), lambda *a: call(*a), f"kvcache paged={paged}")
