"""Long sequences, eight times the longest workload: a 2^18-token causal
forward (d = 64, grouped heads), a 2^18-token sliding-window forward (d =
128), and decoding against 2^18-token caches (contiguous and paged).  The
forward outputs are compared on sampled rows (the first and last rows, rows
on either side of tile and block edges, and seeded random rows: the oracle
evaluates one row in O(N d)); the decoding outputs on every row.  Tolerance:
the forward's for 16-bit inputs, scaled by max(1, |O_ref|) elementwise.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import exact_tiled_attention_04_amd as fa
from oracle import attention_fwd, attention_fwd_kvcache
from tests.gpu_util import announce, compare, to_dev
from workloads import build_pages, random_inputs, round_to

pytestmark = pytest.mark.gpu


def _sample_rows(N, seed, n_random=40):
    edges = [0, 1, 2, 31, 32, 63, 64, 127, 128, 129, N // 2 - 1, N // 2, N - 129, N - 128, N - 65, N - 64,
             N - 2, N - 1]
    rnd = np.random.default_rng(seed).integers(0, N, size=n_random)
    return np.unique(np.clip(np.concatenate([edges, rnd]), 0, N - 1)).astype(np.int64)


def _run_sampled(q, k, v, dtype, causal, wl, scale, rows, label):
    announce(f"long {label} q={q.shape} k={k.shape} causal={causal} wl={wl}")
    qd, kd, vd = (to_dev(x, dtype) for x in (q, k, v))
    o, lse = fa.fwd(qd, kd, vd, causal=causal, window_left=wl, scale=scale)
    idx = torch.from_numpy(rows).cuda()
    o_s = o.index_select(2, idx).double().cpu().numpy()
    l_s = lse.index_select(2, idx).double().cpu().numpy()
    assert torch.isfinite(o).all().item() and torch.isfinite(lse).all().item(), f"{label}: non-finite output"
    return o_s, l_s


def test_long_causal_forward():
    B, Hq, Hkv, N, d = 1, 2, 1, 2 ** 18, 64
    q, k, v = random_inputs(8700, "bf16", B, Hq, Hkv, N, d)
    rows = _sample_rows(N, 8701)
    o, lse = _run_sampled(q, k, v, "bf16", True, -1, d ** -0.5, rows, "causal 2^18")
    ro, rl = attention_fwd(q, k, v, True, -1, d ** -0.5, rows=rows)
    compare(o, lse, ro, rl, "bf16", label=f"causal N=2^18 d=64, {len(rows)} rows", scaled=True)


def test_long_window_forward():
    B, Hq, Hkv, N, d = 1, 2, 2, 2 ** 18, 128
    q, k, v = random_inputs(8710, "f16", B, Hq, Hkv, N, d)
    rows = _sample_rows(N, 8711)
    o, lse = _run_sampled(q, k, v, "f16", True, 8192, d ** -0.5, rows, "window 2^18")
    ro, rl = attention_fwd(q, k, v, True, 8192, d ** -0.5, rows=rows)
    compare(o, lse, ro, rl, "f16", label=f"window 8192 N=2^18 d=128, {len(rows)} rows", scaled=True)


@pytest.mark.parametrize("paged", [False, True])
def test_long_cache(paged):
    B, Hq, Hkv, Nq, Nk, d = 2, 4, 1, 3, 2 ** 18, 128
    rng = np.random.default_rng(8720 + paged)
    q = round_to("f16", rng.standard_normal((B, Hq, Nq, d), dtype=np.float32))
    k = round_to("f16", rng.standard_normal((B, Hkv, Nk, d), dtype=np.float32))
    v = round_to("f16", rng.standard_normal((B, Hkv, Nk, d), dtype=np.float32))
    lens = np.array([Nk, Nk - 12345], dtype=np.int32)
    label = f"cache 2^18 paged={paged} lens={[int(x) for x in lens]}"
    announce(label)
    qd = to_dev(q, "f16")
    sd = torch.from_numpy(lens).cuda()
    if paged:
        kp, vp, table = build_pages(k, v, lens, 256, 8725)
        o, lse = fa.fwd_kvcache_paged(qd, to_dev(kp, "f16"), to_dev(vp, "f16"), torch.from_numpy(table).cuda(), sd,
                                      causal=True)
    else:
        o, lse = fa.fwd_kvcache(qd, to_dev(k, "f16"), to_dev(v, "f16"), sd, causal=True)
    o, lse = o.double().cpu().numpy(), lse.double().cpu().numpy()
    ro, rl = attention_fwd_kvcache(q, k, v, lens, True, -1, None)
    compare(o, lse, ro, rl, "f16", label=label, scaled=True)
