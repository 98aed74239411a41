"""CPU tests of the seeded input generator and FLOP accounting."""
import math

import numpy as np
import pytest
import torch

import workloads as W


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32) * 10.0,
                        np.array([0.0, -0.0, 1.0, 1.00390625, 1.0078125, 3.4e38, -3.4e38,
                                  1e-40, np.inf, -np.inf], dtype=np.float32)])
    # halfway cases: bit 15 set with nothing below -> ties to even
    u = rng.integers(0, 2**31, 1000, dtype=np.uint32) & 0x7F7F0000 | 0x8000
    x = np.concatenate([x, u.view(np.float32)])
    ours = W.round_to_bf16(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float32).numpy()
    np.testing.assert_array_equal(ours.view(np.uint32), ref.view(np.uint32))


def test_f16_rounding_matches_torch():
    x = np.random.default_rng(1).standard_normal(100000).astype(np.float32) * 100
    ref = torch.from_numpy(x).to(torch.float16).to(torch.float32).numpy()
    np.testing.assert_array_equal(W.round_to_f16(x), ref)


def test_inputs_are_deterministic_and_exact_in_dtype():
    w = W.WORKLOADS["gqa_f16_4k"]
    a = W.make_inputs(w, N=64)
    b = W.make_inputs(w, N=64)
    for x, y in zip(a, b):
        np.testing.assert_array_equal(x, y)
    q, k, v = a
    assert q.shape == (4, 32, 64, 128) and k.shape == (4, 8, 64, 128)
    np.testing.assert_array_equal(W.round_to_f16(q), q)
    # the outlier channel: one K channel is 8x the others in scale
    per_channel = np.abs(k).mean(axis=(0, 1, 2))
    c = int(per_channel.argmax())
    assert per_channel[c] > 5 * np.median(per_channel)
    w3 = W.WORKLOADS["causal_8k"]
    q3, _, _ = W.make_inputs(w3, B=1, Hq=1, Hkv=1, N=256)
    assert 0.4 < q3.std() < 0.6          # N(0,1) * 0.5
    np.testing.assert_array_equal(W.round_to_bf16(q3), q3)


@pytest.mark.parametrize("N,causal,wl", [(1, False, -1), (7, True, -1), (7, False, 2), (9, True, 3),
                                         (10, True, 0), (5, True, 100)])
def test_unmasked_pairs_brute_force(N, causal, wl):
    cnt = sum(1 for i in range(N) for j in range(N)
              if not ((causal and j > i) or (wl >= 0 and j < i - wl)))
    assert W.unmasked_pairs(N, causal, wl) == cnt


def test_metric_flops_headline_values():
    assert W.metric_flops(W.WORKLOADS["causal_8k"]) == 4 * 2 * 16 * 8192 ** 2 * 128 / 2
    assert math.isclose(W.metric_flops(W.WORKLOADS["causal_8k"]), 5.4976e11, rel_tol=1e-4)
    # sliding window: exact kept pairs; 125,859,840 per head at N=32768, wl=4096
    assert W.unmasked_pairs(32768, True, 4096) == 125859840
    assert math.isclose(W.metric_flops(W.WORKLOADS["swa_32k"]), 2.0621e12, rel_tol=1e-4)
    assert W.metric_flops(W.WORKLOADS["bf16_n1k_d64"]) == 4 * 8 * 16 * 1024 ** 2 * 64


def test_fp8_rounding_matches_torch_e4m3fn():
    """E4M3 rounding and byte encoding agree with torch's float8_e4m3fn
    conversion (round to nearest even) over normals, subnormals and ties."""
    import torch
    rng = np.random.default_rng(11)
    x = np.concatenate([rng.standard_normal(20000) * 40, rng.standard_normal(5000) * 0.01,
                        np.array([0.0, -0.0, 448.0, -448.0, 2 ** -9, 2 ** -10, 3 * 2 ** -11, 2 ** -6,
                                  1.0625, 1.1875, 17.0, 19.0, 240.0, 232.0])])
    x = np.clip(x, -448, 448)
    ours = W.round_to_fp8(x)
    t = torch.from_numpy(x.astype(np.float32)).to(torch.float8_e4m3fn)
    np.testing.assert_array_equal(ours, t.to(torch.float64).numpy())
    np.testing.assert_array_equal(W.fp8_bits(ours), t.view(torch.uint8).numpy())


def test_fp8_quantisation_recipe():
    w = W.FP8_WORKLOADS["causal_8k_fp8"]
    (qb, qs, qd), (kb, ks, kd), (vb, vs, vd) = W.make_fp8_inputs(w, B=1, Hq=1, Hkv=1, N=64)
    for b, sc, dq in ((qb, qs, qd), (kb, ks, kd), (vb, vs, vd)):
        assert b.dtype == np.uint8 and b.shape == (1, 1, 64, 128)
        assert np.abs(dq).max() == pytest.approx(448 * sc, rel=1e-6)   # the largest value maps to 448
        import torch
        back = torch.from_numpy(b).view(torch.float8_e4m3fn).to(torch.float64).numpy() * sc
        np.testing.assert_array_equal(back, dq)
    # quantisation is within half an E4M3 step of the float32 recipe
    q32, _, _ = W.make_inputs(w.replace(dtype="f32"), B=1, Hq=1, Hkv=1, N=64)
    assert np.abs(qd - q32).max() <= 2 ** -4 * np.abs(q32).max() + 1e-12
    with pytest.raises(ValueError):
        W.round_to_fp8(np.array([500.0]))


def test_decode_inputs_and_pages():
    """Decoding inputs are seeded and exact in their type; paging scatters
    every key of every sequence to the slot its table names, marks the rest,
    and leaves nothing else behind."""
    w = W.DECODE_WORKLOADS["decode_paged_varlen"].replace(B=3, Hq=4, Hkv=2, Nk=256, d=64)
    q, k, v, lens = W.make_decode_inputs(w)
    q2, _, _, lens2 = W.make_decode_inputs(w)
    np.testing.assert_array_equal(q, q2)
    np.testing.assert_array_equal(lens, lens2)
    assert q.shape == (3, 4, 1, 64) and k.shape == (3, 2, 256, 64) and lens.dtype == np.int32
    assert ((lens >= 1) & (lens <= 256)).all()
    np.testing.assert_array_equal(W.round_to_bf16(k), k)
    kp, vp, table = W.build_pages(k, v, lens, 64, w.seed, fill=np.nan, spare_pages=2)
    assert kp.shape == (3 * 4 + 2, 64, 2, 64) and table.shape == (3, 4)
    used = set()
    for b in range(3):
        L = int(lens[b])
        for j in range(4):
            if j * 64 >= L:
                assert table[b, j] == -1
                continue
            page = table[b, j]
            used.add(int(page))
            for t in range(64):
                key = j * 64 + t
                if key < L:
                    np.testing.assert_array_equal(kp[page, t], k[b, :, key])
                    np.testing.assert_array_equal(vp[page, t], v[b, :, key])
                else:
                    assert np.isnan(kp[page, t]).all() and np.isnan(vp[page, t]).all()
    for page in set(range(kp.shape[0])) - used:
        assert np.isnan(kp[page]).all()
    # full lengths by default
    _, _, _, full = W.make_decode_inputs(W.DECODE_WORKLOADS["verify_16_16k"].replace(B=2, Nk=64, Hq=2, Hkv=1))
    np.testing.assert_array_equal(full, [64, 64])
