"""Pins of the decode oracle over the sink-aware mixed-precision KV cache.

ScaleSearch page, Metodologia / ScaleSearchAttention: the first and the last
blocks of the KV cache stay in full precision, the middle ones in NVFP4.
"""
import math

import numpy as np
import torch

import oracle


def _rand(shape, seed):
    g = torch.Generator().manual_seed(seed)
    return torch.randn(*shape, generator=g).to(torch.bfloat16)


def _textbook(q, k, v, L):
    qd, kd, vd = q.double().numpy(), k.double().numpy(), v.double().numpy()
    B, Hq, d = qd.shape
    Hkv = kd.shape[1]
    G = Hq // Hkv
    out = np.zeros((B, Hq, d))
    for b in range(B):
        for h in range(Hq):
            s = kd[b, h // G, : L[b]] @ qd[b, h] / math.sqrt(d)
            p = np.exp(s - s.max())
            out[b, h] = (p / p.sum()) @ vd[b, h // G, : L[b]]
    return out


def test_all_full_precision_context_is_textbook():
    B, Hq, Hkv, d, L = 2, 4, 2, 64, 96
    q, k, v = _rand((B, Hq, d), 0), _rand((B, Hkv, L, d), 1), _rand((B, Hkv, L, d), 2)
    ctx = [96, 80]
    out, _ = oracle.attention_decode(q, k, v, ctx, n_sink=16, n_recent=80 - 16 - 0)
    ref = _textbook(q, k, v, [96 - 16, 80])  # ctx 96 has 16 middle tokens -> not all bf16
    # only batch 1 is entirely sink+recent (80 = 16 + 64)
    np.testing.assert_allclose(out.reshape(B, Hq, d)[1], ref[1], atol=1e-6)


def test_exactly_representable_middle_is_textbook():
    # middle K and V values are code * 2^e with the block maximum hitting code 6: NVFP4
    # stores them exactly, so decode must equal textbook attention on the original values
    B, Hq, Hkv, d = 1, 4, 1, 32
    n_sink, n_recent, M = 16, 16, 64
    L = n_sink + M + n_recent
    rng = np.random.default_rng(3)
    grid = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6])
    k = rng.standard_normal((B, Hkv, L, d)).astype(np.float32)
    v = rng.standard_normal((B, Hkv, L, d)).astype(np.float32)
    kk = grid[rng.integers(0, 8, (M, d))] * np.where(rng.random((M, d)) < 0.5, -1, 1) * 0.25
    kk[:, 0::16] = 6 * 0.25   # every 16-wide K block along d holds its max 6*s
    vv = grid[rng.integers(0, 8, (M, d))] * 0.5
    vv[0::16, :] = -6 * 0.5   # every 16-token V block holds its max
    k[0, 0, n_sink:n_sink + M] = kk
    v[0, 0, n_sink:n_sink + M] = vv
    kt, vt = torch.tensor(k).to(torch.bfloat16), torch.tensor(v).to(torch.bfloat16)
    q = _rand((B, Hq, d), 4)
    out, lse = oracle.attention_decode(q, kt, vt, [L], n_sink, n_recent, scale_search=False)
    ref = _textbook(q, kt, vt, [L])
    np.testing.assert_allclose(out.reshape(B, Hq, d), ref, atol=1e-6)


def test_gqa_identical_heads_and_pair_selection():
    B, Hq, Hkv, d = 2, 8, 2, 64
    n_sink, n_recent, M = 16, 32, 128
    L = n_sink + M + n_recent
    k, v = _rand((B, Hkv, L, d), 5), _rand((B, Hkv, L, d), 6)
    q = _rand((B, Hq, d), 7)
    q[:, 4:8] = q[:, 4:5]   # kv-head 1's group: four identical queries
    out, lse = oracle.attention_decode(q, k, v, [L, L - 16], n_sink, n_recent)
    o = out.reshape(B, Hkv, 4, d)
    for g in range(1, 4):
        np.testing.assert_array_equal(o[:, 1, g], o[:, 1, 0])
    part, _ = oracle.attention_decode(q, k, v, [L, L - 16], n_sink, n_recent, pairs=[3, 0])
    np.testing.assert_array_equal(part[0], o[1, 1])
    np.testing.assert_array_equal(part[1], o[0, 0])


def test_middle_region_matches_quantizer_layouts():
    B, Hq, Hkv, d = 1, 2, 1, 64
    n_sink, n_recent, M = 16, 16, 96
    L = n_sink + M + n_recent
    k, v, q = _rand((B, Hkv, L, d), 8), _rand((B, Hkv, L, d), 9), _rand((B, Hq, d), 10)
    out, _ = oracle.attention_decode(q, k, v, [L], n_sink, n_recent)
    kf, vf = k.float().numpy().copy(), v.float().numpy().copy()
    rk = oracle.quantize(kf[0, 0, n_sink:n_sink + M], 0, True)
    rv = oracle.quantize(vf[0, 0, n_sink:n_sink + M], 1, True)
    kf[0, 0, n_sink:n_sink + M] = oracle.dequantize(rk["codes"], rk["scales"], M, d, 0)
    vf[0, 0, n_sink:n_sink + M] = oracle.dequantize(rv["codes"], rv["scales"], M, d, 1)
    ref = _textbook(q.float(), torch.tensor(kf), torch.tensor(vf), [L])
    np.testing.assert_allclose(out.reshape(B, Hq, d), ref, atol=1e-6)
    # and the FP4 middle is a real approximation: differs from the bf16 context
    plain = _textbook(q, k, v, [L])
    assert np.abs(out.reshape(B, Hq, d) - plain).max() > 1e-3
