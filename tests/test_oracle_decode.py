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


# ---- selective promotion (ThriftAttention page, Metodologia / 1 and / 2, in decode)

def _hybrid_textbook(q, k, v, n_sink, n_recent, L, promoted, blk=128):
    """Textbook attention over the cache as the decode reads it: the middle
    dequantized through the quantizer, except the promoted blocks (indices
    relative to the first middle token), which keep their original values."""
    kf, vf = k.float().numpy().copy(), v.float().numpy().copy()
    B, Hkv, _, d = kf.shape
    M = L - n_sink - n_recent
    for b in range(B):
        for h in range(Hkv):
            rk = oracle.quantize(kf[b, h, n_sink:n_sink + M], 0, True)
            rv = oracle.quantize(vf[b, h, n_sink:n_sink + M], 1, True)
            kd = oracle.dequantize(rk["codes"], rk["scales"], M, d, 0)
            vd = oracle.dequantize(rv["codes"], rv["scales"], M, d, 1)
            for j in promoted[b * Hkv + h]:
                t0, t1 = j * blk, min(j * blk + blk, M)
                kd[t0:t1] = kf[b, h, n_sink + t0:n_sink + t1]
                vd[t0:t1] = vf[b, h, n_sink + t0:n_sink + t1]
            kf[b, h, n_sink:n_sink + M] = kd
            vf[b, h, n_sink:n_sink + M] = vd
    return _textbook(q.float(), torch.tensor(kf), torch.tensor(vf), [L] * B)


def test_selective_all_blocks_is_textbook():
    """pct = 100 promotes every middle block: plain attention on the context."""
    B, Hq, Hkv, d = 1, 4, 2, 64
    n_sink, n_recent, M = 16, 16, 3 * 128 + 48  # a short last block
    L = n_sink + M + n_recent
    q, k, v = _rand((B, Hq, d), 20), _rand((B, Hkv, L, d), 21), _rand((B, Hkv, L, d), 22)
    out, lse, idx, cnt = oracle.attention_decode(q, k, v, [L], n_sink, n_recent, pct=100,
                                                 with_selection=True)
    np.testing.assert_allclose(out.reshape(B, Hq, d), _textbook(q, k, v, [L]), atol=1e-6)
    assert cnt.tolist() == [4, 4] and idx.tolist() == [[0, 1, 2, 3]] * 2


def test_selective_known_ranking_and_ties():
    """Key blocks built as a_j * u (so mean(K_j) = a_j u exactly) and queries
    u: the scores order like a_j.  Equal a_j tie; the lower block wins."""
    B, Hq, Hkv, d = 1, 2, 1, 32
    n_sink, n_recent, nb = 16, 16, 10
    M = nb * 128
    L = n_sink + M + n_recent
    u = np.zeros(d, np.float32)
    u[:8] = 1.0
    a = np.array([0.5, 3.0, -1.0, 2.0, 3.0, 0.25, 2.0, 1.0, -4.0, 2.0], np.float32)
    k = _rand((B, Hkv, L, d), 23).float().numpy()
    for j in range(nb):
        k[0, 0, n_sink + j * 128:n_sink + (j + 1) * 128] = a[j] * u
    q = torch.tensor(np.stack([u, u])[None]).to(torch.bfloat16)
    kt = torch.tensor(k).to(torch.bfloat16)
    v = _rand((B, Hkv, L, d), 24)
    for pct, want in ((20, [1, 4]), (30, [1, 3, 4]), (40, [1, 3, 4, 6]), (10, [1])):
        _, _, idx, cnt = oracle.attention_decode(q, kt, v, [L], n_sink, n_recent, pct=pct,
                                                 with_selection=True)
        k_exp = -(-pct * nb // 100)
        assert cnt[0] == k_exp == len(want)
        assert idx[0, :k_exp].tolist() == want and (idx[0, k_exp:] == -1).all()


def test_selective_uses_the_group_mean_query():
    """G = 2 queries u + w and u - w: the group mean is u, so the ranking is
    u's even where w alone would pick other blocks."""
    B, Hq, Hkv, d = 1, 2, 1, 32
    n_sink, n_recent, nb = 16, 16, 4
    M = nb * 128
    L = n_sink + M + n_recent
    u = np.zeros(d, np.float32)
    u[0] = 1.0
    w = np.zeros(d, np.float32)
    w[1] = 8.0
    blocks = [u * 1.0, w * 1.0, u * 2.0 + w * 0.5, -u]  # scores against u: 1, 0, 2, -1
    k = _rand((B, Hkv, L, d), 25).float().numpy()
    for j in range(nb):
        k[0, 0, n_sink + j * 128:n_sink + (j + 1) * 128] = blocks[j]
    q = torch.tensor(np.stack([u + w, u - w])[None]).to(torch.bfloat16)
    _, _, idx, cnt = oracle.attention_decode(q, torch.tensor(k).to(torch.bfloat16), _rand((B, Hkv, L, d), 26),
                                             [L], n_sink, n_recent, pct=50, with_selection=True)
    assert cnt[0] == 2 and idx[0].tolist() == [0, 2]


def test_selective_output_is_the_hybrid_cache():
    """Promoted blocks read the original K and V, the rest the dequantized
    NVFP4 copy; block boundaries count from the first middle token."""
    B, Hq, Hkv, d = 2, 4, 2, 64
    n_sink, n_recent, M = 16, 32, 2 * 128 + 64
    L = n_sink + M + n_recent
    q, k, v = _rand((B, Hq, d), 27), _rand((B, Hkv, L, d), 28), _rand((B, Hkv, L, d), 29)
    out, _, idx, cnt = oracle.attention_decode(q, k, v, [L, L], n_sink, n_recent, pct=34,
                                               with_selection=True)
    assert (cnt == 2).all()  # ceil(34 * 3 / 100)
    promoted = [[j for j in row if j >= 0] for row in idx.tolist()]
    ref = _hybrid_textbook(q, k, v, n_sink, n_recent, L, promoted)
    np.testing.assert_allclose(out.reshape(B, Hq, d), ref, atol=1e-6)
    plain, _ = oracle.attention_decode(q, k, v, [L, L], n_sink, n_recent)
    assert np.abs(out - plain).max() > 1e-4  # promotion changes the result


def test_block_sums_are_exact():
    """The binary64 block sums of bf16 values are exact here (the values span
    few binades), so they equal the correctly rounded sums of math.fsum."""
    x = _rand((300, 16), 30).float().numpy()
    s = oracle.block_sums(x, 128)
    assert s.shape == (3, 16)
    for j in range(3):
        for c in range(16):
            assert s[j, c] == math.fsum(float(t) for t in x[j * 128:(j + 1) * 128, c])
