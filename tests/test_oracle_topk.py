"""Pins of the oracle's block selection.

ThriftAttention page, Metodologia / 1: Q and K split into blocks; the score of a
block pair is the dot product of the blocks' mean token vectors; the top-k
pairs go to the FP16 path.  Resultados: budgets are a percentage of blocks.
"""
from fractions import Fraction

import numpy as np
import torch

import oracle


def test_count_rule_integer_ceiling():
    assert oracle.topk_count(10, 10) == 1  # 0.1*10 in binary64 would round up past 1
    assert oracle.topk_count(10, 11) == 2
    assert oracle.topk_count(10, 256) == 26
    assert oracle.topk_count(100, 7) == 7
    assert oracle.topk_count(5, 1) == 1
    assert oracle.topk_count(0, 50) == 0


def test_means_exact_on_integer_data():
    rng = np.random.default_rng(0)
    x = rng.integers(-50, 50, size=(300, 16)).astype(np.float32)
    m = oracle.block_means(x, 128)
    assert m.shape == (3, 16)
    assert np.array_equal(m[0], x[:128].astype(np.float64).sum(0) / 128)
    assert np.array_equal(m[2], x[256:].astype(np.float64).sum(0) / 44)


def test_scores_one_rounding_per_channel():
    # each step of the dot product is the exact s + q_c k_c rounded once to
    # binary64 (float() of a Fraction rounds to nearest, ties to even), in
    # ascending channel order
    rng = np.random.default_rng(7)
    qm = rng.standard_normal((5, 24))
    km = rng.standard_normal((6, 24)) * np.exp2(rng.integers(-20, 20, size=(6, 1)))
    got = oracle.block_scores(qm, km)
    separate = 0
    for i in range(5):
        for j in range(6):
            s = 0.0
            t = 0.0
            for c in range(24):
                s = float(Fraction(s) + Fraction(float(qm[i, c])) * Fraction(float(km[j, c])))
                t = t + float(qm[i, c]) * float(km[j, c])  # product rounded, then the sum
            assert got[i, j] == s, (i, j)
            separate += got[i, j] != t
    assert separate > 0  # the fused form is the one pinned, not the two-rounding one


def _brute(qm, km, causal, pct):
    nq, nk = qm.shape[0], km.shape[0]
    out = []
    for i in range(nq):
        vis = list(range(min(i + 1, nk))) if causal else list(range(nk))
        sc = {j: sum(float(qm[i, c]) * float(km[j, c]) for c in range(qm.shape[1])) for j in vis}
        k = -(-pct * len(vis) // 100)
        order = sorted(vis, key=lambda j: (-sc[j], j))
        out.append(sorted(order[:k]))
    return out


def test_topk_matches_sorted_brute_force():
    rng = np.random.default_rng(1)
    for trial in range(30):
        nq = int(rng.integers(1, 12))
        d = 16
        # small integers: the binary64 dot products are exact, so ties are real ties
        qm = rng.integers(-3, 4, size=(nq, d)).astype(np.float64)
        km = rng.integers(-3, 4, size=(nq, d)).astype(np.float64)
        for causal in (True, False):
            for pct in (5, 10, 25, 50, 100):
                idx, cnt = oracle.block_topk(qm, km, causal, pct)
                ref = _brute(qm, km, causal, pct)
                for i in range(nq):
                    got = [j for j in idx[i] if j >= 0]
                    assert got == ref[i], (trial, causal, pct, i)
                    assert cnt[i] == len(ref[i])


def test_known_ranking_and_full_budget():
    d = 8
    nq = 6
    km = np.zeros((nq, d))
    qm = np.zeros((nq, d))
    qm[:, 0] = 1.0
    km[:, 0] = [0.5, 3.0, -1.0, 2.0, 3.0, 0.0]  # ranking 1 = 4 (tie: lower j), 3, 0, 5, 2
    idx, cnt = oracle.block_topk(qm, km, False, 34)  # ceil(34*6/100) = 3
    assert list(idx[0]) == [1, 3, 4] and cnt[0] == 3
    idx, cnt = oracle.block_topk(qm, km, True, 34)
    assert list(idx[5][: cnt[5]]) == [1, 3, 4]
    assert list(idx[1][: cnt[1]]) == [1]            # visible {0,1}: ceil(0.68) = 1
    idx, cnt = oracle.block_topk(qm, km, True, 100)
    for i in range(nq):
        assert list(idx[i][: cnt[i]]) == list(range(i + 1))
        assert all(v == -1 for v in idx[i][cnt[i]:])


def test_selection_inside_attention_matches_standalone():
    g = torch.Generator().manual_seed(2)
    q = torch.randn(1, 2, 384, 32, generator=g).to(torch.bfloat16)
    k = torch.randn(1, 2, 384, 32, generator=g).to(torch.bfloat16)
    v = torch.randn(1, 2, 384, 32, generator=g).to(torch.bfloat16)
    _, _, tidx, tcnt = oracle.attention_fwd(q, k, v, causal=True, kv_tile=64, pct=50,
                                            sel_block=128, rows=[0], with_topk=True)
    for h in range(2):
        qm = oracle.block_means(q[0, h], 128)
        km = oracle.block_means(k[0, h], 128)
        idx, cnt = oracle.block_topk(qm, km, True, 50)
        assert np.array_equal(idx, tidx[h]) and np.array_equal(cnt, tcnt[h])
