"""Pins of the magnitude-balancing pair Q' = Q R^-T, K' = K R (ScaleSearch
page, Metodologia / ScaleSearchAttention: the pair keeps the attention scores
and lowers the mean squared magnitude of the projected tensors).  Reading: R
diagonal with power-of-two entries 2^e_c per (batch, kv head), e_c the
integer in [-8, 8] minimizing ms_q 4^-e + ms_k 4^e."""
import math
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from block_scaled_fp4_amd import synth


def _rand(shape, seed, scale=1.0):
    g = torch.Generator().manual_seed(seed)
    return (torch.randn(*shape, generator=g) * scale).to(torch.bfloat16)


def test_scores_are_kept_exactly():
    q, k = _rand((2, 4, 96, 64), 1), _rand((2, 2, 80, 64), 2)
    k[:, :, :, 5] *= 24
    q[:, :, :, 9] *= 0.05
    e = oracle.balance_exponents(q, k)
    assert np.abs(e).max() >= 1  # the test data does move some channels
    qb, kb = oracle.balance_apply(q, k, e)
    qf, kf = q.float().numpy().astype(np.float64), k.float().numpy().astype(np.float64)
    G = 2
    for b in range(2):
        for h in range(4):
            s0 = qf[b, h] @ kf[b, h // G].T
            s1 = qb[b, h].astype(np.float64) @ kb[b, h // G].astype(np.float64).T
            assert np.array_equal(s0, s1)  # power-of-two scaling: every product identical


@pytest.mark.parametrize("a,b,want", [(1.0, 16.0, -2), (16.0, 1.0, 2), (1.0, 1.0, 0), (2.0, 1.0, 0),
                                      (4.0, 1.0, 1), (1.0, 2.0, -1), (1.0, 4.0, -1), (1.0, 2.0 ** 20, -8),
                                      (2.0 ** 20, 1.0, 8)])
def test_closed_form_exponents(a, b, want):
    """One channel of Q at +-a and of K at +-b: ms_q / ms_k = (a / b)^2; the
    minimizer of (a/b)^2 4^-e + 4^e is the smallest e with 4^(2e+1) >= (a/b)^2.
    a = 2b and b = 2a sit on ties (f(0) = f(1), f(-1) = f(0)): the lower
    exponent wins, 0 and -1.
    Ratios past 4^17 clamp at +-8."""
    d = 16
    q = torch.ones(1, 1, 32, d)
    k = torch.ones(1, 1, 48, d)
    sgn = torch.tensor([1.0, -1.0]).repeat(24)
    q[0, 0, :, 3] = a * sgn[:32]
    k[0, 0, :, 3] = b * sgn[:48]
    e = oracle.balance_exponents(q.to(torch.bfloat16), k.to(torch.bfloat16))
    assert e[0, 0, 3] == want
    assert np.all(np.delete(e[0, 0], 3) == 0)  # the unit channels balance already


def test_exponents_minimize_the_mean_square_sum():
    """Brute force in exact rationals over e in [-8, 8] (ties to the lower e)."""
    rng = np.random.default_rng(7)
    for trial in range(6):
        q = _rand((1, 2, 40, 32), 100 + trial)
        k = _rand((1, 1, 56, 32), 200 + trial)
        scale = torch.tensor(2.0 ** rng.integers(-6, 7, size=32)).float()
        k = (k.float() * scale).to(torch.bfloat16)
        e = oracle.balance_exponents(q, k)
        qf, kf = q.float().numpy().astype(np.float64), k.float().numpy().astype(np.float64)
        for c in range(32):
            sq = sum(Fraction(float(x)) ** 2 for x in qf[0, :, :, c].ravel())
            sk = sum(Fraction(float(x)) ** 2 for x in kf[0, 0, :, c].ravel())
            mq, mk = sq / (2 * 40), sk / 56
            cost = {x: mq * Fraction(4) ** (-x) + mk * Fraction(4) ** x for x in range(-8, 9)}
            best = min(cost.values())
            assert e[0, 0, c] == min(x for x in cost if cost[x] == best)


def test_balanced_mean_squares_within_a_factor_four():
    q, k, _ = synth.qkv(1, 4, 256, 128, seed=11, Hkv=2, k_outliers=4)
    e = oracle.balance_exponents(q, k)
    qb, kb = oracle.balance_apply(q, k, e)
    for hk in range(2):
        mq = (qb[0, 2 * hk:2 * hk + 2].astype(np.float64) ** 2).mean(axis=(0, 1))
        mk = (kb[0, hk].astype(np.float64) ** 2).mean(axis=0)
        r = mq / mk
        assert np.all(r <= 4.0) and np.all(r > 0.25)
    # the K outlier channels (x10) are scaled down, their Q channels up
    for hk in range(2):
        ch = synth.outlier_channels(128, 4, 1000 + 11 * 97 + hk).numpy()
        assert np.all(e[0, hk, ch] < 0)


def test_group_heads_share_one_exponent_vector():
    """With GQA the exponents of a kv head come from all its query heads."""
    q, k, _ = synth.qkv(1, 4, 64, 32, seed=12, Hkv=1)
    q[:, 1] *= 64  # one head of the group much larger
    e4 = oracle.balance_exponents(q, k)
    e_one = oracle.balance_exponents(q[:, 1:2], k)
    assert e4.shape == (1, 1, 32)
    assert not np.array_equal(e4, e_one)  # the mean over the group, not one head
    qb, kb = oracle.balance_apply(q, k, e4)
    for h in range(4):
        assert np.array_equal(qb[0, h], np.ldexp(q[0, h].float().numpy(), -e4[0, 0][None, :]))


def test_zero_channel_keeps_exponent_zero():
    q, k, _ = synth.qkv(1, 1, 32, 16, seed=13)
    k[..., 2] = 0
    q[..., 7] = 0
    e = oracle.balance_exponents(q, k)
    assert e[0, 0, 2] == 0 and e[0, 0, 7] == 0


def test_balance_lowers_fp4_error_on_k_outliers():
    """On keys with outlier channels (x10 on 4 of 128), quantizing the balanced
    pair brings the FP4 attention closer to exact attention; with the Hadamard
    rotation as well (balance first, rotation after) too."""
    q, k, v = synth.qkv(1, 2, 512, 128, seed=14, k_outliers=4)
    ex, _ = oracle.attention_exact(q, k, v, causal=True)
    err = lambda o: np.linalg.norm(o - ex) / np.linalg.norm(ex)
    plain, _ = oracle.attention_fwd(q, k, v, causal=True)
    bal, _ = oracle.attention_fwd(q, k, v, causal=True, balance=True)
    assert err(bal) < err(plain)
    signs = [0x9E3779B9, 0x7F4A7C15, 0x2545F491, 0xD1B54A32]
    had, _ = oracle.attention_fwd(q, k, v, causal=True, hadamard=True, signs=signs)
    both, _ = oracle.attention_fwd(q, k, v, causal=True, hadamard=True, signs=signs, balance=True)
    assert err(both) < err(plain) and err(had) < err(plain)


def test_balance_leaves_the_fp16_path_and_selection_alone():
    """With every pair promoted the FP16 path uses the original Q and K: the
    balanced and the plain oracle agree exactly; the selection is unchanged."""
    q, k, v = synth.qkv(1, 2, 384, 64, seed=15, k_outliers=4)
    a, la, ia, ca = oracle.attention_fwd(q, k, v, causal=True, pct=100, with_topk=True)
    b, lb, ib, cb = oracle.attention_fwd(q, k, v, causal=True, pct=100, with_topk=True, balance=True)
    np.testing.assert_array_equal(a, b)
    np.testing.assert_array_equal(ia, ib)
    _, _, i10, c10 = oracle.attention_fwd(q, k, v, causal=True, pct=34, with_topk=True, rows=[0])
    _, _, j10, d10 = oracle.attention_fwd(q, k, v, causal=True, pct=34, with_topk=True, rows=[0], balance=True)
    np.testing.assert_array_equal(i10, j10)
