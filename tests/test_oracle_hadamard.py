"""Pins of the oracle's incoherence processing (ScaleSearch page, Metodologia /
ScaleSearchAttention: Hadamard transforms of Q and K before quantization,
as QuIP# does; a rotation R applied to both keeps Q K^T).

The transform is R = diag(s) H_n / sqrt(n) with H_n the Sylvester Hadamard
matrix; the pins compare it with scipy's Hadamard matrix, check the
orthogonality and the score invariant, and check that the attention oracle
routes only the FP4 path through it."""
import numpy as np
import pytest
import scipy.linalg
import torch

import oracle


def _signs(n, seed):
    rng = np.random.default_rng(seed)
    bits = rng.integers(0, 2, n)
    words = np.zeros(max(n // 32, 1), np.uint32)
    for j in range(n):
        if bits[j]:
            words[j >> 5] |= np.uint32(1 << (j & 31))
    return words, np.where(bits == 1, -1.0, 1.0)


@pytest.mark.parametrize("n", [16, 32, 64, 128])
def test_unit_vectors_give_the_hadamard_matrix(n):
    c = np.float32(1.0 / np.sqrt(n))
    got = oracle.hadamard_rows(np.eye(n, dtype=np.float32))
    np.testing.assert_array_equal(got, scipy.linalg.hadamard(n).astype(np.float32) * c)
    words, s = _signs(n, n)
    got = oracle.hadamard_rows(np.eye(n, dtype=np.float32), words)
    np.testing.assert_array_equal(got, (s[:, None] * scipy.linalg.hadamard(n)).astype(np.float32) * c)


@pytest.mark.parametrize("n", [64, 128])
def test_matches_the_matrix_product_and_is_orthogonal(n):
    rng = np.random.default_rng(1)
    x = rng.standard_normal((50, n)).astype(np.float32)
    words, s = _signs(n, 2)
    R = (s[:, None] * scipy.linalg.hadamard(n)) / np.sqrt(n)  # row-vector form: y = x R
    y = oracle.hadamard_rows(x, words)
    np.testing.assert_allclose(y, x.astype(np.float64) @ R, rtol=0, atol=2e-5 * np.abs(x).max() * np.sqrt(n))
    np.testing.assert_allclose(np.linalg.norm(y, axis=1), np.linalg.norm(x, axis=1), rtol=1e-5)
    # scores are kept: (Q R)(K R)^T = Q K^T
    q = rng.standard_normal((30, n)).astype(np.float32)
    k = rng.standard_normal((40, n)).astype(np.float32)
    qr, kr = oracle.hadamard_rows(q, words), oracle.hadamard_rows(k, words)
    np.testing.assert_allclose(qr.astype(np.float64) @ kr.T.astype(np.float64), q.astype(np.float64) @ k.T,
                               atol=1e-4)


def test_spreads_an_outlier_channel():
    """The point of the transform: one channel x20 no longer dominates its
    16-element block after the rotation (the worst block's maximum over its
    RMS drops)."""
    rng = np.random.default_rng(3)
    x = rng.standard_normal((256, 128)).astype(np.float32)
    x[:, 5] *= 20.0
    y = oracle.hadamard_rows(x, _signs(128, 4)[0])

    def peak_ratio(a):  # worst block of each row, averaged over rows
        b = a.reshape(256, 8, 16)
        return np.mean((np.abs(b).max(axis=2) / np.sqrt((b ** 2).mean(axis=2))).max(axis=1))

    assert peak_ratio(y) < 0.8 * peak_ratio(x)


def _prefill(S, d, seed):
    g = torch.Generator().manual_seed(seed)
    q = torch.randn(1, 2, S, d, generator=g)
    k = torch.randn(1, 2, S, d, generator=g)
    v = torch.randn(1, 2, S, d, generator=g)
    k[..., [3, 17, 40, 41]] *= 10.0  # outlier channels, as in the prefill workload
    return q.to(torch.bfloat16), k.to(torch.bfloat16), v.to(torch.bfloat16)


def test_attention_fp16_path_ignores_the_rotation():
    """With every block pair promoted the FP4 path is unused: the rotated and
    the plain oracle agree exactly."""
    q, k, v = _prefill(256, 64, 5)
    words = _signs(64, 6)[0]
    a, la = oracle.attention_fwd(q, k, v, causal=True, pct=100)
    b, lb = oracle.attention_fwd(q, k, v, causal=True, pct=100, hadamard=True, signs=words)
    np.testing.assert_array_equal(a, b)
    np.testing.assert_array_equal(la, lb)


def test_attention_error_drops_with_the_rotation():
    """On keys with outlier channels the FP4 path with the rotation is closer
    to exact attention than without it (the reason the page applies it)."""
    q, k, v = _prefill(512, 128, 7)
    words = _signs(128, 8)[0]
    ex, _ = oracle.attention_exact(q, k, v, causal=True)
    plain, _ = oracle.attention_fwd(q, k, v, causal=True)
    rot, _ = oracle.attention_fwd(q, k, v, causal=True, hadamard=True, signs=words)
    e_plain = np.linalg.norm(plain - ex) / np.linalg.norm(ex)
    e_rot = np.linalg.norm(rot - ex) / np.linalg.norm(ex)
    assert e_rot < e_plain, (e_rot, e_plain)
