"""Pins of the MXFP4 variant of the oracle: E2M1 elements with one
power-of-two (E8M0) scale per 32 elements, the classic block floating point
the ScaleSearch page contrasts NVFP4 with (Declaracion del Problema).  The
scale rule is the OCP microscaling one: shared exponent floor(log2 amax) - 2.

Pinned by an independent exact-rational implementation (Python fractions) on
random blocks, closed forms, and attention cases whose probabilities are
exact powers of two."""
import math
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle

E2M1 = [Fraction(0), Fraction(1, 2), Fraction(1), Fraction(3, 2), Fraction(2), Fraction(3), Fraction(4), Fraction(6)]


def _code(t: Fraction) -> int:
    """Nearest E2M1 magnitude code, ties to the even code, saturating at 6."""
    if t >= 6:
        return 7
    best = min(range(8), key=lambda c: (abs(t - E2M1[c]), c % 2))
    return best


def _ref_block(y):
    a = max(abs(Fraction(float(v))) for v in y)
    if a == 0:
        return 0, [8 * (math.copysign(1.0, float(v)) < 0) for v in y]
    e = math.floor(math.log2(a))
    while Fraction(2) ** e > a:   # exact floor(log2 a) for a rational
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    shared = max(min(e - 2, 127), -127)
    X = Fraction(2) ** shared
    codes = [_code(abs(Fraction(float(v))) / X) | (8 if math.copysign(1.0, float(v)) < 0 else 0) for v in y]
    return shared + 127, codes


def test_scale_byte_rule():
    for a, b in ((1.0, 125), (0.999, 124), (4.0, 127), (7.99, 127), (8.0, 128), (0.0, 0),
                 (float("inf"), 255), (2.0 ** -200, 0), (2.0 ** 200, 254)):
        assert oracle.mx_scale_byte(a) == b, a


@pytest.mark.parametrize("axis", [0, 1])
def test_quantizer_matches_exact_rationals(axis):
    rng = np.random.default_rng(11 + axis)
    x = rng.standard_normal((64, 64)).astype(np.float32) * np.exp2(rng.integers(-6, 6, (64, 1))).astype(np.float32)
    x = torch.tensor(x).to(torch.bfloat16).float().numpy()
    x[3, :] = 0.0
    r = oracle.mx_quantize(x, axis)
    for blk in range(64 * 2):
        if axis == 0:
            rr, c0 = blk // 2, (blk % 2) * 32
            y = x[rr, c0:c0 + 32]
            got_s = r["scales"][rr, c0 // 32]
            got_c = [(r["codes"][rr, (c0 + t) // 2] >> (4 * ((c0 + t) & 1))) & 0xF for t in range(32)]
        else:
            r0, cc = (blk // 64) * 32, blk % 64
            y = x[r0:r0 + 32, cc]
            got_s = r["scales"][r0 // 32, cc]
            got_c = [(r["codes"][(r0 + t) // 2, cc] >> (4 * ((r0 + t) & 1))) & 0xF for t in range(32)]
        want_s, want_c = _ref_block(y)
        assert got_s == want_s and got_c == want_c, blk


def test_closed_forms():
    ones = np.ones((1, 32), np.float32)
    r = oracle.mx_quantize(ones, 0)
    assert r["scales"][0, 0] == 125 and (r["codes"] == 0x66).all()      # scale 1/4, code 4 (value 4)
    np.testing.assert_array_equal(oracle.mx_dequantize(r["codes"], r["scales"], 1, 32, 0), ones)
    sev = np.full((1, 32), 7.0, np.float32)
    r = oracle.mx_quantize(sev, 0)
    assert r["scales"][0, 0] == 127                                      # scale 1: 7 clips to 6
    np.testing.assert_array_equal(oracle.mx_dequantize(r["codes"], r["scales"], 1, 32, 0), np.full((1, 32), 6.0))


def _rand(shape, seed):
    g = torch.Generator().manual_seed(seed)
    return torch.randn(*shape, generator=g).to(torch.bfloat16)


def _mxdeq(x, axis):
    r = oracle.mx_quantize(x, axis)
    return oracle.mx_dequantize(r["codes"], r["scales"], x.shape[0], x.shape[1], axis)


def test_attention_zero_keys_gives_mean_of_values():
    """K = 0: every e = 1, the block scale is 1/4 and every code 4, so every
    weight is exactly 1: O is the mean of the MXFP4 V rows."""
    q = _rand((1, 1, 64, 64), 1)
    k = torch.zeros(1, 1, 128, 64, dtype=torch.bfloat16)
    v = _rand((1, 1, 128, 64), 2)
    out, _ = oracle.attention_fwd(q, k, v, kv_tile=64, mx=True)
    vh = _mxdeq(v[0, 0].float().numpy(), 1)
    np.testing.assert_allclose(out[0], np.broadcast_to(vh.mean(0), (64, 64)), atol=2e-6)


def test_attention_worked_example():
    """Power-of-two probabilities 1, 1/2, 1/4, 1/16 and 1/256 (score factor 1
    with softmax scale ln 2): the 32-key block scale is 1/4, e / (1/4) = 4, 2,
    1, 1/4, 1/64 -> codes 4, 2, 1, 0 (1/4 ties between 0 and 1/2: the even
    code 0) and 0, so P^ = 1, 1/2, 1/4, 0, 0."""
    d = 32
    x = [0, -1, -2, -4] + [-8] * 28
    q = torch.zeros(1, 1, 1, d)
    q[0, 0, 0, 0] = 4.0
    k = torch.zeros(1, 1, 32, d)
    for j, xj in enumerate(x):
        k[0, 0, j, 0] = xj / 4.0
    v = _rand((1, 1, 32, d), 3)
    out, _ = oracle.attention_fwd(q.to(torch.bfloat16), k.to(torch.bfloat16), v, kv_tile=64,
                                  softmax_scale=float(np.float32(math.log(2.0))), mx=True)
    vh = _mxdeq(v[0, 0].float().numpy(), 1)
    e = np.array([2.0 ** xj for xj in x])
    p_hat = np.array([1.0, 0.5, 0.25] + [0.0] * 29)
    np.testing.assert_allclose(out[0, 0], (p_hat[:, None] * vh).sum(0) / e.sum(), atol=1e-6)


def test_nvfp4_with_scalesearch_is_more_accurate():
    """The ScaleSearch page's premise: scales with mantissa bits (and the
    offset search) beat power-of-two block scales."""
    g = torch.Generator().manual_seed(4)
    q, k, v = (torch.randn(1, 2, 256, 128, generator=g).to(torch.bfloat16) for _ in range(3))
    ex, _ = oracle.attention_exact(q, k, v, causal=True)
    nv, _ = oracle.attention_fwd(q, k, v, causal=True)
    mx, _ = oracle.attention_fwd(q, k, v, causal=True, mx=True)
    assert np.linalg.norm(nv - ex) < np.linalg.norm(mx - ex)


def test_smallest_scale_is_a_real_scale():
    """Byte 0 is the scale 2^-127, not a zero flag: a block whose maximum is
    2^-125 quantizes to code 4 at that scale."""
    y = np.zeros((1, 32), np.float32)
    y[0, 0] = np.float32(2.0 ** -125)
    r = oracle.mx_quantize(y, 0)
    assert r["scales"][0, 0] == 0 and (r["codes"][0, 0] & 0xF) == 6
    assert oracle.mx_dequantize(r["codes"], r["scales"], 1, 32, 0)[0, 0] == 2.0 ** -125


def test_attention_reference_is_the_power_of_two_above_the_tile_maximum():
    """A tile maximum of 0.5 (score factor 1): the MXFP4 tile reference is
    ceil(0.5) = 1, so e = 2^-0.5 and 2^-1.5 for scores 0.5 and -0.5; the block
    maximum 0.7071 has exponent -1, scale 2^-3, t = 5.66 -> 6 (P^ 0.75) and
    t = 2.83 -> 3 (P^ 0.375).  The denominator sums the e."""
    d = 32
    q = torch.zeros(1, 1, 1, d)
    q[0, 0, 0, 0] = 4.0
    k = torch.zeros(1, 1, 32, d)
    k[0, 0, :, 0] = -8.0          # x = -32: e ~ 1e-10, code 0
    k[0, 0, 0, 0] = 0.125         # x = 0.5
    k[0, 0, 1, 0] = -0.125        # x = -0.5
    v = _rand((1, 1, 32, d), 5)
    out, _ = oracle.attention_fwd(q.to(torch.bfloat16), k.to(torch.bfloat16), v, kv_tile=64,
                                  softmax_scale=float(np.float32(math.log(2.0))), mx=True)
    vh = _mxdeq(v[0, 0].float().numpy(), 1)
    e0, e1 = 2.0 ** -0.5, 2.0 ** -1.5
    want = (0.75 * vh[0] + 0.375 * vh[1]) / (e0 + e1 + 30 * 2.0 ** -33)
    np.testing.assert_allclose(out[0, 0], want, atol=1e-6)
