"""Pins of the oracle's number formats against library routines and exact rationals.

E2M1 grid and E4M3 scale format: ScaleSearch page, Declaracion del Problema
(NVFP4 = 4-bit elements with an 8-bit E4M3 block scale); Attn-QAT page, Resumo
tecnico / 1 (FP4 has 15 distinct values).
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle

GRID = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def test_e2m1_grid_and_15_distinct_values():
    vals = [oracle.e2m1_value(c) for c in range(16)]
    assert vals[:8] == GRID
    assert vals[8:] == [-g for g in GRID]
    assert len(set(vals)) == 15  # +0 and -0 coincide


def test_e4m3_decode_matches_torch_float8():
    raw = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = raw.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    ours = np.array([oracle.e4m3_value(b) for b in range(256)])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])
    assert oracle.e4m3_value(0x7E) == 448.0
    assert oracle.e4m3_value(0x01) == 2.0 ** -9
    assert oracle.e4m3_value(0x08) == 2.0 ** -6


def test_e4m3_encode_matches_torch_on_all_bf16_below_448():
    # every non-negative bf16 pattern up to 448: torch's float8_e4m3fn cast is
    # round-to-nearest-even there; above 448 the oracle saturates to 448.
    pats = torch.arange(0, 0x7F80, dtype=torch.int32).to(torch.int16).view(torch.bfloat16)
    v = pats.to(torch.float32)
    v = v[v <= 448.0]
    ref = v.to(torch.float8_e4m3fn).view(torch.uint8).to(torch.int32).numpy()
    ours = np.array([oracle.e4m3_encode(float(x)) for x in v.numpy()])
    assert np.array_equal(ours, ref)
    for big in (448.0, 463.9, 464.0, 1e6, 3.0e38):
        assert oracle.e4m3_encode(big) == 0x7E


def test_e4m3_encode_roundtrip_and_midpoints():
    for b in range(0x7F):
        assert oracle.e4m3_encode(oracle.e4m3_value(b)) == b
    # exact midpoints go to the even byte
    for b in range(0, 0x7E):
        mid = (Fraction(oracle.e4m3_value(b)) + Fraction(oracle.e4m3_value(b + 1))) / 2
        expect = b if b % 2 == 0 else b + 1
        assert oracle.e4m3_encode(float(mid)) == expect


def _nearest_even(t: Fraction) -> int:
    best = None
    for c, g in enumerate(GRID):
        d = abs(t - Fraction(g))
        if best is None or d < best[0] or (d == best[0] and c % 2 == 0):
            best = (d, c)
    return best[1]


def test_e2m1_encode_ties_and_dense_grid():
    ties = {0.25: 0, 0.75: 2, 1.25: 2, 1.75: 4, 2.5: 4, 3.5: 6, 5.0: 6}
    for t, c in ties.items():
        assert oracle.e2m1_encode(t) == c, t
    assert oracle.e2m1_encode(6.0) == 7 and oracle.e2m1_encode(100.0) == 7
    # saturation holds however large t is (binary64 distances to 4 and 6 coincide at 1e30)
    assert oracle.e2m1_encode(1e30) == 7 and oracle.e2m1_encode(3.0e38) == 7
    rng = np.random.default_rng(0)
    ts = np.concatenate([rng.uniform(0, 7, 3000), np.arange(0, 7, 1 / 64)]).astype(np.float32)
    for t in ts:
        assert oracle.e2m1_encode(float(t)) == _nearest_even(Fraction(float(t))), t


def test_reciprocal_is_correctly_rounded():
    for b in range(1, 0x7F):
        s = Fraction(oracle.e4m3_value(b))
        r = oracle.recip(b)
        exact = 1 / s
        # distance to the next binary32 neighbours must not be smaller
        up = np.nextafter(np.float32(r), np.float32(np.inf))
        dn = np.nextafter(np.float32(r), np.float32(0))
        d = abs(Fraction(float(r)) - exact)
        assert d <= abs(Fraction(float(up)) - exact)
        assert d <= abs(Fraction(float(dn)) - exact)


def test_round_fp16_matches_numpy():
    rng = np.random.default_rng(1)
    xs = np.concatenate([rng.standard_normal(20000) * 10.0 ** rng.uniform(-9, 4, 20000),
                         [0.0, 65504.0, 2.0 ** -24, 2.0 ** -25, 3 * 2.0 ** -26, 1e-9]])
    ours = np.array([oracle.round_fp16(float(x)) for x in xs])
    ref = xs.astype(np.float16).astype(np.float64)
    assert np.array_equal(ours, ref)


def test_score_factor_ln2_gives_one():
    # softmax_scale = ln 2 makes the base-2 score factor exactly 1 (used by worked examples)
    assert oracle.score_factor(float(np.log(2.0)), 16) == 1.0
    assert oracle.score_factor(0.0, 64) == np.float32(1.4426950408889634 / 8.0)
