"""Pins of the oracle's fake-quant FP4 attention forward.

ScaleSearch page, Metodologia / ScaleSearchAttention (QK^T and PV on NVFP4
operands with FP32 accumulation); ThriftAttention page, Metodologia / 2 (FP16
path for selected block pairs, FP4 path with two-level P for the rest, both
fused by an online softmax in the manner of FlashAttention-2).
"""
import math
import os

import numpy as np
import pytest
import torch

import oracle

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _rand(shape, seed, dtype=torch.bfloat16):
    g = torch.Generator().manual_seed(seed)
    return torch.randn(*shape, generator=g).to(dtype)


def _deq(x, axis, ss=True):
    r = oracle.quantize(x, axis, ss)
    return oracle.dequantize(r["codes"], r["scales"], x.shape[0], x.shape[1], axis)


def test_two_level_p_worked_example():
    rows = []
    with open(os.path.join(GOLD, "two_level_p_worked.txt")) as f:
        for line in f:
            line = line.split("#")[0].strip()
            if line:
                rows.append(line.split())
    n = len(rows)
    assert n == 32
    d = 32
    q = np.zeros((1, 1, 1, d), np.float32)
    q[..., 0] = 1.0
    k = np.zeros((1, 1, n, d), np.float32)
    v = np.zeros((1, 1, n, d), np.float32)
    for j, r in enumerate(rows):
        k[0, 0, j, 0] = float(r[1])
        v[0, 0, j, j] = 1.0
    # preconditions: the inputs are exact in NVFP4 under ScaleSearch
    assert np.array_equal(_deq(k[0, 0], 0), k[0, 0])
    assert np.array_equal(_deq(v[0, 0], 1), v[0, 0])
    assert np.array_equal(_deq(q[0, 0], 0), q[0, 0])
    out, lse = oracle.attention_fwd(q, k, v, causal=False, softmax_scale=math.log(2.0), kv_tile=32)
    e = np.array([np.float32(2.0) ** np.float32(float(r[1])) for r in rows], np.float64)
    e[6] = float(np.float32(2.0 ** -0.5))
    l = e.sum()
    phat = np.array([float(r[5]) for r in rows])
    expect = phat / 2688.0 / l
    np.testing.assert_allclose(out[0, 0], expect, rtol=1e-6, atol=1e-9)
    assert abs(lse[0, 0] - math.log(l)) < 1e-6
    # rounding ambiguity: keys 3 and 19 sit exactly on the E2M1 midpoint 0.75
    # (ties to the even code, value 1; the other rounding is 0.5).  Under any
    # positive slack each can move its weight by 0.5 * s2 (448 and 56), each V
    # row has max 1, and no scale input (448, 56) is near an E4M3 boundary:
    # amb = (0.5 * 448 + 0.5 * 56) / 2688 / l.  Zero slack leaves both closed.
    *_, amb = oracle.attention_fwd(q, k, v, causal=False, softmax_scale=math.log(2.0), kv_tile=32,
                                   tie_slack=(1e-6, 0.0))
    assert abs(amb[0, 0] - (0.5 * 448 + 0.5 * 56) / 2688.0 / l) < 1e-12
    *_, amb0 = oracle.attention_fwd(q, k, v, causal=False, softmax_scale=math.log(2.0), kv_tile=32,
                                    tie_slack=(0.0, 0.0))
    assert amb0[0, 0] == 0.0
    # the output with key 3's code taken the other way moves by exactly its share of the bound
    alt = expect.copy()
    alt[3] = 0.5 * 448 / 2688.0 / l
    assert abs(np.abs(alt - expect).max() - 0.5 * 448 / 2688.0 / l) < 1e-12


def test_zero_keys_closed_form_mean_of_dequantized_v():
    # K = 0: all scores 0, e = 1 on every visible key, P' = 2688 -> s2 = 448, code 6:
    # every probability is exactly 1/n, so O is the mean of the dequantized V rows.
    q = _rand((1, 1, 200, 64), 0)
    k = torch.zeros(1, 1, 208, 64, dtype=torch.bfloat16)
    v = _rand((1, 1, 208, 64), 1)
    vh = _deq(v[0, 0].float().numpy(), 1)
    out, lse = oracle.attention_fwd(q, k[:, :, :200 + 8], v, causal=False, kv_tile=64)
    np.testing.assert_allclose(out[0], np.broadcast_to(vh.mean(0), (200, 64)), rtol=0, atol=2e-6)
    np.testing.assert_allclose(lse[0], math.log(208), atol=1e-5)
    # every t is 6 and every block scale input 448: no decision is near a
    # rounding boundary, so the ambiguity bound is exactly 0 under a slack far
    # larger than any binary32 evaluation error
    *_, amb = oracle.attention_fwd(q, k[:, :, :200 + 8], v, causal=False, kv_tile=64, tie_slack=(1e-3, 1e-4))
    assert np.all(amb == 0.0)
    # causal: row i sees i+1 keys
    q2 = _rand((1, 1, 208, 64), 2)
    out, _ = oracle.attention_fwd(q2, k, v, causal=True, kv_tile=64)
    cm = np.cumsum(vh, 0) / np.arange(1, 209)[:, None]
    np.testing.assert_allclose(out[0], cm, atol=2e-6)


def test_causal_first_row_is_first_value_row():
    q, k, v = _rand((1, 2, 128, 64), 3), _rand((1, 2, 128, 64), 4), _rand((1, 2, 128, 64), 5)
    out, _ = oracle.attention_fwd(q, k, v, causal=True, kv_tile=64, rows=[0])
    for h in range(2):
        vh = _deq(v[0, h].float().numpy(), 1)
        np.testing.assert_allclose(out[h, 0], vh[0], atol=1e-7)


def test_full_budget_equals_fp16_textbook_attention():
    # every pair promoted: the FP16 path alone, i.e. softmax attention on fp16
    # operands with fp16 probabilities
    B, H, S, d = 1, 2, 256, 64
    q, k, v = _rand((B, H, S, d), 6), _rand((B, H, S, d), 7), _rand((B, H, S, d), 8)
    for causal in (False, True):
        out, lse = oracle.attention_fwd(q, k, v, causal=causal, kv_tile=128, pct=100, sel_block=128)
        ex, exl = oracle.attention_exact(q, k, v, causal=causal)
        qf = q.to(torch.float16).double().numpy()
        kf = k.to(torch.float16).double().numpy()
        vf = v.to(torch.float16).double().numpy()
        s = np.einsum("bhid,bhjd->bhij", qf, kf) / math.sqrt(d)
        if causal:
            s = np.where(np.tril(np.ones((S, S), bool)), s, -np.inf)
        p = np.exp(s - s.max(-1, keepdims=True))
        ref = (p / p.sum(-1, keepdims=True)) @ vf
        np.testing.assert_allclose(out.reshape(B, H, S, d), ref, atol=1e-3)
        assert np.abs(out - ex).max() < 2e-3
        np.testing.assert_allclose(lse, exl, atol=1e-5)


def test_fp4_path_error_is_quantization_sized():
    B, H, S, d = 1, 2, 256, 64
    q, k, v = _rand((B, H, S, d), 9), _rand((B, H, S, d), 10), _rand((B, H, S, d), 11)
    out, _ = oracle.attention_fwd(q, k, v, causal=False, kv_tile=64)
    ex, _ = oracle.attention_exact(q, k, v, causal=False)
    rel = np.linalg.norm(out - ex) / np.linalg.norm(ex)
    assert 0.02 < rel < 0.35
    # a partial budget lands between the FP4 path and the FP16 path
    out50, _ = oracle.attention_fwd(q, k, v, causal=False, kv_tile=64, pct=50, sel_block=128)
    rel50 = np.linalg.norm(out50 - ex) / np.linalg.norm(ex)
    assert rel50 < rel


def test_lse_consistency_with_quantized_scores():
    B, H, S, d = 1, 1, 192, 64
    q, k, v = _rand((B, H, S, d), 12), _rand((B, H, S, d), 13), _rand((B, H, S, d), 14)
    out, lse = oracle.attention_fwd(q, k, v, causal=True, kv_tile=64)
    qh = _deq(q[0, 0].float().numpy(), 0)
    kh = _deq(k[0, 0].float().numpy(), 0)
    s = qh @ kh.T / math.sqrt(d)
    for i in range(S):
        tot = np.exp(s[i, : i + 1] - lse[0, i]).sum()
        assert abs(tot - 1.0) < 1e-5


def test_power_of_two_value_scaling_is_exact():
    q, k, v = _rand((1, 1, 128, 64), 15), _rand((1, 1, 128, 64), 16), _rand((1, 1, 128, 64), 17)
    o1, _ = oracle.attention_fwd(q, k, v, causal=True, kv_tile=64)
    o2, _ = oracle.attention_fwd(q, k, v * 4, causal=True, kv_tile=64)
    np.testing.assert_allclose(o2, 4 * o1, rtol=1e-6, atol=1e-7)


def test_key_permutation_inside_16_blocks_is_invariant():
    # quantization blocks of K run along d (per key) and of V along 16 tokens;
    # P's level-2 blocks are 16 keys: permuting keys inside a 16-key block changes nothing
    q, k, v = _rand((1, 1, 96, 64), 18), _rand((1, 1, 128, 64), 19), _rand((1, 1, 128, 64), 20)
    perm = np.arange(128)
    rng = np.random.default_rng(0)
    for b in range(8):
        perm[16 * b:16 * b + 16] = 16 * b + rng.permutation(16)
    o1, l1 = oracle.attention_fwd(q, k, v, causal=False, kv_tile=64)
    o2, l2 = oracle.attention_fwd(q, k[:, :, perm], v[:, :, perm], causal=False, kv_tile=64)
    np.testing.assert_allclose(o1, o2, rtol=1e-6, atol=1e-7)
    np.testing.assert_allclose(l1, l2, atol=1e-6)


def test_row_and_head_selection_consistent():
    q, k, v = _rand((2, 2, 80, 32), 21), _rand((2, 1, 80, 32), 22), _rand((2, 1, 80, 32), 23)
    full, lf = oracle.attention_fwd(q, k, v, causal=True, kv_tile=32)
    part, lp = oracle.attention_fwd(q, k, v, causal=True, kv_tile=32, rows=[79, 3, 40], heads=[3, 0])
    np.testing.assert_array_equal(part[0], full[3][[79, 3, 40]])
    np.testing.assert_array_equal(part[1], full[0][[79, 3, 40]])
    np.testing.assert_array_equal(lp[1], lf[0][[79, 3, 40]])


# ---- single-level P (Attn-QAT page, Metodologia / B: FP4 attention without the
# two-level step): P takes only the NVFP4 block scale E4M3(amax(e)/6)

def test_single_level_p_zero_keys_closed_form():
    """K = 0: every e = 1, so each block's scale is E4M3(1/6) = 0x23 =
    0.171875 and t = 1 * R(0x23) = 5.818 rounds to code 6: every weight is
    6 * 0.171875 = 1.03125 against a denominator of n, so O is 1.03125 times
    the mean of the dequantized V rows (the two-level P gives exactly the
    mean: its row level maps e = 1 to 2688 = 6 * 448)."""
    q = _rand((1, 1, 64, 64), 10)
    k = torch.zeros(1, 1, 192, 64, dtype=torch.bfloat16)
    v = _rand((1, 1, 192, 64), 11)
    vh = _deq(v[0, 0].float().numpy(), 1)
    out, lse = oracle.attention_fwd(q, k, v, kv_tile=64, single_level_p=True)
    np.testing.assert_allclose(out[0], np.broadcast_to(1.03125 * vh.mean(0), (64, 64)), rtol=0, atol=2e-6)
    np.testing.assert_allclose(lse[0], math.log(192), atol=1e-5)  # the denominator sums the unquantized e


def test_single_level_p_worked_example():
    """Scores built so that e is a power of two (softmax scale ln 2 makes the
    score factor exactly 1; q = 4 e_0 and k_j = -a_j e_0 quantize exactly under
    ScaleSearch).  One 16-key block with e = 1, 1/2, 1/4, 1/16, 1/256 and
    eleven keys at e = 1/256: s2 = E4M3(1/6) = 0.171875, R(s2) = fl32(1/s2)
    = 5.8181815, so t = 5.818, 2.909, 1.4545, 0.3636, 0.0227 -> E2M1 6, 3,
    1.5, 0.5, 0 -> P^ = 1.03125, 0.515625, 0.2578125, 0.0859375, 0."""
    d = 16
    x = [0, -1, -2, -4] + [-8] * 12             # tile-row maximum 0
    q = torch.zeros(1, 1, 1, d)
    q[0, 0, 0, 0] = 4.0
    k = torch.zeros(1, 1, 16, d)
    for j, xj in enumerate(x):
        k[0, 0, j, 0] = xj / 4.0
    v = _rand((1, 1, 16, d), 12)  # any values: the check goes through the dequantized V
    vh = _deq(v[0, 0].float().numpy(), 1)
    out, lse = oracle.attention_fwd(q.to(torch.bfloat16), k.to(torch.bfloat16), v, kv_tile=64,
                                    softmax_scale=float(np.float32(math.log(2.0))), single_level_p=True)
    e = np.array([2.0 ** xj for xj in x])
    p_hat = np.array([1.03125, 0.515625, 0.2578125, 0.0859375] + [0.0] * 12)
    want = (p_hat[:, None] * vh).sum(0) / e.sum()
    np.testing.assert_allclose(out[0, 0], want, rtol=0, atol=1e-6)
    # the two-level P of the same scores keeps e = 1/2 and 1/4 exactly (s2 = 448)
    two, _ = oracle.attention_fwd(q.to(torch.bfloat16), k.to(torch.bfloat16), v, kv_tile=64,
                                  softmax_scale=float(np.float32(math.log(2.0))))
    assert np.abs(two[0, 0] - want).max() > 1e-3


# ---- the FP4/FP16 mix at a partial budget (ThriftAttention page, Metodologia /
# 1 and 2): a closed form that does not go through the oracle's attention code
# (tests/mix_closed_form.py explains the construction)

import mix_closed_form as mcf  # noqa: E402


def _mix_case(H, S, d, kv_tile, sel_block, causal, pct, seed, zero_keys=False):
    q, k, v, a = mcf.construct(H, S, d, kv_tile, seed, zero_keys=zero_keys)
    assert mcf.operands_exact(q, k)
    scale = 0.25 / d
    want, wlse = mcf.expected(q, k, v, a, causal, pct, sel_block, scale, kv_tile)
    return q, k, v, a, scale, want, wlse


@pytest.mark.parametrize("kv_tile,sel_block", [(64, 128), (128, 128), (64, 256)])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("pct", [10, 34, 50])
def test_partial_budget_mix_closed_form(kv_tile, sel_block, causal, pct):
    H, S, d = 2, 704, 64  # 5.5 selection blocks of 128: a ragged last block
    q, k, v, a, scale, want, wlse = _mix_case(H, S, d, kv_tile, sel_block, causal, pct, seed=pct + 7 * kv_tile)
    out, lse, idx, cnt = oracle.attention_fwd(q, k, v, causal=causal, softmax_scale=scale, kv_tile=kv_tile,
                                              pct=pct, sel_block=sel_block, with_topk=True)
    np.testing.assert_allclose(out, want, rtol=0, atol=1e-6)
    np.testing.assert_allclose(lse, wlse, rtol=0, atol=1e-6)
    # the oracle's selection is the construction's ranking
    for h in range(H):
        sel = mcf.selection(a[h], S, causal, pct, sel_block)
        for i, s in enumerate(sel):
            assert cnt[h, i] == len(s)
            assert list(idx[h, i, : cnt[h, i]]) == s
            assert all(x == -1 for x in idx[h, i, cnt[h, i]:])


@pytest.mark.parametrize("causal", [False, True])
def test_partial_budget_zero_keys_promote_lowest_blocks(causal):
    """K = 0: every score ties, so the lowest visible blocks are promoted and
    O_i is the mean of fp16(V) over their keys and of V^ over the rest."""
    H, S, d, pct = 1, 640, 64, 34
    q, k, v, a, scale, want, wlse = _mix_case(H, S, d, 64, 128, causal, pct, seed=3, zero_keys=True)
    out, lse, idx, cnt = oracle.attention_fwd(q, k, v, causal=causal, softmax_scale=scale, kv_tile=64,
                                              pct=pct, sel_block=128, with_topk=True)
    np.testing.assert_allclose(out, want, rtol=0, atol=1e-6)
    np.testing.assert_allclose(lse[0], np.log(np.arange(1, S + 1) if causal else np.full(S, S)), atol=1e-6)
    for i in range(5):
        n = i + 1 if causal else 5
        kc = -(-pct * n // 100)
        assert list(idx[0, i, : cnt[0, i]]) == list(range(kc))
    # the same mean written out directly for the last row
    vb = v[0, 0]
    r = oracle.quantize(vb, 1, True)
    vh = oracle.dequantize(r["codes"], r["scales"], S, d, 1).astype(np.float64)
    v16 = vb.to(torch.float16).double().numpy()
    kc = -(-pct * 5 // 100)
    w = np.concatenate([v16[: 128 * kc], vh[128 * kc:]])
    np.testing.assert_allclose(out[0, S - 1], w.mean(0), atol=1e-6)


def test_partial_budget_closed_form_tells_wrong_maps_apart():
    """The closed form is sensitive to the mistakes it is meant to catch: a
    tile index taken for the block index (identical at kv_tile = sel_block,
    wrong at 64 against 128), a block shifted by one, and FP4 weights left in
    units of 2688 e.  Each moves the output far beyond the pin's 1e-6."""
    H, S, d, kv_tile, sel_block, pct = 2, 704, 64, 64, 128, 34
    q, k, v, a, scale, want, _ = _mix_case(H, S, d, kv_tile, sel_block, True, pct, seed=5)
    by_tile, _ = mcf.expected(q, k, v, a, True, pct, sel_block, scale, kv_tile, block_of_key=lambda j: j // kv_tile)
    shifted, _ = mcf.expected(q, k, v, a, True, pct, sel_block, scale, kv_tile,
                              block_of_key=lambda j: j // sel_block + 1)
    assert np.abs(by_tile - want).max() > 1e-3
    assert np.abs(shifted - want).max() > 1e-3
    out, _ = oracle.attention_fwd(q, k, v, causal=True, softmax_scale=scale, kv_tile=kv_tile, pct=pct,
                                  sel_block=sel_block)
    assert np.abs(out - by_tile).max() > 1e-3 and np.abs(out - shifted).max() > 1e-3
    # the units: with the FP4 weights 2688 times too large, rows mixing both paths move
    _, Hn, Sn, dn = q.shape
    qf, kf = q[0].float().double().numpy(), k[0].float().double().numpy()
    c = float(np.float32(math.log2(math.e) * scale))
    h, i = 0, S - 1
    vb = v[0, h]
    r = oracle.quantize(vb, 1, True)
    vh = oracle.dequantize(r["codes"], r["scales"], S, d, 1).astype(np.float64)
    v16 = vb.to(torch.float16).double().numpy()
    x = (qf[h, i] @ kf[h].T).astype(np.float32) * np.float32(c)
    p = np.exp2(x.astype(np.float64) - x.max())
    chosen = set(mcf.selection(a[h], S, True, pct, sel_block)[i // sel_block])
    prom = np.array([j // sel_block in chosen for j in range(S)])
    p_bad = np.where(prom, p, 2688.0 * p)
    w = np.where(prom[:, None], v16, vh)
    bad = (p_bad[:, None] * w).sum(0) / p.sum()
    assert np.abs(bad - out[h, i]).max() > 1e-3


def test_rounding_ambiguity_bound_is_rare_and_grows_with_slack():
    """On random inputs few rows have an open P decision under a slack of a
    few binary32 ulps, the bound grows with the slack, and it vanishes at zero
    slack (no input lands exactly on a boundary here)."""
    q, k, v = _rand((1, 2, 512, 64), 31), _rand((1, 2, 512, 64), 32), _rand((1, 2, 512, 64), 33)
    *_, a0 = oracle.attention_fwd(q, k, v, causal=True, kv_tile=64, tie_slack=(0.0, 0.0))
    *_, a1 = oracle.attention_fwd(q, k, v, causal=True, kv_tile=64, tie_slack=(2.0 ** -20, 2.0 ** -22))
    *_, a2 = oracle.attention_fwd(q, k, v, causal=True, kv_tile=64, tie_slack=(2.0 ** -10, 2.0 ** -12))
    assert np.all(a0 == 0.0)
    assert np.all(a2 >= a1) and np.count_nonzero(a1) <= 0.02 * a1.size
    assert np.count_nonzero(a2) > np.count_nonzero(a1)
