"""GPU parity of the magnitude-balancing pair Q' = Q R^-T, K' = K R with
R = diag(2^e) (ScaleSearch page, Metodologia / ScaleSearchAttention): the
exponents (integers decided in binary64), the balanced quantization (codes and
scales bit-exact) and the attention forward (the oracle's tolerance)."""
import math

import numpy as np
import pytest
import torch

import oracle
from block_scaled_fp4_amd import synth
from gpu_helpers import TIE_SLACK, assert_close_attn_rows, case

pytestmark = pytest.mark.gpu


def _margins(q, k):
    """Distance, in binary exponent units, of each channel's ms_q / ms_k from
    the nearest decision boundary 4^(2e+1): the exponents may depend on the
    order of the binary64 sums only when this is a few ulps."""
    qf, kf = q.float().numpy().astype(np.float64), k.float().numpy().astype(np.float64)
    B, H, Sq, d = qf.shape
    Hkv = kf.shape[1]
    G = H // Hkv
    m = np.full((B, Hkv, d), np.inf)
    for b in range(B):
        for hk in range(Hkv):
            mq = (qf[b, hk * G:(hk + 1) * G] ** 2).mean(axis=(0, 1))
            mk = (kf[b, hk] ** 2).mean(axis=0)
            ok = (mq > 0) & (mk > 0)
            x = np.log2(mq[ok] / mk[ok])
            m[b, hk, ok] = np.abs(x - (4 * np.round((x - 2) / 4) + 2))
    return m


def _check_exponents(fp4, q, k, what):
    e = fp4.fp4_qk_balance(q.cuda(), k.cuda())
    torch.cuda.synchronize()
    ref = oracle.balance_exponents(q, k)
    far = _margins(q, k) > 1e-9
    assert far.mean() > 0.99, what
    got = e.cpu().numpy()
    np.testing.assert_array_equal(got[far], ref[far], err_msg=what)
    return e, ref


@pytest.mark.parametrize("B,H,Hkv,S,d", [(1, 2, 2, 384, 128), (2, 8, 2, 200, 64), (1, 4, 1, 1040, 128)])
def test_exponents_match_the_oracle(gpu, B, H, Hkv, S, d):
    q, k, _ = synth.qkv(B, H, S, d, seed=160 + d, Hkv=Hkv, k_outliers=4)
    case(f"balance exponents B={B} H={H} Hkv={Hkv} S={S} d={d}")
    e, ref = _check_exponents(gpu, q, k, "exponents")
    assert np.abs(ref).max() >= 1


def test_exponents_closed_form(gpu):
    """Q channel 3 at +-1 against K channel 3 at +-16: e = -2 (the pair's
    magnitudes meet at 4); the other channels (all ones) stay at 0."""
    d = 64
    q = torch.ones(1, 1, 32, d)
    k = torch.ones(1, 1, 48, d)
    sgn = torch.tensor([1.0, -1.0]).repeat(24)
    q[0, 0, :, 3] = sgn[:32]
    k[0, 0, :, 3] = 16 * sgn[:48]
    case("balance exponents closed form")
    e = gpu.fp4_qk_balance(q.to(torch.bfloat16).cuda(), k.to(torch.bfloat16).cuda())
    torch.cuda.synchronize()
    want = np.zeros((1, 1, d), np.int32)
    want[0, 0, 3] = -2
    np.testing.assert_array_equal(e.cpu().numpy(), want)


@pytest.mark.parametrize("had", [False, True])
def test_balanced_quantization_bit_exact(gpu, had):
    B, H, Hkv, S, d = 1, 4, 2, 256, 128
    q, k, _ = synth.qkv(B, H, S, d, seed=170, Hkv=Hkv, k_outliers=4)
    case(f"balanced quantization hadamard={had}")
    e, ref = _check_exponents(gpu, q, k, "exponents")
    signs = [0x9E3779B9, 0x7F4A7C15, 0x2545F491, 0xD1B54A32] if had else None
    qb, kb = oracle.balance_apply(q, k, ref)
    gmode = gpu.GLOBAL_NONE
    for x, xb, neg, rows in ((q, qb, True, (H // Hkv) * S), (k, kb, False, S)):
        r = gpu.fp4_quantize(x.cuda().view(-1, d), 0, True, -2, 6, gmode, channel_exp=e.view(-1, d),
                             exp_negate=neg, exp_rows=rows, hadamard=had, hadamard_signs=signs)
        torch.cuda.synchronize()
        src = oracle.hadamard_rows(xb, signs) if had else xb
        o = oracle.quantize(src.reshape(-1, d), 0, True, -2, 6, 0)
        np.testing.assert_array_equal(r["codes"].cpu().numpy(), o["codes"])
        np.testing.assert_array_equal(r["scales"].cpu().numpy(), o["scales"])


@pytest.mark.parametrize("causal,pct,had,kv_tile", [(True, 0, False, 128), (False, 0, False, 64), (True, 30, False, 128),
                                                    (True, 0, True, 128), (True, 30, True, 64)])
def test_balanced_attention(gpu, causal, pct, had, kv_tile):
    B, H, Hkv, S, d = 1, 4, 2, 640, 128
    q, k, v = synth.qkv(B, H, S, d, seed=180, Hkv=Hkv, k_outliers=4)
    _check_exponents(gpu, q, k, "exponents")
    signs = [0x9E3779B9, 0x7F4A7C15, 0x2545F491, 0xD1B54A32] if had else None
    case(f"balanced attention causal={causal} pct={pct} hadamard={had} kv_tile={kv_tile}")
    out, lse = gpu.fp4_attention_fwd(q.cuda(), k.cuda(), v.cuda(), causal=causal, kv_tile=kv_tile,
                                     fp16_budget_pct=pct, out_dtype=gpu.FP32, balance=True, hadamard=had,
                                     hadamard_signs=signs)
    torch.cuda.synchronize()
    ref, rlse, amb = oracle.attention_fwd(q, k, v, causal=causal, kv_tile=kv_tile, pct=pct, balance=True,
                                          hadamard=had, signs=signs, tie_slack=TIE_SLACK)
    assert_close_attn_rows(out.cpu().numpy().reshape(ref.shape), ref, amb, "balanced attention")
    np.testing.assert_allclose(lse.cpu().numpy().reshape(rlse.shape), rlse, atol=1e-3)
    plain, _ = oracle.attention_fwd(q, k, v, causal=causal, kv_tile=kv_tile, pct=pct, hadamard=had, signs=signs)
    assert np.abs(plain - ref).max() > 1e-3  # the option changes the FP4 operands: the test tells them apart


def test_balanced_prefill_workload_heads(gpu):
    """B=1, H=32, S=8192, d=128, causal, K outlier channels: every row of
    heads 0 and 31 with the balance pair, and lower error against exact
    attention than without it."""
    q, k, v = synth.prefill(S=8192)
    heads = [0, 31]
    case("balanced attention prefill 8K, heads 0 and 31")
    _check_exponents(gpu, q, k, "exponents 8K")
    out, _ = gpu.fp4_attention_fwd(q.cuda(), k.cuda(), v.cuda(), causal=True, out_dtype=gpu.FP32, balance=True)
    torch.cuda.synchronize()
    ref, _, amb = oracle.attention_fwd(q, k, v, causal=True, balance=True, heads=heads, tie_slack=TIE_SLACK)
    got = out.cpu().numpy().reshape(32, 8192, 128)[heads]
    assert_close_attn_rows(got, ref, amb, "balanced prefill 8K")
    ex, _ = oracle.attention_exact(q, k, v, causal=True, heads=heads, rows=list(range(0, 8192, 64)))
    plain, _ = gpu.fp4_attention_fwd(q.cuda(), k.cuda(), v.cuda(), causal=True, out_dtype=gpu.FP32)
    torch.cuda.synchronize()
    pl = plain.cpu().numpy().reshape(32, 8192, 128)[heads][:, ::64]
    rel = lambda a: np.linalg.norm(a - ex) / np.linalg.norm(ex)
    assert rel(got[:, ::64]) < rel(pl)
