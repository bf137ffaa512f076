"""GPU attention-forward parity against the oracle's fake-quant numerics
(ScaleSearch page, Metodologia / ScaleSearchAttention; ThriftAttention page,
Metodologia / 2).  Outputs in binary32, max-abs 2e-3 and relative L2 1e-3."""
import math

import numpy as np
import pytest
import torch

import oracle
from block_scaled_fp4_amd import synth
from gpu_helpers import assert_close_attn, case

pytestmark = pytest.mark.gpu


def _gpu(fp4, q, k, v, **kw):
    out, lse, idx, cnt = fp4.fp4_attention_fwd(q.cuda(), k.cuda(), v.cuda(), out_dtype=fp4.FP32, return_topk=True,
                                               **kw)
    torch.cuda.synchronize()
    return out.cpu().numpy(), lse.cpu().numpy(), idx, cnt


def _check(fp4, q, k, v, causal, kv_tile, search, pct=0, rows=None, heads=None, softmax_scale=0.0):
    B, H, Sq, d = q.shape
    out, lse, idx, cnt = _gpu(fp4, q, k, v, causal=causal, kv_tile=kv_tile, scale_search=search,
                              fp16_budget_pct=pct, softmax_scale=softmax_scale)
    ref, rlse = oracle.attention_fwd(q, k, v, causal=causal, kv_tile=kv_tile, scale_search=search, pct=pct,
                                     sel_block=128, rows=rows, heads=heads,
                                     softmax_scale=float(np.float32(softmax_scale)))
    got = out.reshape(B * H, Sq, d)
    gl = lse.reshape(B * H, Sq)
    if heads is not None:
        got, gl = got[heads], gl[heads]
    if rows is not None:
        got, gl = got[:, rows], gl[:, rows]
    assert_close_attn(got, ref)
    np.testing.assert_allclose(gl, rlse, atol=1e-3)
    return out, idx, cnt


def test_tiny_config(gpu):
    """B=1 H=1 S=256 d=64 fp16, non-causal, max-scaling only, no FP16 path, 64x64 tiles."""
    q, k, v = synth.tiny()
    case("attn tiny 256x64 non-causal kv_tile 64")
    _check(gpu, q, k, v, causal=False, kv_tile=64, search=False)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("kv_tile", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_ragged_tiles(gpu, d, kv_tile, causal):
    # 400 = 3*128 + 16: several key tiles, a ragged last tile and a ragged query tile
    q, k, v = synth.qkv(1, 2, 400, d, seed=5, k_outliers=4)
    case(f"attn ragged S=400 d={d} kv_tile={kv_tile} causal={causal}")
    _check(gpu, q, k, v, causal=causal, kv_tile=kv_tile, search=True)


def test_gqa_and_cross_lengths(gpu):
    q, k, v = synth.qkv(2, 4, 200, 128, Hkv=2, Sk=336, seed=6)
    case("attn gqa Sq=200 Sk=336 non-causal")
    _check(gpu, q, k, v, causal=False, kv_tile=128, search=True)


def test_fp16_inputs_and_custom_scale(gpu):
    q, k, v = synth.qkv(1, 2, 256, 64, dtype=torch.float16, seed=7)
    case("attn fp16 inputs softmax_scale=0.2")
    _check(gpu, q, k, v, causal=True, kv_tile=64, search=True, softmax_scale=0.2)


@pytest.mark.parametrize("pct", [10, 30, 100])
def test_selective_fp16_path(gpu, pct):
    q, k, v = synth.qkv(1, 2, 1024 + 64, 128, seed=8, k_outliers=4)
    case(f"attn selective pct={pct} S=1088 causal")
    out, idx, cnt = _check(gpu, q, k, v, causal=True, kv_tile=128, search=True, pct=pct)
    assert idx is not None and cnt is not None


def test_full_budget_equals_textbook_fp16_attention(gpu):
    """All block pairs on the FP16 path: softmax attention with fp16 operands."""
    q, k, v = synth.qkv(1, 2, 384, 128, seed=9)
    case("attn pct=100 vs textbook")
    out, _, _, _ = _gpu(gpu, q, k, v, causal=True, kv_tile=128, fp16_budget_pct=100)
    qf, kf, vf = (t.to(torch.float16).double().numpy() for t in (q, k, v))
    s = np.einsum("bhid,bhjd->bhij", qf, kf) / math.sqrt(128)
    s = np.where(np.tril(np.ones((384, 384), bool)), s, -np.inf)
    p = np.exp(s - s.max(-1, keepdims=True))
    ref = (p / p.sum(-1, keepdims=True)) @ vf
    assert_close_attn(out, ref, "pct=100 vs textbook")


def test_zero_keys_give_mean_of_values(gpu):
    q, _, v = synth.qkv(1, 1, 256, 128, seed=10)
    k = torch.zeros_like(v)
    case("attn zero keys")
    out, lse, _, _ = _gpu(gpu, q, k, v, causal=False, kv_tile=128)
    r = oracle.quantize(v[0, 0], 1, True)
    vh = oracle.dequantize(r["codes"], r["scales"], 256, 128, 1)
    np.testing.assert_allclose(out[0, 0], np.broadcast_to(vh.mean(0), (256, 128)), atol=1e-5)
    np.testing.assert_allclose(lse[0, 0], math.log(256), atol=1e-5)


def test_bf16_output_and_prequantized_operands(gpu):
    q, k, v = synth.qkv(1, 2, 256, 128, seed=11)
    qc, kc, vc = q.cuda(), k.cuda(), v.cuda()
    case("attn prequantized operands")
    rq = gpu.fp4_quantize(qc.view(-1, 128), 0, True)
    rk = gpu.fp4_quantize(kc.view(-1, 128), 0, True)
    rv = gpu.fp4_quantize(vc.view(-1, 128), 1, True)
    quant = dict(q_codes=rq["codes"], q_scales=rq["scales"], k_codes=rk["codes"], k_scales=rk["scales"],
                 v_codes=rv["codes"], v_scales=rv["scales"], q_shape=(1, 2, 256, 128), kv_shape=(2, 256))
    o1, _ = gpu.fp4_attention_fwd(None, None, None, causal=True, out_dtype=gpu.FP32, quantized=quant)
    o2, _ = gpu.fp4_attention_fwd(qc, kc, vc, causal=True, out_dtype=gpu.FP32)
    o3, _ = gpu.fp4_attention_fwd(qc, kc, vc, causal=True, out_dtype=gpu.BF16)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2)
    assert (o3.float() - o2).abs().max().item() <= 2 ** -8 * max(1.0, o2.abs().max().item())


def test_prefill_workload_sampled_rows(gpu):
    """B=1, H=32, S=8192, d=128, causal, ScaleSearch Q/K/V, two-level P, kv_tile 128."""
    q, k, v = synth.prefill(S=8192)
    rows = sorted(set([0, 1, 127, 128, 4095, 8191] + list(range(37, 8192, 523))))
    heads = [0, 13, 31]
    case("attn prefill 8K causal full size, sampled rows")
    _check(gpu, q, k, v, causal=True, kv_tile=128, search=True, rows=rows, heads=heads)


def test_selective_workload_sampled_rows(gpu):
    """B=1, H=32, S=32768, causal, top 10% 128x128 block pairs on the FP16 path."""
    q, k, v = synth.prefill(S=32768)
    rows = [0, 130, 5000, 16383, 16384, 29999, 32767]
    heads = [0, 31]
    case("attn selective 32K causal full size, sampled rows")
    out, idx, cnt = _check(gpu, q, k, v, causal=True, kv_tile=128, search=True, pct=10, rows=rows, heads=heads)
    for h in heads:
        qm = oracle.block_means(q[0, h], 128)
        km = oracle.block_means(k[0, h], 128)
        ri, rc = oracle.block_topk(qm, km, True, 10)
        np.testing.assert_array_equal(idx[0, h].cpu().numpy(), ri)
        np.testing.assert_array_equal(cnt[0, h].cpu().numpy(), rc)


def test_deterministic(gpu):
    q, k, v = synth.qkv(1, 4, 1024, 128, seed=12)
    qc, kc, vc = q.cuda(), k.cuda(), v.cuda()
    case("attn determinism")
    a, _ = gpu.fp4_attention_fwd(qc, kc, vc, causal=True, fp16_budget_pct=10, out_dtype=gpu.FP32)
    b, _ = gpu.fp4_attention_fwd(qc, kc, vc, causal=True, fp16_budget_pct=10, out_dtype=gpu.FP32)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


@pytest.mark.parametrize("d,kv_tile,causal,pct", [(64, 64, False, 0), (128, 128, True, 0), (128, 128, True, 25),
                                                  (128, 64, False, 0)])
def test_single_level_p(gpu, d, kv_tile, causal, pct):
    """Single-level P (Attn-QAT page, Metodologia / B: no two-level step)
    against the oracle's single-level numerics."""
    q, k, v = synth.qkv(1, 2, 320, d, torch.bfloat16, seed=60 + d, k_outliers=4)
    case(f"single-level P d={d} kv_tile={kv_tile} causal={causal} pct={pct}")
    out, lse = gpu.fp4_attention_fwd(q.cuda(), k.cuda(), v.cuda(), causal=causal, kv_tile=kv_tile,
                                     fp16_budget_pct=pct, out_dtype=gpu.FP32, single_level_p=True)
    torch.cuda.synchronize()
    ref, rlse = oracle.attention_fwd(q, k, v, causal=causal, kv_tile=kv_tile, pct=pct, single_level_p=True)
    assert_close_attn(out.cpu().numpy().reshape(-1, d), ref.reshape(-1, d), "single-level P")
    np.testing.assert_allclose(lse.cpu().numpy().reshape(-1), rlse.reshape(-1), atol=1e-3)
    two, _ = oracle.attention_fwd(q, k, v, causal=causal, kv_tile=kv_tile, pct=pct)
    assert np.abs(two - ref).max() > 1e-3  # the two schemes differ: the test tells them apart


@pytest.mark.parametrize("single", [False, True])
def test_peaked_scores_move_the_reference(gpu, single):
    """Scores that jump by tens of binades between tiles.  Keys 20 and 300 lie
    along a direction u that every query shares, 40 and about 100 binades above
    the rest: rows that see key 300 raise their running reference at its tile,
    and later tiles fall more than 2^64 below it and are left out.  Those rows
    are one-hot in the quantized operands too (key 300 gets e = 1, P^ = 1
    exactly), so the comparison does not hinge on ulp-level rounding near a
    code boundary."""
    q, k, v = synth.qkv(1, 2, 640, 128, seed=131)
    u = torch.ones(128) / 128 ** 0.5
    q = (q.float() + 2.0 * u).to(torch.bfloat16)
    k = k.float()
    k[:, :, 20] = 160.0 * u
    k[:, :, 300] = 400.0 * u
    k = k.to(torch.bfloat16)
    case(f"attn peaked scores S=640 single_level={single}")
    for causal in (True, False):
        out, lse = gpu.fp4_attention_fwd(q.cuda(), k.cuda(), v.cuda(), causal=causal, out_dtype=gpu.FP32,
                                         single_level_p=single)
        torch.cuda.synchronize()
        ref, rlse = oracle.attention_fwd(q, k, v, causal=causal, single_level_p=single)
        assert_close_attn(out.cpu().numpy().reshape(ref.shape), ref, "peaked scores")
        np.testing.assert_allclose(lse.cpu().numpy().reshape(rlse.shape), rlse, atol=1e-3)
