"""Strided attention inputs (fp4.h: the strides of fp4_attn_problem).  Q, K and
V laid out as one fused projection [B, S, H + 2 Hkv, d] are read in place: the
quantization, block means, balance exponents, selection and FP16 path see the
same values as with dense copies, so every result equals the dense call's bit
for bit."""
import pytest
import torch

from block_scaled_fp4_amd import synth
from gpu_helpers import case

pytestmark = pytest.mark.gpu


def _fused(q, k, v):
    """q [B,H,S,d], k/v [B,Hkv,S,d] copied into one [B, S, H + 2 Hkv, d] buffer;
    returns the three strided [B, heads, S, d] views of it."""
    B, H, S, d = q.shape
    Hkv = k.shape[1]
    buf = torch.empty((B, S, H + 2 * Hkv, d), dtype=q.dtype, device="cuda")
    buf[:, :, :H] = q.transpose(1, 2).cuda()
    buf[:, :, H:H + Hkv] = k.transpose(1, 2).cuda()
    buf[:, :, H + Hkv:] = v.transpose(1, 2).cuda()
    views = (buf[:, :, :H].transpose(1, 2), buf[:, :, H:H + Hkv].transpose(1, 2),
             buf[:, :, H + Hkv:].transpose(1, 2))
    for t in views:
        assert not t.is_contiguous() and t.stride(-1) == 1
    return views


@pytest.mark.parametrize("B,S,d,H,Hkv,causal,pct,kv_tile,extra", [
    (1, 384, 128, 4, 2, True, 0, 128, {}),
    (2, 640, 128, 4, 4, True, 34, 64, {}),                  # FP16 path, means inside the quantizer
    (2, 512, 64, 2, 1, False, 50, 128, {"balance": True}),  # balance exponents from strided Q and K
    (1, 384, 128, 2, 2, True, 10, 128, {"hadamard": True}),
])
def test_forward_strided_equals_dense(gpu, B, S, d, H, Hkv, causal, pct, kv_tile, extra):
    q, k, v = synth.qkv(B, H, S, d, torch.bfloat16, seed=300 + S, Hkv=Hkv, k_outliers=2)
    qs, ks, vs = _fused(q, k, v)
    case(f"strided forward B={B} S={S} d={d} H={H}/{Hkv} pct={pct} tile={kv_tile} {extra}")
    kw = dict(causal=causal, fp16_budget_pct=pct, kv_tile=kv_tile, out_dtype=gpu.FP32, return_topk=pct > 0, **extra)
    got = gpu.fp4_attention_fwd(qs, ks, vs, **kw)
    ref = gpu.fp4_attention_fwd(q.cuda(), k.cuda(), v.cuda(), **kw)
    torch.cuda.synchronize()
    for a, b in zip(got, ref):
        assert torch.equal(a, b)


def test_given_codes_with_strided_originals(gpu):
    # pre-quantized operands with a budget: the standalone block-means kernel and
    # the FP16 path read the strided originals
    B, S, d, H, Hkv = 1, 768, 128, 2, 1
    q, k, v = synth.qkv(B, H, S, d, torch.bfloat16, seed=41, Hkv=Hkv, k_outliers=2)
    qs, ks, vs = _fused(q, k, v)
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    rq = gpu.fp4_quantize(qd.view(-1, d), 0, True, with_offsets=False)
    rk = gpu.fp4_quantize(kd.view(-1, d), 0, True, with_offsets=False)
    rv = gpu.fp4_quantize(vd.view(-1, d), 1, True, with_offsets=False)
    quant = dict(q_codes=rq["codes"], q_scales=rq["scales"], k_codes=rk["codes"], k_scales=rk["scales"],
                 v_codes=rv["codes"], v_scales=rv["scales"])
    case("strided originals with given codes, pct 20")
    kw = dict(causal=True, fp16_budget_pct=20, kv_tile=128, out_dtype=gpu.FP32, quantized=quant, return_topk=True)
    got = gpu.fp4_attention_fwd(qs, ks, vs, **kw)
    ref = gpu.fp4_attention_fwd(qd, kd, vd, **kw)
    torch.cuda.synchronize()
    for a, b in zip(got, ref):
        assert torch.equal(a, b)
    # the selection alone
    idx_s, cnt_s = gpu.fp4_block_topk(qs, ks, True, 20, 128)
    idx_d, cnt_d = gpu.fp4_block_topk(qd, kd, True, 20, 128)
    torch.cuda.synchronize()
    assert torch.equal(idx_s, idx_d) and torch.equal(cnt_s, cnt_d)
    # the balance exponents alone
    assert torch.equal(gpu.fp4_qk_balance(qs, ks), gpu.fp4_qk_balance(qd, kd))


def test_training_strided_equals_dense(gpu):
    B, S, d, H, Hkv = 1, 320, 128, 4, 2
    q, k, v = synth.qkv(B, H, S, d, torch.bfloat16, seed=77, Hkv=Hkv, k_outliers=2)
    qs, ks, vs = _fused(q, k, v)
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    g = torch.Generator().manual_seed(3)
    do = torch.randn(B, H, S, d, generator=g).to(torch.bfloat16).cuda()
    case("strided training step S=320 H=4/2")
    fs = gpu.fp4_attention_fwd_train(qs, ks, vs, causal=True)
    fd = gpu.fp4_attention_fwd_train(qd, kd, vd, causal=True)
    for a, b in zip(fs, fd):
        assert torch.equal(a, b)
    gs = gpu.fp4_attention_bwd(qs, ks, vs, fs[1], fs[2], do, causal=True)
    gd = gpu.fp4_attention_bwd(qd, kd, vd, fd[1], fd[2], do, causal=True)
    torch.cuda.synchronize()
    for a, b in zip(gs, gd):
        assert torch.equal(a, b)


def test_mx_rejects_strided(gpu):
    q, k, v = synth.qkv(1, 2, 256, 128, torch.bfloat16, seed=5)
    qs, ks, vs = _fused(q, k, v)
    with pytest.raises(gpu.FP4Error, match="dense"):
        gpu.fp4_attention_fwd_mx(qs, ks, vs, causal=True)
