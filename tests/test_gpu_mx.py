"""GPU parity of the MXFP4 variant (E2M1 with one power-of-two scale per 32
elements, the block floating point the ScaleSearch page contrasts NVFP4 with,
Declaracion del Problema): the quantizer bit-exact against the oracle, the
attention forward on the block-scaled FP4 matrix instructions within the
attention tolerance (max-abs 2e-3, relative L2 1e-3 on binary32 outputs)."""
import numpy as np
import pytest
import torch

import oracle
from block_scaled_fp4_amd import synth
from gpu_helpers import assert_close_attn, case

pytestmark = pytest.mark.gpu


def _special_rows(x):
    """Blocks that reach the edges of the scale rule: all zero, tiny (the
    exponent clamp at -127), a value at the top of a binade, one Inf, one NaN."""
    x = x.clone()
    x[0, :32] = 0.0
    x[1, :32] = 1e-39 * torch.arange(32, dtype=torch.float32)
    x[2, 32:64] = 7.99
    x[3, :32] = 3.0 * 2.0 ** -140
    x[4, 5] = float("inf")
    x[5, 40] = float("nan")
    return x


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16, torch.float32])
@pytest.mark.parametrize("axis", [0, 1])
def test_quantizer_bit_exact(gpu, dtype, axis):
    g = torch.Generator().manual_seed(120 + axis)
    rows = 333 if axis == 0 else 352  # ragged against the launch; blocks along rows need rows % 32 == 0
    x = torch.randn(rows, 128, generator=g) * torch.exp(torch.randn(rows, 1, generator=g) * 2)
    x[:, 7] *= 40.0
    if dtype == torch.float32:
        x = _special_rows(x)
    elif dtype == torch.bfloat16:
        x[0, :32] = 0.0
        x[4, 5] = float("inf")
    x = x.to(dtype)
    case(f"mx quantize {dtype} axis={axis} rows={rows}")
    r = gpu.fp4_mx_quantize(x.cuda(), axis)
    torch.cuda.synchronize()
    want = oracle.mx_quantize(x.float(), axis)
    np.testing.assert_array_equal(r["scales"].cpu().numpy(), want["scales"])
    np.testing.assert_array_equal(r["codes"].cpu().numpy(), want["codes"])


def test_quantizer_workload_size(gpu):
    """bf16 [32768, 128] with outlier channels, both block axes."""
    x = synth.quant_tensor()
    for axis in (0, 1):
        case(f"mx quantize [32768,128] axis={axis}")
        r = gpu.fp4_mx_quantize(x.cuda(), axis)
        torch.cuda.synchronize()
        want = oracle.mx_quantize(x.float(), axis)
        np.testing.assert_array_equal(r["scales"].cpu().numpy(), want["scales"])
        np.testing.assert_array_equal(r["codes"].cpu().numpy(), want["codes"])


def test_quantizer_empty(gpu):
    x = torch.zeros(0, 64, dtype=torch.bfloat16, device="cuda")
    r = gpu.fp4_mx_quantize(x, 0)
    torch.cuda.synchronize()
    assert r["codes"].numel() == 0 and r["scales"].numel() == 0


def _check(gpu, q, k, v, causal, kv_tile, rows=None, heads=None, softmax_scale=0.0):
    B, H, Sq, d = q.shape
    out, lse = gpu.fp4_attention_fwd_mx(q.cuda(), k.cuda(), v.cuda(), causal=causal, kv_tile=kv_tile,
                                        softmax_scale=softmax_scale, out_dtype=gpu.FP32)
    torch.cuda.synchronize()
    ref, rlse = oracle.attention_fwd(q, k, v, causal=causal, kv_tile=kv_tile, rows=rows, heads=heads, mx=True,
                                     softmax_scale=float(np.float32(softmax_scale)))
    got = out.cpu().numpy().reshape(B * H, Sq, d)
    gl = lse.cpu().numpy().reshape(B * H, Sq)
    if heads is not None:
        got, gl = got[heads], gl[heads]
    if rows is not None:
        got, gl = got[:, rows], gl[:, rows]
    assert_close_attn(got, ref, "mx attention")
    np.testing.assert_allclose(gl, rlse, atol=1e-3)
    return out


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("kv_tile", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_attention_ragged_tiles(gpu, d, kv_tile, causal):
    # 416 = 3*128 + 32: several key tiles, a ragged last key tile and query tile
    q, k, v = synth.qkv(1, 2, 416, d, seed=125, k_outliers=4)
    case(f"mx attention S=416 d={d} kv_tile={kv_tile} causal={causal}")
    _check(gpu, q, k, v, causal, kv_tile)


def test_attention_gqa_cross_lengths_fp16(gpu):
    q, k, v = synth.qkv(2, 4, 200, 128, dtype=torch.float16, Hkv=2, Sk=352, seed=126)
    case("mx attention gqa Sq=200 Sk=352 fp16 softmax_scale=0.2")
    _check(gpu, q, k, v, False, 128, softmax_scale=0.2)


def test_attention_peaked_rows(gpu):
    """Large scores (one dominant key per row) move the integer reference far
    between tiles: rescales and skipped tiles both occur."""
    q, k, v = synth.qkv(1, 2, 512, 128, seed=127)
    k = k.float()
    k[:, :, 300] *= 30.0
    k[:, :, 5] *= 12.0
    k = k.to(torch.bfloat16)
    case("mx attention peaked scores S=512")
    _check(gpu, q, k, v, True, 64)
    _check(gpu, q, k, v, False, 128)


def test_prequantized_operands_match(gpu):
    q, k, v = synth.qkv(1, 4, 384, 128, seed=128, Hkv=2)
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    B, H, S, d = q.shape
    qq = gpu.fp4_mx_quantize(qd.reshape(-1, d), 0)
    kq = gpu.fp4_mx_quantize(kd.reshape(-1, d), 0)
    vq = gpu.fp4_mx_quantize(vd.reshape(-1, d), 1)
    quant = dict(q_codes=qq["codes"], q_scales=qq["scales"], k_codes=kq["codes"], k_scales=kq["scales"],
                 v_codes=vq["codes"], v_scales=vq["scales"], q_shape=(B, H, S, d), kv_shape=(2, S))
    case("mx attention pre-quantized operands")
    a, la = gpu.fp4_attention_fwd_mx(None, None, None, causal=True, out_dtype=gpu.FP32, quantized=quant)
    b, lb = gpu.fp4_attention_fwd_mx(qd, kd, vd, causal=True, out_dtype=gpu.FP32)
    torch.cuda.synchronize()
    assert torch.equal(a, b) and torch.equal(la, lb)


@pytest.mark.parametrize("out_dtype", ["bf16", "fp16"])
def test_output_dtypes(gpu, out_dtype):
    q, k, v = synth.qkv(1, 2, 256, 64, seed=129)
    dt = gpu.BF16 if out_dtype == "bf16" else gpu.FP16
    case(f"mx attention out {out_dtype}")
    o32, _ = gpu.fp4_attention_fwd_mx(q.cuda(), k.cuda(), v.cuda(), causal=True, out_dtype=gpu.FP32)
    o, _ = gpu.fp4_attention_fwd_mx(q.cuda(), k.cuda(), v.cuda(), causal=True, out_dtype=dt)
    torch.cuda.synchronize()
    want = o32.to(torch.bfloat16 if out_dtype == "bf16" else torch.float16)
    assert torch.equal(o, want)


def test_prefill_workload_sampled_rows(gpu):
    """B=1, H=32, S=8192, d=128, causal, kv_tile 128 -- the prefill workload in MXFP4."""
    q, k, v = synth.prefill(S=8192)
    rows = sorted(set([0, 1, 127, 128, 4095, 8191] + list(range(37, 8192, 611))))
    heads = [0, 17, 31]
    case("mx attention prefill 8K causal, sampled rows")
    _check(gpu, q, k, v, True, 128, rows=rows, heads=heads)


def test_deterministic(gpu):
    q, k, v = synth.qkv(1, 4, 1024, 128, seed=130)
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    a, _ = gpu.fp4_attention_fwd_mx(qd, kd, vd, causal=True)
    b, _ = gpu.fp4_attention_fwd_mx(qd, kd, vd, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(a, b)
