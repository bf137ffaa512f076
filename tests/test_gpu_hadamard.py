"""GPU parity of incoherence processing (ScaleSearch page, Metodologia /
ScaleSearchAttention: Hadamard transforms of Q and K before quantization):
the rotated quantizer bit-exact against the oracle (rotation then
quantization), attention with the rotation within tolerance."""
import numpy as np
import pytest
import torch

import oracle
from block_scaled_fp4_amd import synth
from gpu_helpers import assert_close_attn, case

pytestmark = pytest.mark.gpu

SIGNS = [0x9E3779B9, 0x7F4A7C15, 0x2545F491, 0xD1B54A32]


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16, torch.float32])
@pytest.mark.parametrize("cols", [16, 32, 64, 128])
def test_quantizer_bit_exact(gpu, dtype, cols):
    g = torch.Generator().manual_seed(90 + cols)
    x = torch.randn(333, cols, generator=g)
    x[:, 3] *= 20.0
    x = x.to(dtype)
    case(f"hadamard quantize {dtype} cols={cols}")
    r = gpu.fp4_quantize(x.cuda(), 0, True, hadamard=True, hadamard_signs=SIGNS)
    torch.cuda.synchronize()
    want = oracle.quantize(oracle.hadamard_rows(x, SIGNS), 0, True, -2, 6)
    np.testing.assert_array_equal(r["codes"].cpu().numpy(), want["codes"])
    np.testing.assert_array_equal(r["scales"].cpu().numpy(), want["scales"])
    np.testing.assert_array_equal(r["offsets"].cpu().numpy(), want["offsets"])


def test_quantizer_given_global_scale_and_workload_size(gpu):
    """bf16 [32768, 128] with outlier channels, a caller-given per-tensor scale."""
    x = synth.quant_tensor()
    gval = torch.tensor([0.01], dtype=torch.float32)
    case("hadamard quantize [32768,128] given g")
    r = gpu.fp4_quantize(x.cuda(), 0, True, global_scale=gpu.GLOBAL_GIVEN, g=gval.cuda(), hadamard=True,
                         hadamard_signs=SIGNS)
    torch.cuda.synchronize()
    want = oracle.quantize(oracle.hadamard_rows(x, SIGNS), 0, True, -2, 6, global_mode=2, g=0.01)
    np.testing.assert_array_equal(r["codes"].cpu().numpy(), want["codes"])
    np.testing.assert_array_equal(r["scales"].cpu().numpy(), want["scales"])


@pytest.mark.parametrize("d,causal,pct", [(64, False, 0), (128, True, 0), (128, True, 25)])
def test_attention_with_rotation(gpu, d, causal, pct):
    q, k, v = synth.qkv(1, 2, 384, d, torch.bfloat16, seed=95, k_outliers=4)
    case(f"hadamard attention d={d} causal={causal} pct={pct}")
    out, lse = gpu.fp4_attention_fwd(q.cuda(), k.cuda(), v.cuda(), causal=causal, fp16_budget_pct=pct,
                                     out_dtype=gpu.FP32, hadamard=True, hadamard_signs=SIGNS)
    torch.cuda.synchronize()
    ref, rlse = oracle.attention_fwd(q, k, v, causal=causal, pct=pct, hadamard=True, signs=SIGNS)
    assert_close_attn(out.cpu().numpy().reshape(-1, d), ref.reshape(-1, d), "attention with rotation")
    np.testing.assert_allclose(lse.cpu().numpy().reshape(-1), rlse.reshape(-1), atol=1e-3)
