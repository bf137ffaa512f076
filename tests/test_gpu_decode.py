"""GPU decode parity over the sink-aware mixed-precision KV cache (ScaleSearch
page, Metodologia / ScaleSearchAttention): bf16 sink and recent tokens, NVFP4
middle (ScaleSearch, K blocks along d, V blocks of 16 tokens)."""
import numpy as np
import pytest
import torch

import oracle
from block_scaled_fp4_amd import synth
from gpu_helpers import assert_close_attn, build_cache, case

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("d", [64, 128])
def test_small_cache(gpu, d):
    B, Hq, Hkv = 3, 8, 2
    n_sink, n_recent, cap = 16, 32, 400
    L = n_sink + cap + n_recent
    q, k, v = synth.decode_context(B, Hq, Hkv, L, d)
    ctx = [L, n_sink + n_recent + 16 * 7, n_sink + n_recent]   # full, partial, empty middle
    case(f"decode small d={d}")
    cache = build_cache(gpu, k.cuda(), v.cuda(), ctx, n_sink, n_recent, cap)
    out, lse = gpu.fp4_attention_decode(q.cuda(), cache, out_dtype=gpu.FP32)
    torch.cuda.synchronize()
    ref, rlse = oracle.attention_decode(q, k, v, ctx, n_sink, n_recent)
    assert_close_attn(out.cpu().numpy().reshape(-1, d), ref.reshape(-1, d), "decode small")
    np.testing.assert_allclose(lse.cpu().numpy().reshape(-1), rlse.reshape(-1), atol=1e-3)


def test_gqa_group_of_one_and_sixteen(gpu):
    for Hq, Hkv in ((4, 4), (16, 1)):
        n_sink, n_recent, cap = 32, 64, 256
        L = n_sink + cap + n_recent
        q, k, v = synth.decode_context(2, Hq, Hkv, L, 128, seed=20)
        ctx = [L, L - 128]
        case(f"decode Hq={Hq} Hkv={Hkv}")
        cache = build_cache(gpu, k.cuda(), v.cuda(), ctx, n_sink, n_recent, cap)
        out, _ = gpu.fp4_attention_decode(q.cuda(), cache, out_dtype=gpu.FP32)
        torch.cuda.synchronize()
        ref, _ = oracle.attention_decode(q, k, v, ctx, n_sink, n_recent)
        assert_close_attn(out.cpu().numpy().reshape(-1, 128), ref.reshape(-1, 128), f"decode G={Hq // Hkv}")


def test_decode_workload_two_batches(gpu):
    """batch 16, 32 q heads / 8 kv heads, context 131072, d 128, sink 128 +
    recent 256 bf16: every kv head (all 32 query heads) of batches 0 and 15."""
    B, Hq, Hkv, L, d = 16, 32, 8, 131072, 128
    n_sink, n_recent = 128, 256
    cap = L - n_sink - n_recent
    case("decode full workload: generating context on GPU")
    q, k, v = synth.decode_context(B, Hq, Hkv, L, d, device="cuda")
    ctx = [L] * B
    cache = build_cache(gpu, k, v, ctx, n_sink, n_recent, cap)
    case("decode full workload: kernel")
    out, lse = gpu.fp4_attention_decode(q, cache, out_dtype=gpu.FP32)
    torch.cuda.synchronize()
    for b in (0, 15):
        case(f"decode full workload: oracle for batch {b}")
        ref, rlse = oracle.attention_decode(q[b:b + 1].cpu(), k[b:b + 1].cpu(), v[b:b + 1].cpu(), [L], n_sink,
                                            n_recent)
        got = out[b].cpu().numpy()
        assert_close_attn(got, ref.reshape(Hq, d), f"decode batch {b}")
        np.testing.assert_allclose(lse[b].cpu().numpy(), rlse.reshape(Hq), atol=1e-3)
