"""The allocation-free decode entry point (fp4_attention_decode_noalloc,
for callers that cannot allocate) against fp4_attention_decode on the same
inputs, through the C ABI: two calls in a row, the second on a smaller
problem, so the shared device array is reused with stale contents."""
import pytest
import torch

from block_scaled_fp4_amd import synth
from gpu_helpers import build_cache, case

pytestmark = pytest.mark.gpu


def _pair(fp4, B, Hq, Hkv, d, n_sink, n_recent, cap, ctx, seed):
    L = n_sink + cap + n_recent
    q, k, v = synth.decode_context(B, Hq, Hkv, L, d, seed=seed)
    cache = build_cache(fp4, k.cuda(), v.cuda(), ctx, n_sink, n_recent, cap)
    qc = q.cuda()
    ref, rlse = fp4.fp4_attention_decode(qc, cache, out_dtype=fp4.FP32)
    lse = torch.empty((B, Hq), dtype=torch.float32, device="cuda")
    got, _ = fp4.fp4_attention_decode_noalloc(qc, cache, out_dtype=fp4.FP32, lse=lse)
    torch.cuda.synchronize()
    return ref, rlse, got, lse


def test_noalloc_decode_matches_workspace_decode(gpu):
    case("noalloc decode: first call B=3 d=128 context 16+640+32")
    a = _pair(gpu, 3, 8, 2, 128, 16, 32, 640, [16 + 640 + 32, 16 + 32 + 16 * 9, 16 + 32], seed=90)
    case("noalloc decode: second call, smaller (B=2 d=64 context 16+256+32)")
    b = _pair(gpu, 2, 4, 1, 64, 16, 32, 256, [16 + 256 + 32, 16 + 32 + 48], seed=91)
    for ref, rlse, got, lse in (a, b):
        # same kernels and partial layout: identical results
        assert torch.equal(got, ref) and torch.equal(lse, rlse)


def test_noalloc_decode_at_the_decode_workload_shape(gpu):
    """batch 16, 32 q heads / 8 kv heads, context 131072, d 128 (the workspace
    this shape needs fits the fixed array)."""
    B, Hq, Hkv, L, d = 16, 32, 8, 131072, 128
    n_sink, n_recent = 128, 256
    case("noalloc decode: full decode workload")
    q, k, v = synth.decode_context(B, Hq, Hkv, L, d, device="cuda")
    cache = build_cache(gpu, k, v, [L] * B, n_sink, n_recent, L - n_sink - n_recent)
    ref, rlse = gpu.fp4_attention_decode(q, cache, out_dtype=gpu.FP32)
    lse = torch.empty((B, Hq), dtype=torch.float32, device="cuda")
    got, _ = gpu.fp4_attention_decode_noalloc(q, cache, out_dtype=gpu.FP32, lse=lse)
    torch.cuda.synchronize()
    assert torch.equal(got, ref) and torch.equal(lse, rlse)
