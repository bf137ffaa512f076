"""GPU parity of decode with selective promotion (ThriftAttention page,
Metodologia / 1 and / 2, applied to one query token per head; the cache keeps
a full-precision copy of its middle beside the NVFP4 one, Significado): the
selection bit-exact, the output within the attention tolerance, the block
sums and the dual-copy append bit-exact."""
import numpy as np
import pytest
import torch

import oracle
from block_scaled_fp4_amd import synth
from gpu_helpers import assert_close_attn, build_cache, case

pytestmark = pytest.mark.gpu


def _check_selection(sidx, scnt, ridx, rcnt, what):
    np.testing.assert_array_equal(scnt.reshape(-1), rcnt.reshape(-1), err_msg=f"{what}: counts")
    kmax = ridx.shape[-1]
    np.testing.assert_array_equal(sidx.reshape(-1, kmax), ridx.reshape(-1, kmax), err_msg=f"{what}: indices")


@pytest.mark.parametrize("d,Hq,Hkv,pct", [(64, 8, 2, 10), (128, 8, 2, 34), (128, 16, 1, 100), (128, 4, 4, 25)])
def test_selective_small(gpu, d, Hq, Hkv, pct):
    B = 3
    n_sink, n_recent, cap = 16, 32, 5 * 128 + 48  # a short last block at full length
    L = n_sink + cap + n_recent
    q, k, v = synth.decode_context(B, Hq, Hkv, L, d, seed=70 + d + pct)
    ctx = [L, n_sink + n_recent + 16 * 9, n_sink + n_recent]  # full, 144-token middle, empty middle
    case(f"selective decode d={d} Hq={Hq} Hkv={Hkv} pct={pct}")
    cache = build_cache(gpu, k.cuda(), v.cuda(), ctx, n_sink, n_recent, cap, dual=True)
    out, lse, sidx, scnt = gpu.fp4_attention_decode(q.cuda(), cache, out_dtype=gpu.FP32, fp16_budget_pct=pct,
                                                    return_selection=True)
    torch.cuda.synchronize()
    kmax = gpu.decode_sel_kmax(cap, pct)
    ref, rlse, ridx, rcnt = oracle.attention_decode(q, k, v, ctx, n_sink, n_recent, pct=pct, kmax=kmax,
                                                    with_selection=True)
    _check_selection(sidx.cpu().numpy(), scnt.cpu().numpy(), ridx, rcnt, "selection")
    assert_close_attn(out.cpu().numpy().reshape(-1, d), ref.reshape(-1, d), "selective decode")
    np.testing.assert_allclose(lse.cpu().numpy().reshape(-1), rlse.reshape(-1), atol=1e-3)


def test_budget_zero_is_the_plain_decode(gpu):
    B, Hq, Hkv, d = 2, 8, 2, 128
    n_sink, n_recent, cap = 16, 32, 256
    L = n_sink + cap + n_recent
    q, k, v = synth.decode_context(B, Hq, Hkv, L, d, seed=80)
    case("selective decode pct=0 vs plain")
    cache = build_cache(gpu, k.cuda(), v.cuda(), [L, L - 64], n_sink, n_recent, cap, dual=True)
    a, la = gpu.fp4_attention_decode(q.cuda(), cache, out_dtype=gpu.FP32)
    b, lb = gpu.fp4_attention_decode(q.cuda(), cache, out_dtype=gpu.FP32, fp16_budget_pct=0)
    torch.cuda.synchronize()
    assert torch.equal(a, b) and torch.equal(la, lb)


def test_block_sums_bit_exact(gpu):
    B, Hkv, d, cap = 2, 3, 128, 400
    g = torch.Generator().manual_seed(81)
    km = torch.randn(B, Hkv, cap, d, generator=g).to(torch.bfloat16)
    mids = [400, 144]
    cache = gpu.KVCache(torch.zeros((B, Hkv, 0, d), dtype=torch.bfloat16, device="cuda"),
                        torch.zeros((B, Hkv, 0, d), dtype=torch.bfloat16, device="cuda"),
                        torch.zeros((B, Hkv, cap, d // 2), dtype=torch.uint8, device="cuda"),
                        torch.zeros((B, Hkv, cap, d // 16), dtype=torch.uint8, device="cuda"),
                        torch.zeros((B, Hkv, cap // 2, d), dtype=torch.uint8, device="cuda"),
                        torch.zeros((B, Hkv, cap // 16, d), dtype=torch.uint8, device="cuda"),
                        torch.zeros((B, Hkv, 0, d), dtype=torch.bfloat16, device="cuda"),
                        torch.zeros((B, Hkv, 0, d), dtype=torch.bfloat16, device="cuda"),
                        torch.tensor(mids, dtype=torch.int32, device="cuda"), km.cuda(), km.cuda(),
                        torch.full((B, Hkv, 4, d), float("nan"), dtype=torch.float64, device="cuda"))
    case("kv block sums")
    gpu.fp4_kv_block_sums(cache)
    torch.cuda.synchronize()
    got = cache.k_sum.cpu().numpy()
    for b in range(B):
        for h in range(Hkv):
            want = oracle.block_sums(km[b, h, :mids[b]])
            nb = want.shape[0]
            np.testing.assert_array_equal(got[b, h, :nb], want)
            assert (got[b, h, nb:] == 0).all()


def test_append_keeps_the_dual_copy(gpu):
    B, Hkv, d, n_sink, n_recent, cap = 2, 2, 128, 16, 32, 384
    L = n_sink + cap + n_recent
    _, k, v = synth.decode_context(B, 4, Hkv, L, d, seed=82)
    M0 = 112
    cache = build_cache(gpu, k.cuda(), v.cuda(), [n_sink + M0 + n_recent] * B, n_sink, n_recent, cap, dual=True)
    host = [cache.k_recent.float().cpu().numpy(), cache.v_recent.float().cpu().numpy(), cache.k_codes.cpu().numpy(),
            cache.k_scales.cpu().numpy(), cache.v_codes.cpu().numpy(), cache.v_scales.cpu().numpy(),
            cache.mid_len.cpu().numpy()]
    dual = [cache.k_mid.float().cpu().numpy(), cache.v_mid.float().cpu().numpy(), cache.k_sum.cpu().numpy()]
    pos, step = n_sink + M0 + n_recent, 16
    while pos + step <= L:
        kn, vn = k[:, :, pos:pos + step].contiguous(), v[:, :, pos:pos + step].contiguous()
        case(f"dual append at {pos} (+{step})")
        over = gpu.fp4_kv_cache_append(cache, kn.cuda(), vn.cuda())
        out = oracle.kv_append(*host, kn, vn, *dual)
        host, dual = list(out[:7]), list(out[8:])
        assert not over.cpu().numpy().any() and not out[7].any()
        pos += step
        step = 48 if step == 16 else 16
    torch.cuda.synchronize()
    got = [cache.k_recent.float().cpu().numpy(), cache.v_recent.float().cpu().numpy(), cache.k_codes.cpu().numpy(),
           cache.k_scales.cpu().numpy(), cache.v_codes.cpu().numpy(), cache.v_scales.cpu().numpy(),
           cache.mid_len.cpu().numpy()]
    for a, b_, name in zip(got, host, ["k_recent", "v_recent", "k_codes", "k_scales", "v_codes", "v_scales",
                                       "mid_len"]):
        np.testing.assert_array_equal(a, b_, err_msg=name)
    M = int(host[6][0])
    nb = (M + 127) // 128
    np.testing.assert_array_equal(cache.k_mid.float().cpu().numpy()[:, :, :M], dual[0][:, :, :M])
    np.testing.assert_array_equal(cache.v_mid.float().cpu().numpy()[:, :, :M], dual[1][:, :, :M])
    np.testing.assert_array_equal(cache.k_sum.cpu().numpy()[:, :, :nb], dual[2][:, :, :nb])


def test_selective_workload_sampled_pairs(gpu):
    """batch 16, 32 q / 8 kv heads, context 131072, d 128, 128 sink + 256
    recent bf16, budget 10%: selection of every pair bit-exact (oracle block
    sums and scores from the context), outputs of two sampled pairs."""
    B, Hq, Hkv, L, d, pct = 16, 32, 8, 131072, 128, 10
    n_sink, n_recent = 128, 256
    cap = L - n_sink - n_recent
    case("selective decode workload: context on GPU")
    q, k, v = synth.decode_context(B, Hq, Hkv, L, d, device="cuda")
    cache = build_cache(gpu, k, v, [L] * B, n_sink, n_recent, cap, dual=True)
    case("selective decode workload: kernel")
    out, lse, sidx, scnt = gpu.fp4_attention_decode(q, cache, out_dtype=gpu.FP32, fp16_budget_pct=pct,
                                                    return_selection=True)
    torch.cuda.synchronize()
    kmax = gpu.decode_sel_kmax(cap, pct)
    G = Hq // Hkv
    # selection of every (batch, kv head): block means from the oracle's sums of the context
    ks = cache.k_sum.cpu().numpy()
    for b in (0, 7, 15):
        for hk in range(Hkv):
            kb = k[b, hk, n_sink:n_sink + cap].float().cpu().numpy()
            means = oracle.block_means(kb, 128)
            np.testing.assert_array_equal(ks[b, hk], oracle.block_sums(kb, 128))
            qm = q[b, hk * G:(hk + 1) * G].double().cpu().numpy().sum(axis=0) / G
            ridx, rcnt = oracle.block_topk(qm[None], means, False, pct)
            assert int(scnt[b, hk]) == int(rcnt[0]) and ridx.shape[1] == kmax
            np.testing.assert_array_equal(sidx[b, hk].cpu().numpy(), ridx[0])
    for b, hk in ((0, 0), (15, 7)):
        ref, rlse = oracle.attention_decode(q[b:b + 1, hk * G:(hk + 1) * G].cpu(), k[b:b + 1, hk:hk + 1].cpu(),
                                            v[b:b + 1, hk:hk + 1].cpu(), [L], n_sink, n_recent, pct=pct, kmax=kmax)
        assert_close_attn(out[b, hk * G:(hk + 1) * G].cpu().numpy(), ref.reshape(G, d), f"pair b={b} kvh={hk}")
        np.testing.assert_allclose(lse[b, hk * G:(hk + 1) * G].cpu().numpy(), rlse.reshape(G), atol=1e-3)
