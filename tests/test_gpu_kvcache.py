"""GPU parity of the quantize-on-write cache append (ScaleSearch page,
Metodologia / ScaleSearchAttention): codes, scales, window, mid_len and the
overflow flags bit-exact against the oracle; decode over an appended cache
against the decode oracle over the whole context."""
import numpy as np
import pytest
import torch

import oracle
from block_scaled_fp4_amd import synth
from gpu_helpers import assert_close_attn, case

pytestmark = pytest.mark.gpu


def _cache(fp4, B, H, d, n_sink, n_recent, cap, seed, mid):
    g = torch.Generator().manual_seed(seed)
    k_sink = torch.randn(B, H, n_sink, d, generator=g).to(torch.bfloat16)
    v_sink = torch.randn(B, H, n_sink, d, generator=g).to(torch.bfloat16)
    kr = torch.randn(B, H, n_recent, d, generator=g).to(torch.bfloat16)
    vr = torch.randn(B, H, n_recent, d, generator=g).to(torch.bfloat16)
    kc = torch.randint(0, 256, (B, H, cap, d // 2), generator=g, dtype=torch.uint8)
    ks = torch.randint(0, 127, (B, H, cap, d // 16), generator=g, dtype=torch.uint8)
    vc = torch.randint(0, 256, (B, H, cap // 2, d), generator=g, dtype=torch.uint8)
    vs = torch.randint(0, 127, (B, H, cap // 16, d), generator=g, dtype=torch.uint8)
    ml = torch.tensor(mid, dtype=torch.int32)
    host = dict(kr=kr, vr=vr, kc=kc, ks=ks, vc=vc, vs=vs, ml=ml)
    dev = fp4.KVCache(k_sink.cuda(), v_sink.cuda(), kc.cuda(), ks.cuda(), vc.cuda(), vs.cuda(), kr.cuda(),
                      vr.cuda(), ml.cuda())
    return host, dev


@pytest.mark.parametrize("d,n_recent,n_new", [(64, 48, 16), (128, 32, 32), (128, 0, 16), (128, 16, 48),
                                              (128, 480, 16), (64, 496, 16), (128, 256, 256)])
def test_append_bit_exact(gpu, d, n_recent, n_new):
    # windows plus new tokens up to 496 take the one-pass kernel (the sequence of
    # one operand and 64 channels in LDS); (64, 496, 16) and (128, 256, 256) the
    # two-launch path
    B, H = 3, 2
    cap = max(96, 2 * n_new + 32)
    # room, exactly full after, no room (rounded down to a multiple of 16: cap - 6 -> cap - 16)
    mid = [16, cap - n_new, cap - 6] if n_new >= 32 else [16, cap - n_new, 90]
    host, dev = _cache(gpu, B, H, d, 16, n_recent, cap, seed=30 + d + n_recent, mid=mid)
    g = torch.Generator().manual_seed(7)
    kn = torch.randn(B, H, n_new, d, generator=g).to(torch.bfloat16)
    vn = torch.randn(B, H, n_new, d, generator=g).to(torch.bfloat16)
    case(f"kv append d={d} n_recent={n_recent} n_new={n_new}")
    over = gpu.fp4_kv_cache_append(dev, kn.cuda(), vn.cuda())
    torch.cuda.synchronize()
    want = oracle.kv_append(host["kr"], host["vr"], host["kc"].numpy(), host["ks"].numpy(), host["vc"].numpy(),
                            host["vs"].numpy(), host["ml"].numpy(), kn, vn)
    got = [dev.k_recent.float().cpu().numpy(), dev.v_recent.float().cpu().numpy(), dev.k_codes.cpu().numpy(),
           dev.k_scales.cpu().numpy(), dev.v_codes.cpu().numpy(), dev.v_scales.cpu().numpy(),
           dev.mid_len.cpu().numpy(), over.cpu().numpy()]
    for a, b, name in zip(got, want, ["k_recent", "v_recent", "k_codes", "k_scales", "v_codes", "v_scales",
                                      "mid_len", "overflow"]):
        np.testing.assert_array_equal(a, b, err_msg=name)


def test_decode_after_appends_matches_decode_oracle(gpu):
    """Fill a cache by appends from a context, then decode: equals the decode
    oracle run on the whole context (which builds its cache directly)."""
    B, Hq, Hkv, d = 2, 8, 2, 128
    n_sink, n_recent, cap = 16, 32, 128
    L = n_sink + cap + n_recent
    q, k, v = synth.decode_context(B, Hq, Hkv, L, d, seed=40)
    kd, vd = k.cuda(), v.cuda()
    kc = torch.zeros((B, Hkv, cap, d // 2), dtype=torch.uint8, device="cuda")
    ks = torch.zeros((B, Hkv, cap, d // 16), dtype=torch.uint8, device="cuda")
    vc = torch.zeros((B, Hkv, cap // 2, d), dtype=torch.uint8, device="cuda")
    vs = torch.zeros((B, Hkv, cap // 16, d), dtype=torch.uint8, device="cuda")
    cache = gpu.KVCache(kd[:, :, :n_sink].contiguous(), vd[:, :, :n_sink].contiguous(), kc, ks, vc, vs,
                        kd[:, :, n_sink:n_sink + n_recent].contiguous(), vd[:, :, n_sink:n_sink + n_recent].contiguous(),
                        torch.zeros(B, dtype=torch.int32, device="cuda"))
    pos = n_sink + n_recent
    case("kv append: fill by appends of 16 and 32 tokens")
    step = 16
    while pos < L:
        over = gpu.fp4_kv_cache_append(cache, kd[:, :, pos:pos + step].contiguous(),
                                       vd[:, :, pos:pos + step].contiguous())
        assert int(over.sum().item()) == 0
        pos += step
        step = 32 if step == 16 else 16
    torch.cuda.synchronize()
    assert cache.mid_len.cpu().tolist() == [cap] * B
    case("kv append: decode over the appended cache")
    out, lse = gpu.fp4_attention_decode(q.cuda(), cache, out_dtype=gpu.FP32)
    torch.cuda.synchronize()
    ref, rlse = oracle.attention_decode(q, k, v, [L] * B, n_sink, n_recent)
    assert_close_attn(out.cpu().numpy().reshape(-1, d), ref.reshape(-1, d), "decode after appends")
    np.testing.assert_allclose(lse.cpu().numpy().reshape(-1), rlse.reshape(-1), atol=1e-3)


def test_append_decode_workload_shape(gpu):
    """Batch 16, 8 kv heads, d 128, 256 recent tokens, a 130,688-token NVFP4
    region one group short of full: the group written and the window are
    bit-exact (checked on the touched region: the quantization does not
    depend on the position)."""
    B, Hkv, d, n_recent, cap = 16, 8, 128, 256, 130688
    g = torch.Generator(device="cuda").manual_seed(50)
    kr = torch.randn(B, Hkv, n_recent, d, generator=g, device="cuda").to(torch.bfloat16)
    vr = torch.randn(B, Hkv, n_recent, d, generator=g, device="cuda").to(torch.bfloat16)
    kn = torch.randn(B, Hkv, 16, d, generator=g, device="cuda").to(torch.bfloat16)
    vn = torch.randn(B, Hkv, 16, d, generator=g, device="cuda").to(torch.bfloat16)
    kc = torch.zeros((B, Hkv, cap, d // 2), dtype=torch.uint8, device="cuda")
    ks = torch.zeros((B, Hkv, cap, d // 16), dtype=torch.uint8, device="cuda")
    vc = torch.zeros((B, Hkv, cap // 2, d), dtype=torch.uint8, device="cuda")
    vs = torch.zeros((B, Hkv, cap // 16, d), dtype=torch.uint8, device="cuda")
    m = cap - 16
    sink = torch.zeros((B, Hkv, 16, d), dtype=torch.bfloat16, device="cuda")
    cache = gpu.KVCache(sink, sink, kc, ks, vc, vs, kr.clone(), vr.clone(),
                        torch.full((B,), m, dtype=torch.int32, device="cuda"))
    case("kv append workload shape")
    over = gpu.fp4_kv_cache_append(cache, kn, vn)
    torch.cuda.synchronize()
    assert over.cpu().tolist() == [0] * B and cache.mid_len.cpu().tolist() == [cap] * B
    # oracle on a 16-token region (position-independent quantization)
    z = np.zeros
    want = oracle.kv_append(kr.cpu(), vr.cpu(), z((B, Hkv, 16, d // 2), np.uint8), z((B, Hkv, 16, d // 16), np.uint8),
                            z((B, Hkv, 8, d), np.uint8), z((B, Hkv, 1, d), np.uint8), np.zeros(B, np.int32),
                            kn.cpu(), vn.cpu())
    np.testing.assert_array_equal(cache.k_recent.float().cpu().numpy(), want[0])
    np.testing.assert_array_equal(cache.v_recent.float().cpu().numpy(), want[1])
    np.testing.assert_array_equal(kc[:, :, m:].cpu().numpy(), want[2])
    np.testing.assert_array_equal(ks[:, :, m:].cpu().numpy(), want[3])
    np.testing.assert_array_equal(vc[:, :, m // 2:].cpu().numpy(), want[4])
    np.testing.assert_array_equal(vs[:, :, m // 16:].cpu().numpy(), want[5])
    # nothing before the group was touched
    assert int(kc[:, :, :m].count_nonzero().item()) == 0 and int(vs[:, :, :m // 16].count_nonzero().item()) == 0
