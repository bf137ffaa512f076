"""Calls captured in a HIP graph (torch.cuda.graph) and replayed: the cache
append, the decode, the allocation-free decode and the attention forward
(quantization, selection and FP16 path included).  Each graph is replayed
several times, with new inputs copied in and eager calls between the replays,
and every replay is compared bit for bit with the same call run eagerly on
identical inputs (the library issues no memset and no host synchronization,
so its launches are capturable; bench.py times the launch-bound legs this
way)."""
import pytest
import torch

from block_scaled_fp4_amd import synth
from gpu_helpers import build_cache, case

pytestmark = pytest.mark.gpu


def _clone_cache(fp4, c):
    t = [None if x is None else x.clone() for x in (c.k_sink, c.v_sink, c.k_codes, c.k_scales, c.v_codes,
                                                      c.v_scales, c.k_recent, c.v_recent, c.mid_len)]
    return fp4.KVCache(*t)


def _cache_tensors(c):
    return [c.k_codes, c.k_scales, c.v_codes, c.v_scales, c.k_recent, c.v_recent, c.mid_len]


def test_cache_append_replayed_from_a_graph(gpu):
    B, H, d, n_sink, n_recent, cap, n_new = 3, 2, 128, 16, 64, 256, 16
    g = torch.Generator(device="cuda").manual_seed(70)
    rnd = lambda *s: torch.randn(*s, generator=g, device="cuda").to(torch.bfloat16)  # noqa: E731
    base = gpu.KVCache(rnd(B, H, n_sink, d), rnd(B, H, n_sink, d),
                       torch.zeros((B, H, cap, d // 2), dtype=torch.uint8, device="cuda"),
                       torch.zeros((B, H, cap, d // 16), dtype=torch.uint8, device="cuda"),
                       torch.zeros((B, H, cap // 2, d), dtype=torch.uint8, device="cuda"),
                       torch.zeros((B, H, cap // 16, d), dtype=torch.uint8, device="cuda"),
                       rnd(B, H, n_recent, d), rnd(B, H, n_recent, d),
                       torch.tensor([0, 32, 64], dtype=torch.int32, device="cuda"))
    eager, graphed = _clone_cache(gpu, base), _clone_cache(gpu, base)
    kn, vn = rnd(B, H, n_new, d), rnd(B, H, n_new, d)  # the graph's input buffers
    ws = torch.empty(1 << 22, dtype=torch.uint8, device="cuda")
    case("graph: cache append capture")
    gpu.fp4_kv_cache_append(_clone_cache(gpu, base), kn, vn, workspace=ws)  # warm-up on a scratch copy
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        gpu.fp4_kv_cache_append(graphed, kn, vn, workspace=ws)
    for r in range(4):
        case(f"graph: cache append replay {r}")
        kn.copy_(rnd(B, H, n_new, d))
        vn.copy_(rnd(B, H, n_new, d))
        graph.replay()
        gpu.fp4_kv_cache_append(eager, kn, vn, workspace=ws)
        torch.cuda.synchronize()
        for a, b in zip(_cache_tensors(graphed), _cache_tensors(eager)):
            assert torch.equal(a, b), f"replay {r}"
    assert eager.mid_len.tolist() == [4 * n_new, 32 + 4 * n_new, 64 + 4 * n_new]


@pytest.mark.parametrize("noalloc", [False, True])
def test_decode_replayed_from_a_graph(gpu, noalloc):
    B, Hq, Hkv, d, n_sink, n_recent, cap = 2, 8, 2, 128, 16, 32, 512
    L = n_sink + cap + n_recent
    q, k, v = synth.decode_context(B, Hq, Hkv, L, d, seed=71)
    cache = build_cache(gpu, k.cuda(), v.cuda(), [L, n_sink + n_recent + 16 * 11], n_sink, n_recent, cap)
    qs = q.cuda().clone()  # the graph's input buffer
    out = torch.empty((B, Hq, d), dtype=torch.float32, device="cuda")
    lse = torch.empty((B, Hq), dtype=torch.float32, device="cuda")
    ws = torch.empty(1 << 24, dtype=torch.uint8, device="cuda")

    def call():
        if noalloc:
            gpu.fp4_attention_decode_noalloc(qs, cache, out_dtype=gpu.FP32, out=out, lse=lse)
        else:
            o, l_ = gpu.fp4_attention_decode(qs, cache, out_dtype=gpu.FP32, workspace=ws, out=out)
            lse.copy_(l_)

    case(f"graph: decode capture (noalloc={noalloc})")
    call()  # warm-up
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call()
    gen = torch.Generator(device="cuda").manual_seed(72)
    for r in range(4):
        case(f"graph: decode replay {r} (noalloc={noalloc})")
        qs.copy_(torch.randn(B, Hq, d, generator=gen, device="cuda").to(torch.bfloat16))
        graph.replay()
        torch.cuda.synchronize()
        got, got_lse = out.clone(), lse.clone()
        ref, rlse = gpu.fp4_attention_decode(qs, cache, out_dtype=gpu.FP32)
        torch.cuda.synchronize()
        assert torch.equal(got, ref) and torch.equal(got_lse, rlse), f"replay {r}"


@pytest.mark.parametrize("S,d,causal,pct,search", [(256, 64, False, 0, False), (512, 128, True, 10, True)])
def test_attention_forward_replayed_from_a_graph(gpu, S, d, causal, pct, search):
    """The tiny configuration (fp16, one quantizer launch and the attention
    kernel) and a causal case whose graph holds the quantization with block
    means, the selection and the FP16 path."""
    dt = torch.float16 if S == 256 else torch.bfloat16
    H = 2
    qs, ks, vs = (t.cuda() for t in synth.qkv(1, H, S, d, dt, seed=73))  # the graph's input buffers
    out = torch.empty((1, H, S, d), dtype=torch.float32, device="cuda")
    kw = dict(causal=causal, kv_tile=64 if d == 64 else 128, scale_search=search, fp16_budget_pct=pct,
              out_dtype=gpu.FP32)

    def call():
        gpu.fp4_attention_fwd(qs, ks, vs, return_lse=False, out=out, **kw)

    case(f"graph: forward capture S={S} pct={pct}")
    call()  # warm-up
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call()
    for r in range(3):
        case(f"graph: forward replay {r} S={S} pct={pct}")
        nq, nk, nv = synth.qkv(1, H, S, d, dt, seed=74 + r)
        qs.copy_(nq.cuda())
        ks.copy_(nk.cuda())
        vs.copy_(nv.cuda())
        graph.replay()
        torch.cuda.synchronize()
        got = out.clone()
        ref, _ = gpu.fp4_attention_fwd(qs, ks, vs, **kw)
        torch.cuda.synchronize()
        assert torch.equal(got, ref), f"replay {r}"
