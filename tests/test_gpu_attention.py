"""GPU attention-forward parity against the oracle's fake-quant numerics
(ScaleSearch page, Metodologia / ScaleSearchAttention; ThriftAttention page,
Metodologia / 2).  Outputs in binary32, max-abs 2e-3 and relative L2 1e-3."""
import math

import numpy as np
import pytest
import torch

import oracle
from block_scaled_fp4_amd import synth
from gpu_helpers import TIE_SLACK, assert_close_attn, assert_close_attn_rows, case
import mix_closed_form as mcf

pytestmark = pytest.mark.gpu


def _gpu(fp4, q, k, v, **kw):
    out, lse, idx, cnt = fp4.fp4_attention_fwd(q.cuda(), k.cuda(), v.cuda(), out_dtype=fp4.FP32, return_topk=True,
                                               **kw)
    torch.cuda.synchronize()
    return out.cpu().numpy(), lse.cpu().numpy(), idx, cnt


def _check(fp4, q, k, v, causal, kv_tile, search, pct=0, rows=None, heads=None, softmax_scale=0.0, sel_block=128):
    B, H, Sq, d = q.shape
    out, lse, idx, cnt = _gpu(fp4, q, k, v, causal=causal, kv_tile=kv_tile, scale_search=search,
                              fp16_budget_pct=pct, softmax_scale=softmax_scale, sel_block=sel_block)
    ref, rlse, amb = oracle.attention_fwd(q, k, v, causal=causal, kv_tile=kv_tile, scale_search=search, pct=pct,
                                          sel_block=sel_block, rows=rows, heads=heads,
                                          softmax_scale=float(np.float32(softmax_scale)), tie_slack=TIE_SLACK)
    got = out.reshape(B * H, Sq, d)
    gl = lse.reshape(B * H, Sq)
    if heads is not None:
        got, gl = got[heads], gl[heads]
    if rows is not None:
        got, gl = got[:, rows], gl[:, rows]
    assert_close_attn_rows(got, ref, amb)
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
@pytest.mark.parametrize("sel_block", [128, 256])
@pytest.mark.parametrize("kv_tile", [64, 128])
@pytest.mark.parametrize("d", [64, 128])
def test_selective_fp16_path(gpu, d, kv_tile, sel_block, pct):
    """Random inputs with the FP16 path on: head dims 64 and 128, key tiles of
    64 (two tiles per 128-token selection block) and 128, selection blocks of
    128 and 256 tokens (two query tiles of the kernel share a selection row)."""
    q, k, v = synth.qkv(1, 2, 1024 + 64, d, seed=8 + d, k_outliers=4)
    case(f"attn selective d={d} kv_tile={kv_tile} sel_block={sel_block} pct={pct} S=1088 causal")
    out, idx, cnt = _check(gpu, q, k, v, causal=True, kv_tile=kv_tile, search=True, pct=pct, sel_block=sel_block)
    _, _, ridx, rcnt = oracle.attention_fwd(q, k, v, causal=True, kv_tile=kv_tile, pct=pct, sel_block=sel_block,
                                            rows=[0], with_topk=True)
    np.testing.assert_array_equal(idx.cpu().numpy().reshape(ridx.shape), ridx)
    np.testing.assert_array_equal(cnt.cpu().numpy().reshape(rcnt.shape), rcnt)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("sel_block,pct", [(128, 10), (128, 34), (256, 50)])
@pytest.mark.parametrize("kv_tile", [64, 128])
@pytest.mark.parametrize("d", [64, 128])
def test_partial_budget_mix_closed_form(gpu, d, kv_tile, sel_block, pct, causal):
    """The FP4/FP16 mix against its closed form (tests/mix_closed_form.py):
    scores constant inside every key tile make P quantization lossless, so the
    output is softmax attention over fp16(V) on the selected blocks' keys and
    the dequantized V elsewhere.  A wrong tile -> block map, a shifted block or
    FP4 weights in other units move it by 3e-2 or more in relative L2."""
    H, S = 2, 960  # 7.5 selection blocks of 128
    q, k, v, a = mcf.construct(H, S, d, kv_tile, seed=pct + kv_tile + d)
    assert mcf.operands_exact(q, k)
    scale = 0.25 / d
    case(f"attn mix closed form d={d} kv_tile={kv_tile} sel_block={sel_block} pct={pct} causal={causal}")
    out, lse, idx, cnt = _gpu(gpu, q, k, v, causal=causal, kv_tile=kv_tile, fp16_budget_pct=pct,
                              sel_block=sel_block, softmax_scale=scale)
    want, wlse = mcf.expected(q, k, v, a, causal, pct, sel_block, scale, kv_tile)
    assert_close_attn(out.reshape(H, S, d), want, "mix vs closed form")
    np.testing.assert_allclose(lse.reshape(H, S), wlse, atol=1e-4)
    ref, _ = oracle.attention_fwd(q, k, v, causal=causal, softmax_scale=scale, kv_tile=kv_tile, pct=pct,
                                  sel_block=sel_block)
    assert_close_attn(out.reshape(H, S, d), ref, "mix vs oracle")
    idx, cnt = idx.cpu().numpy().reshape(H, -1, idx.shape[-1]), cnt.cpu().numpy().reshape(H, -1)
    for h in range(H):
        for i, s in enumerate(mcf.selection(a[h], S, causal, pct, sel_block)):
            assert cnt[h, i] == len(s) and list(idx[h, i, : cnt[h, i]]) == s


@pytest.mark.parametrize("kv_tile", [64, 128])
def test_partial_budget_zero_keys(gpu, kv_tile):
    """K = 0 at a partial budget: ties promote the lowest visible blocks, and
    every row is the mean of fp16(V) over their keys and of V^ elsewhere."""
    H, S, d, pct = 1, 640, 128, 34
    q, k, v, a = mcf.construct(H, S, d, kv_tile, seed=3, zero_keys=True)
    case(f"attn mix zero keys kv_tile={kv_tile}")
    for causal in (False, True):
        out, lse, _, _ = _gpu(gpu, q, k, v, causal=causal, kv_tile=kv_tile, fp16_budget_pct=pct)
        want, wlse = mcf.expected(q, k, v, a, causal, pct, 128, 1.0 / math.sqrt(d), kv_tile)
        assert_close_attn(out.reshape(H, S, d), want, "mix zero keys")
        np.testing.assert_allclose(lse.reshape(H, S), wlse, atol=1e-4)


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


@pytest.mark.parametrize("B,H,Hkv,S,d,dt", [
    (2, 4, 2, 384, 64, torch.float16),
    (1, 8, 2, 8192, 128, torch.bfloat16),  # Q alone fills the 2048 workgroups of its range
])
def test_one_launch_quantization_equals_separate(gpu, B, H, Hkv, S, d, dt):
    # without rotation, balance or selection the forward quantizes Q, K and V in
    # one launch; its codes must be those of three standalone quantizer calls
    q, k, v = synth.qkv(B, H, S, d, dt, seed=90 + d, Hkv=Hkv, k_outliers=2)
    qc, kc, vc = q.cuda(), k.cuda(), v.cuda()
    case(f"attn one-launch quantization B={B} H={H}/{Hkv} S={S} d={d} {dt}")
    rq = gpu.fp4_quantize(qc.view(-1, d), 0, True, with_offsets=False)
    rk = gpu.fp4_quantize(kc.view(-1, d), 0, True, with_offsets=False)
    rv = gpu.fp4_quantize(vc.view(-1, d), 1, True, with_offsets=False)
    quant = dict(q_codes=rq["codes"], q_scales=rq["scales"], k_codes=rk["codes"], k_scales=rk["scales"],
                 v_codes=rv["codes"], v_scales=rv["scales"])
    kw = dict(causal=True, kv_tile=128, out_dtype=gpu.FP32)
    o1, l1 = gpu.fp4_attention_fwd(qc, kc, vc, quantized=quant, **kw)
    o2, l2 = gpu.fp4_attention_fwd(qc, kc, vc, **kw)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_prefill_workload_all_heads(gpu):
    """B=1, H=32, S=8192, d=128, causal, ScaleSearch Q/K/V, two-level P,
    kv_tile 128: every row of every head against the oracle."""
    q, k, v = synth.prefill(S=8192)
    case("attn prefill 8K causal full size, all rows of all 32 heads")
    _check(gpu, q, k, v, causal=True, kv_tile=128, search=True)


def test_selective_workload_two_heads(gpu):
    """B=1, H=32, S=32768, causal, top 10% 128x128 block pairs on the FP16
    path: all 32768 rows of heads 0 and 31 (workgroups of different XCDs)
    against the oracle, and the selection of every head bit-exact."""
    q, k, v = synth.prefill(S=32768)
    heads = [0, 31]
    case("attn selective 32K causal full size, all rows of heads 0 and 31")
    out, idx, cnt = _check(gpu, q, k, v, causal=True, kv_tile=128, search=True, pct=10, heads=heads)
    for h in range(32):
        qm = oracle.block_means(q[0, h], 128)
        km = oracle.block_means(k[0, h], 128)
        ri, rc = oracle.block_topk(qm, km, True, 10)
        np.testing.assert_array_equal(idx[0, h].cpu().numpy(), ri)
        np.testing.assert_array_equal(cnt[0, h].cpu().numpy(), rc)
    assert int(cnt[0].sum().item()) == 32 * 3406


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


def test_given_selection_contract(gpu):
    """A caller's selection list that repeats, disorders or pads entries, or
    whose count runs past kmax, promotes exactly the entries that exceed every
    entry before them (include/fp4.h): the output is bit-identical to the one
    for that clean ascending list, and no key is counted twice."""
    B, H, S, d, pct = 1, 2, 1024, 128, 50
    q, k, v = synth.qkv(B, H, S, d, seed=140, k_outliers=4)
    qc, kc, vc = q.cuda(), k.cuda(), v.cuda()
    nqb = nkb = S // 128
    kmax = (pct * nkb + 99) // 100
    rng = np.random.default_rng(140)
    messy = np.full((B, H, nqb, kmax), -1, np.int32)
    clean = np.full((B, H, nqb, kmax), -1, np.int32)
    mcnt = np.zeros((B, H, nqb), np.int32)
    ccnt = np.zeros((B, H, nqb), np.int32)
    for h in range(H):
        for i in range(nqb):
            row = [int(x) for x in rng.integers(-2, i + 1, size=kmax)]  # causal: blocks 0..i visible
            messy[0, h, i] = row
            mcnt[0, h, i] = kmax + 3 if i % 2 else kmax  # odd rows: a count past kmax (clamped)
            rec, top = [], -1
            for x in row:
                if x > top:
                    rec.append(x)
                    top = x
            clean[0, h, i, :len(rec)] = rec
            ccnt[0, h, i] = len(rec)
    assert (mcnt > 0).all() and (ccnt < kmax).any()
    t = lambda a: torch.from_numpy(a).cuda()
    case("attn given selection: messy list vs its clean records")
    o1, l1 = gpu.fp4_attention_fwd(qc, kc, vc, causal=True, fp16_budget_pct=pct, out_dtype=gpu.FP32,
                                   selection=(t(messy), t(mcnt)))
    o2, l2 = gpu.fp4_attention_fwd(qc, kc, vc, causal=True, fp16_budget_pct=pct, out_dtype=gpu.FP32,
                                   selection=(t(clean), t(ccnt)))
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    assert torch.isfinite(o1).all()


def test_binding_rejects_mismatched_out_buffer(gpu):
    """The C ABI takes a bare output pointer, so the binding refuses a given
    buffer whose dtype or size differs from what the kernel writes (it raises
    before anything is launched)."""
    q, k, v = synth.qkv(1, 1, 128, 64, seed=150)
    qc, kc, vc = q.cuda(), k.cuda(), v.cuda()
    case("binding: output buffer checks (nothing launched)")
    with pytest.raises(gpu.FP4Error):
        gpu.fp4_attention_fwd(qc, kc, vc, out_dtype=gpu.FP32, out=torch.empty_like(qc))  # bf16 buffer, fp32 output
    with pytest.raises(gpu.FP4Error):
        gpu.fp4_attention_fwd(qc, kc, vc, out_dtype=gpu.BF16, out=torch.empty(10, dtype=torch.bfloat16, device="cuda"))
    with pytest.raises(gpu.FP4Error):
        gpu.fp4_quantize(qc.view(-1, 64), 0, True, out=dict(codes=torch.empty(7, dtype=torch.uint8, device="cuda"),
                                                            scales=torch.empty(512, dtype=torch.uint8, device="cuda")))
