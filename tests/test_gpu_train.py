"""GPU parity of the training forward (O') and backward (Attn-QAT page,
Metodologia / A and B) against the training oracle.  Forward outputs use the
attention tolerance; gradients, whose scale grows with the sequence, are
compared with the same bounds relative to the largest reference gradient
(max-abs 2e-3 * max|ref|, relative L2 1e-3)."""
import numpy as np
import pytest
import torch

import oracle
from block_scaled_fp4_amd import synth
from gpu_helpers import TIE_SLACK, assert_close_attn, assert_close_attn_rows, case

pytestmark = pytest.mark.gpu


def _close_grad(got, ref, what):
    got, ref = np.asarray(got, np.float64), np.asarray(ref, np.float64)
    scale = np.abs(ref).max()
    err = np.abs(got - ref).max()
    rel = np.linalg.norm(got - ref) / np.linalg.norm(ref)
    assert np.all(np.isfinite(got)), what
    assert err <= 2e-3 * scale and rel <= 1e-3, f"{what}: max-abs {err:.3e} (scale {scale:.3e}) rel-L2 {rel:.3e}"


@pytest.mark.parametrize("S,d,H,Hkv,causal,kv_tile,single,dt", [
    (256, 64, 2, 2, True, 128, False, torch.bfloat16),
    (208, 128, 4, 2, False, 64, False, torch.bfloat16),   # ragged length, GQA
    (192, 128, 2, 1, True, 64, True, torch.float16),      # single-level P, fp16 inputs
    (1040, 128, 2, 2, True, 128, False, torch.bfloat16),  # several 128-tiles of every product, ragged tail
    (336, 64, 4, 1, False, 128, False, torch.float16),    # fp16 dO split in both GEMMs that read it, G = 4
])
def test_train_step(gpu, S, d, H, Hkv, causal, kv_tile, single, dt):
    q, k, v = synth.qkv(1, H, S, d, dt, seed=120 + S, Hkv=Hkv, k_outliers=2)
    g = torch.Generator().manual_seed(7)
    do = torch.randn(1, H, S, d, generator=g).to(dt)
    case(f"train step S={S} d={d} H={H}/{Hkv} causal={causal} tile={kv_tile} single={single}")
    out, out_hp, lse = gpu.fp4_attention_fwd_train(q.cuda(), k.cuda(), v.cuda(), causal=causal, kv_tile=kv_tile,
                                                   single_level_p=single)
    dq, dk, dv = gpu.fp4_attention_bwd(q.cuda(), k.cuda(), v.cuda(), out_hp, lse, do.cuda(), causal=causal,
                                       kv_tile=kv_tile, single_level_p=single)
    ref_out, _ = gpu.fp4_attention_fwd(q.cuda(), k.cuda(), v.cuda(), causal=causal, kv_tile=kv_tile,
                                       out_dtype=gpu.FP32, single_level_p=single)
    torch.cuda.synchronize()
    assert torch.equal(out, ref_out)  # the training forward's output is the inference output
    r = oracle.attention_train(q, k, v, do, causal=causal, kv_tile=kv_tile, single_level_p=single)
    assert_close_attn(out.cpu().numpy().reshape(-1, d), r["out"].reshape(-1, d), "out")
    assert_close_attn(out_hp.cpu().numpy().reshape(-1, d), r["out_hp"].reshape(-1, d), "out_hp")
    np.testing.assert_allclose(lse.cpu().numpy().reshape(-1), r["lse"].reshape(-1), atol=1e-3)
    _close_grad(dv.cpu().numpy(), r["dv"], "dv")
    _close_grad(dq.cpu().numpy(), r["dq"], "dq")
    _close_grad(dk.cpu().numpy(), r["dk"], "dk")


def test_train_step_full_size(gpu):
    # the training workload as timed (B=1 H=32 S=4096 d=128 causal, bf16, two-level P,
    # kv_tile 128, one launch of each kernel over all heads); heads 0, 13 and 31 are
    # compared with the oracle, which runs one head at a time
    S, H, d = 4096, 32, 128
    q, k, v = synth.qkv(1, H, S, d, torch.bfloat16, seed=0, k_outliers=4)
    g = torch.Generator().manual_seed(5)
    do = torch.randn(1, H, S, d, generator=g).to(torch.bfloat16)
    case(f"train step full size S={S} d={d} H={H}")
    out, out_hp, lse = gpu.fp4_attention_fwd_train(q.cuda(), k.cuda(), v.cuda(), causal=True)
    dq, dk, dv = gpu.fp4_attention_bwd(q.cuda(), k.cuda(), v.cuda(), out_hp, lse, do.cuda(), causal=True)
    torch.cuda.synchronize()
    for h in (0, 13, 31):
        sl = slice(h, h + 1)
        r = oracle.attention_train(q[:, sl], k[:, sl], v[:, sl], do[:, sl], causal=True, kv_tile=128)
        # the FP4 output against the forward oracle's rows with their rounding-ambiguity bounds
        # (peaked rows whose P codes sit on a rounding boundary, from the outlier channels)
        ref, _, amb = oracle.attention_fwd(q[:, sl], k[:, sl], v[:, sl], causal=True, kv_tile=128,
                                           tie_slack=TIE_SLACK)
        assert_close_attn_rows(out[:, sl].cpu().numpy().reshape(-1, d), ref.reshape(-1, d), amb.reshape(-1),
                               f"out head {h}")
        assert_close_attn(out_hp[:, sl].cpu().numpy().reshape(-1, d), r["out_hp"].reshape(-1, d), f"out_hp head {h}")
        np.testing.assert_allclose(lse[:, sl].cpu().numpy().reshape(-1), r["lse"].reshape(-1), atol=1e-3)
        _close_grad(dv[:, sl].cpu().numpy(), r["dv"], f"dv head {h}")
        _close_grad(dq[:, sl].cpu().numpy(), r["dq"], f"dq head {h}")
        _close_grad(dk[:, sl].cpu().numpy(), r["dk"], f"dk head {h}")
