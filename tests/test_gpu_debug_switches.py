"""The debug switches on the GPU: FP4_SYNC_CHECK waits for each launch (and
would return a kernel-time error from the launching call), FP4_LOG reports
each launch; neither changes results."""
import pytest
import torch

from block_scaled_fp4_amd import synth
from gpu_helpers import case

pytestmark = pytest.mark.gpu


def test_sync_check_and_log_leave_results_unchanged(gpu, capfd, monkeypatch):
    x = synth.quant_tensor(rows=512).cuda()
    q, k, v = (t.cuda() for t in synth.qkv(1, 2, 256, 64, seed=140))
    case("debug switches: quantize + attention with FP4_SYNC_CHECK=1 FP4_LOG=1")
    ref_q = gpu.fp4_quantize(x, 0, True)
    ref_o, _ = gpu.fp4_attention_fwd(q, k, v, causal=True, out_dtype=gpu.FP32)
    torch.cuda.synchronize()
    monkeypatch.setenv("FP4_SYNC_CHECK", "1")
    monkeypatch.setenv("FP4_LOG", "1")
    got_q = gpu.fp4_quantize(x, 0, True)
    got_o, _ = gpu.fp4_attention_fwd(q, k, v, causal=True, out_dtype=gpu.FP32)
    monkeypatch.delenv("FP4_SYNC_CHECK")
    monkeypatch.delenv("FP4_LOG")
    torch.cuda.synchronize()
    assert torch.equal(got_q["codes"], ref_q["codes"]) and torch.equal(got_q["scales"], ref_q["scales"])
    assert torch.equal(got_o, ref_o)
    err = capfd.readouterr().err
    assert "[fp4] fp4_quantize launch: ok" in err and "[fp4] fp4_attention_fwd launch: ok" in err
