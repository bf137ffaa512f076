"""GPU block selection parity: top-k indices and counts bit-exact to the oracle
(ThriftAttention page, Metodologia / 1)."""
import numpy as np
import pytest
import torch

import oracle
from block_scaled_fp4_amd import synth
from gpu_helpers import case

pytestmark = pytest.mark.gpu


def _oracle_topk(q, k, causal, pct, sel_block):
    B, H, Sq, d = q.shape
    Hkv = k.shape[1]
    out_i, out_c = [], []
    for b in range(B):
        for h in range(H):
            qm = oracle.block_means(q[b, h], sel_block)
            km = oracle.block_means(k[b, h // (H // Hkv)], sel_block)
            i, c = oracle.block_topk(qm, km, causal, pct)
            out_i.append(i)
            out_c.append(c)
    nqb = out_i[0].shape[0]
    return np.stack(out_i).reshape(B, H, nqb, -1), np.stack(out_c).reshape(B, H, nqb)


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("pct", [5, 10, 50, 100])
def test_small_bit_exact(gpu, causal, pct):
    # ragged last block: 1008 = 7 * 128 + 112, 1040 = 8 * 128 + 16
    q, k, _ = synth.qkv(2, 4, 1008 if not causal else 1040, 64, Hkv=2, seed=3, k_outliers=2)
    case(f"topk small causal={causal} pct={pct}")
    idx, cnt = gpu.fp4_block_topk(q.cuda(), k.cuda(), causal, pct, 128)
    torch.cuda.synchronize()
    ri, rc = _oracle_topk(q, k, causal, pct, 128)
    np.testing.assert_array_equal(cnt.cpu().numpy(), rc)
    np.testing.assert_array_equal(idx.cpu().numpy(), ri)


def test_selective_workload_full_size(gpu):
    """B=1, H=32, S=32768, d=128, 128-token blocks, top 10% per query block."""
    q, k, _ = synth.prefill(S=32768)
    case("topk full 32K")
    idx, cnt = gpu.fp4_block_topk(q.cuda(), k.cuda(), True, 10, 128)
    torch.cuda.synchronize()
    ri, rc = _oracle_topk(q, k, True, 10, 128)
    np.testing.assert_array_equal(cnt.cpu().numpy(), rc)
    np.testing.assert_array_equal(idx.cpu().numpy(), ri)
    assert int(rc.sum()) == 32 * 3406  # sum over query blocks of ceil(10 * (i+1) / 100)


@pytest.mark.parametrize("dtype,d,sel_block,causal,hadamard,balance", [
    (torch.bfloat16, 128, 128, True, False, False),
    (torch.float16, 64, 256, False, False, False),
    (torch.bfloat16, 128, 256, True, True, False),
    (torch.float16, 128, 128, False, False, True),
])
def test_forward_selection_bit_exact(gpu, dtype, d, sel_block, causal, hadamard, balance):
    """The selection the forward computes itself (its Q and K quantization
    launches also write the block means, from the input before any rotation or
    balance) equals the oracle's: ragged last blocks, GQA, selection blocks of
    one and of two 128-row chunks."""
    S = 1040 if causal else 1008
    q, k, v = synth.qkv(2, 4, S, d, dtype, seed=5, Hkv=2, k_outliers=2)
    case(f"forward selection {dtype} d={d} sel_block={sel_block} causal={causal} had={hadamard} bal={balance}")
    _, _, idx, cnt = gpu.fp4_attention_fwd(q.cuda(), k.cuda(), v.cuda(), causal=causal, fp16_budget_pct=10,
                                           sel_block=sel_block, return_topk=True, hadamard=hadamard,
                                           balance=balance)
    torch.cuda.synchronize()
    ri, rc = _oracle_topk(q, k, causal, 10, sel_block)
    np.testing.assert_array_equal(cnt.cpu().numpy(), rc)
    np.testing.assert_array_equal(idx.cpu().numpy(), ri)


def test_forward_selection_full_size(gpu):
    """The 32K selective workload: the selection inside fp4_attention_fwd equals
    the oracle's, bit for bit."""
    q, k, v = synth.prefill(S=32768)
    case("forward selection full 32K")
    _, _, idx, cnt = gpu.fp4_attention_fwd(q.cuda(), k.cuda(), v.cuda(), causal=True, fp16_budget_pct=10,
                                           return_topk=True, return_lse=False)
    torch.cuda.synchronize()
    ri, rc = _oracle_topk(q, k, True, 10, 128)
    np.testing.assert_array_equal(cnt.cpu().numpy(), rc)
    np.testing.assert_array_equal(idx.cpu().numpy(), ri)
