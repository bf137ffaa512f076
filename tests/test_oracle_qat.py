"""Pins of the training oracle (Attn-QAT page, Metodologia / A: P recomputed
in FP4 in the backward, a high-precision output O' for the softmax gradient's
row term; / B: fake-quantized forward).

The explicit gradient formulas of oracle.attention_train are checked against
torch autograd (float64) on the same fake-quantized graph, built
independently: quantized operands and the FP4 probabilities enter through
straight-through estimators (x + (xq - x).detach()), the softmax is torch's."""
import math

import numpy as np
import pytest
import torch

import oracle


def _rand(shape, seed):
    g = torch.Generator().manual_seed(seed)
    return torch.randn(*shape, generator=g).to(torch.bfloat16)


def _fq(x, axis):
    r = oracle.quantize(x, axis, True, -2, 6)
    return oracle.dequantize(r["codes"], r["scales"], x.shape[0], x.shape[1], axis)


def _autograd(q, k, v, do, causal, single_level, kv_tile):
    """Gradients of sum(O * dO) through the straight-through fake-quant graph."""
    B, H, Sq, d = q.shape
    Hkv, Sk = k.shape[1], k.shape[2]
    G = H // Hkv
    _, _, _, Ph = oracle.attention_fwd(q, k, v, causal=causal, kv_tile=kv_tile, single_level_p=single_level,
                                       with_probs=True)
    Ph = torch.tensor(Ph.reshape(B, H, Sq, Sk))
    s = float(oracle.score_factor(0.0, d)) * math.log(2.0)
    qt = torch.tensor(q.float().numpy(), dtype=torch.float64, requires_grad=True)
    kt = torch.tensor(k.float().numpy(), dtype=torch.float64, requires_grad=True)
    vt = torch.tensor(v.float().numpy(), dtype=torch.float64, requires_grad=True)
    qh = torch.tensor(np.stack([[_fq(q[b, h].float().numpy(), 0) for h in range(H)] for b in range(B)]))
    kh = torch.tensor(np.stack([[_fq(k[b, h].float().numpy(), 0) for h in range(Hkv)] for b in range(B)]))
    vh = torch.tensor(np.stack([[_fq(v[b, h].float().numpy(), 1) for h in range(Hkv)] for b in range(B)]))
    Qs = qt + (qh - qt).detach()
    Ks = (kt + (kh - kt).detach()).repeat_interleave(G, dim=1)
    Vs = (vt + (vh - vt).detach()).repeat_interleave(G, dim=1)
    S = torch.matmul(Qs, Ks.transpose(-1, -2).contiguous()) * s
    if causal:
        S = S.masked_fill(torch.ones(Sq, Sk, dtype=torch.bool).triu(1), float("-inf"))
    P = torch.softmax(S, dim=-1)
    Pst = P + (Ph - P).detach()
    O = torch.matmul(Pst, Vs)
    (O * torch.tensor(do.float().numpy(), dtype=torch.float64)).sum().backward()
    return qt.grad.numpy(), kt.grad.numpy(), vt.grad.numpy(), O.detach().numpy()


@pytest.mark.parametrize("causal,single,H,Hkv,kv_tile", [(True, False, 2, 1, 128), (False, True, 2, 2, 64),
                                                         (True, True, 4, 2, 64)])
def test_gradients_match_autograd(causal, single, H, Hkv, kv_tile):
    B, S, d = 1, 192, 64
    q, k, v, do = _rand((B, H, S, d), 1), _rand((B, Hkv, S, d), 2), _rand((B, Hkv, S, d), 3), _rand((B, H, S, d), 4)
    r = oracle.attention_train(q, k, v, do, causal=causal, kv_tile=kv_tile, single_level_p=single)
    gq, gk, gv, O = _autograd(q, k, v, do, causal, single, kv_tile)
    np.testing.assert_allclose(r["out"], O, atol=2e-6)   # the emitted weights reproduce the forward
    for got, ref, name in ((r["dq"], gq, "dq"), (r["dk"], gk, "dk"), (r["dv"], gv, "dv")):
        np.testing.assert_allclose(got, ref, rtol=0, atol=1e-5 * np.abs(ref).max(), err_msg=name)


def test_probabilities_and_the_row_term():
    B, H, S, d = 1, 2, 160, 64
    q, k, v, do = _rand((B, H, S, d), 5), _rand((B, H, S, d), 6), _rand((B, H, S, d), 7), _rand((B, H, S, d), 8)
    _, _, P, Ph = oracle.attention_fwd(q, k, v, causal=True, kv_tile=64, with_probs=True)
    P = P.reshape(B, H, S, S)
    np.testing.assert_allclose(P.sum(-1), 1.0, atol=1e-12)
    assert (np.triu(P[0, 0], 1) == 0).all() and (np.triu(Ph.reshape(B, H, S, S)[0, 0], 1) == 0).all()
    r = oracle.attention_train(q, k, v, do, causal=True, kv_tile=64)
    vh = _fq(v[0, 0].float().numpy(), 1)
    dP = do[0, 0].double().numpy() @ vh.T
    np.testing.assert_allclose((do[0, 0].double().numpy() * r["out_hp"][0, 0]).sum(-1), (P[0, 0] * dP).sum(-1),
                               atol=1e-10)
    # the first query sees one key: P = 1 there, so its score gradient and dQ vanish
    assert np.abs(r["dq"][:, :, 0]).max() < 1e-12
