"""A closed form for the FP4/FP16 mix of the attention forward at a partial
FP16 budget (ThriftAttention page, Metodologia / 1: blocks ranked by the dot
product of their mean query and mean key, top-k pairs kept; Metodologia / 2:
selected pairs on the FP16 path, the rest on the FP4 path, one online softmax).

Construction.  A direction u of +-1 entries; query rows q_i = beta_i u and key
rows k_j = a_g u with one value a_g per group of 64 consecutive keys.  Every
beta and a is a small dyadic number whose 16-element blocks NVFP4 holds
exactly (checked by the caller through the quantizer), so Q^ = Q, K^ = K,
fp16(Q) = Q and fp16(K) = K.  Then:
  - the score of (i, j) is beta_i a_g d exactly, on either path, and it is the
    same for every key of a 64-key group; a key tile of 64 or 128 keys holds
    one or two groups, so inside a tile every e = 2^(x - tm) is 1 on the keys
    of the group holding the maximum.  To keep every key at e = 1, the two
    groups of a 128-key tile get the same a whenever kv_tile is 128;
  - with e = 1 the two-level P gives P' = 2688, s2 = E4M3(448) = 448, code 6,
    so P^ / 2688 = 1 exactly; the FP16 path's fp16(e) is 1 as well.  P
    quantization loses nothing, and the forward reduces to plain softmax
    attention with weights 2^(x_j) over the values w_j = fp16(V_j) when the
    block of key j is selected for the query's block and w_j = V^_j (the
    dequantized NVFP4 V) when it is not;
  - the block means are mean(beta) u and mean(a) u, so the ranking of key
    blocks is the ranking of mean(a) over each block's groups (mean(beta) > 0),
    ties to the lower block, and the count is ceil(pct n / 100).
The expected output therefore depends on the promotion map only through which
keys carry fp16(V) and which V^: a mistake in that map (tile index taken for
block index, a shifted block) or in the units with which FP4 and FP16 tiles
meet in one row moves it by far more than rounding.
"""
import math

import numpy as np
import torch

import oracle

# dyadic values whose all-equal (up to sign) 16-element blocks NVFP4 holds exactly
A_VALUES = (0.0, 0.25, -0.25, 0.5, -0.5, 0.75, -0.75, 1.0, -1.0, 1.5, -1.5, 0.375, -0.375)
BETA_VALUES = (0.5, 1.0, 2.0, 1.5)


def construct(H, S, d, kv_tile, seed, zero_keys=False):
    """q [1,H,S,d], k, v [1,H,S,d] bf16 and the per-group key values a [H, groups]."""
    rng = np.random.default_rng(seed)
    u = rng.choice([-1.0, 1.0], size=d)
    ng = (S + 63) // 64
    a = np.zeros((H, ng))
    if not zero_keys:
        for h in range(H):
            a[h] = rng.choice(A_VALUES, size=ng)
            if kv_tile == 128:
                a[h, 1::2] = a[h, 0::2][: a[h, 1::2].size]
    beta = np.array([BETA_VALUES[(3 * i + seed) % len(BETA_VALUES)] for i in range(S)])
    q = np.broadcast_to(beta[None, :, None] * u[None, None, :], (H, S, d)).copy()
    k = np.zeros((H, S, d))
    for h in range(H):
        k[h] = a[h, np.arange(S) // 64][:, None] * u[None, :]
    g = torch.Generator().manual_seed(seed + 17)
    v = torch.randn(1, H, S, d, generator=g).to(torch.bfloat16)
    to = lambda x: torch.from_numpy(x[None]).to(torch.bfloat16)
    return to(q), to(k), v, a


def selection(a_h, S, causal, pct, sel_block):
    """Selected key blocks per query block, from the construction's key values
    (independent of any top-k code): ranking by mean(a) over the block's keys,
    ties to the lower block, count ceil(pct n / 100) in integers."""
    nb = (S + sel_block - 1) // sel_block
    groups = np.arange(S) // 64
    mean_a = [float(np.mean(a_h[groups[j * sel_block:(j + 1) * sel_block]])) for j in range(nb)]
    sel = []
    for i in range(nb):
        vis = list(range(i + 1)) if causal else list(range(nb))
        kcount = -(-pct * len(vis) // 100)
        ranked = sorted(vis, key=lambda j: (-mean_a[j], j))
        sel.append(sorted(ranked[:kcount]))
    return sel


def expected(q, k, v, a, causal, pct, sel_block, softmax_scale, kv_tile, block_of_key=None):
    """Closed-form output [H, S, d] and lse [H, S] (float64).  block_of_key maps
    a key index to the selection block whose promotion covers it; the default
    is the pages' j // sel_block (a test passes a wrong map to show the form
    tells it apart)."""
    _, H, S, d = q.shape
    if block_of_key is None:
        block_of_key = lambda j: j // sel_block
    c = float(np.float32(math.log2(math.e) * softmax_scale))
    out = np.zeros((H, S, d))
    lse = np.zeros((H, S))
    qf = q[0].float().numpy().astype(np.float64)
    kf = k[0].float().numpy().astype(np.float64)
    for h in range(H):
        vb = v[0, h]
        r = oracle.quantize(vb, 1, True)
        vhat = oracle.dequantize(r["codes"], r["scales"], S, d, 1).astype(np.float64)
        v16 = vb.to(torch.float16).double().numpy()
        sel = selection(a[h], S, causal, pct, sel_block) if pct > 0 else None
        s = qf[h] @ kf[h].T  # exact: dyadic products, d terms
        x = (s.astype(np.float32) * np.float32(c)).astype(np.float64)
        for i in range(S):
            n = i + 1 if causal else S
            xi = x[i, :n]
            m = xi.max()
            p = np.exp2(xi - m)
            if sel is not None:
                chosen = set(sel[i // sel_block])
                prom = np.array([block_of_key(j) in chosen for j in range(n)])
            else:
                prom = np.zeros(n, bool)
            w = np.where(prom[:, None], v16[:n], vhat[:n])
            out[h, i] = (p[:, None] * w).sum(0) / p.sum()
            lse[h, i] = (m + math.log2(p.sum())) * math.log(2.0)
    return out, lse


def operands_exact(q, k):
    """The construction's precondition: NVFP4 with ScaleSearch holds Q and K
    exactly (and fp16 does too)."""
    for t in (q, k):
        x = t[0].reshape(-1, t.shape[-1])
        r = oracle.quantize(x, 0, True)
        back = oracle.dequantize(r["codes"], r["scales"], x.shape[0], x.shape[1], 0)
        if not np.array_equal(back, x.float().numpy()):
            return False
        if not torch.equal(x.to(torch.float16).float(), x.float()):
            return False
    return True
