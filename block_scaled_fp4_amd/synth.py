"""Seeded synthetic inputs shaped like the pages' workloads.

Holds no quantization or attention arithmetic: only random draws, rounding to
the storage dtype and the outlier-channel pattern.  Both the GPU tests and the
oracle consume what these functions return.

Workloads (no dataset is used; these stand in for the long-context inputs the
pages measure on):
  tiny      B=1 H=1 S=256 d=64, fp16 N(0,1)                      seeds 0,1,2
  quant     bf16 [32768,128] N(0,1), 3 of 128 channels (2%) x20  seeds 4 (data), 3 (channels)
  prefill   B=1 H=32 S=8192 d=128, bf16 N(0,1); K: 4 channels per head x10
  select    as prefill with S=32768
  decode    batch 16, 32 q heads / 8 kv heads, context 131072, d=128, bf16;
            K with the prefill outlier pattern; sink 128 + recent 256 bf16 tokens
"""
from __future__ import annotations

import math

import torch


def _randn(shape, seed, device="cpu"):
    if device == "cpu" or str(device).startswith("cpu"):
        g = torch.Generator().manual_seed(seed)
        return torch.randn(*shape, generator=g, dtype=torch.float32)
    g = torch.Generator(device=device).manual_seed(seed)
    return torch.randn(*shape, generator=g, dtype=torch.float32, device=device)


def outlier_channels(n_channels: int, count: int, seed: int) -> torch.Tensor:
    g = torch.Generator().manual_seed(seed)
    return torch.randperm(n_channels, generator=g)[:count].sort().values


def qkv(B, H, S, d, dtype=torch.bfloat16, seed=0, Hkv=None, k_outliers=0, outlier_scale=10.0, Sk=None,
        device="cpu"):
    """q [B,H,S,d], k/v [B,Hkv,Sk,d] ~ N(0,1) rounded to dtype; K channels scaled per kv head."""
    Hkv = Hkv or H
    Sk = Sk or S
    q = _randn((B, H, S, d), seed, device)
    k = _randn((B, Hkv, Sk, d), seed + 1, device)
    v = _randn((B, Hkv, Sk, d), seed + 2, device)
    if k_outliers:
        for h in range(Hkv):
            ch = outlier_channels(d, k_outliers, 1000 + seed * 97 + h).to(k.device)
            k[:, h, :, ch] *= outlier_scale
    return q.to(dtype), k.to(dtype), v.to(dtype)


def tiny(device="cpu"):
    return qkv(1, 1, 256, 64, torch.float16, seed=0, device=device)


def quant_tensor(rows=32768, cols=128, frac=0.02, scale=20.0, device="cpu"):
    x = _randn((rows, cols), 4, device)
    n = math.ceil(frac * cols)
    ch = outlier_channels(cols, n, 3).to(x.device)
    x[:, ch] *= scale
    return x.to(torch.bfloat16)


def prefill(S=8192, H=32, d=128, device="cpu"):
    return qkv(1, H, S, d, torch.bfloat16, seed=0, k_outliers=4, device=device)


def decode_context(B=16, Hq=32, Hkv=8, L=131072, d=128, device="cpu", seed=10):
    """q [B,Hq,d], k/v [B,Hkv,L,d] bf16 (K with 4 outlier channels x10 per kv head)."""
    q = _randn((B, Hq, d), seed, device).to(torch.bfloat16)
    k = _randn((B, Hkv, L, d), seed + 1, device)
    for h in range(Hkv):
        ch = outlier_channels(d, 4, 2000 + h).to(k.device)
        k[:, h, :, ch] *= 10.0
    k = k.to(torch.bfloat16)
    v = _randn((B, Hkv, L, d), seed + 2, device).to(torch.bfloat16)
    return q, k, v
