"""Shared helpers of the GPU parity tests (comparison rules, case logging and
building a decode cache with the library's quantizer)."""
import sys

import numpy as np
import torch

# Attention outputs vs the oracle's identical fake-quant numerics: max-abs 2e-3
# and relative L2 1e-3 over the compared elements, on binary32 outputs.
ATOL = 2e-3
REL_L2 = 1e-3


def case(msg: str):
    """Name the case on stdout before a GPU step, so a fault is attributable."""
    print(f"[gpu case] {msg}", flush=True)
    sys.stdout.flush()


def assert_close_attn(got, ref, what="attention"):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    err = np.abs(got - ref)
    rel = np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-30)
    assert err.max() <= ATOL and rel <= REL_L2, f"{what}: max-abs {err.max():.3e} rel-L2 {rel:.3e}"
    return err.max(), rel


# Relative slack for the open P decisions of the attention forward (the
# oracle's tie_slack, see attn_row in oracle/fp4_oracle.c).  The kernel forms
# the quantization input t = 2^(fma(S, c, lg - tm)) with one hardware exp2;
# the oracle forms fl32(RN(2^fl32(fl32(S c) - tm)) * fl32(2688 / s2)).  A
# binary32 rounding of an exponent-domain value y moves t by at most
# ln 2 * 2^-24 * |y| (relative); the values rounded are tm, lg (and lg - tm),
# x twice (the score's fp32 accumulation and its product with c) and z, so
# with |x| <= |tm| + |z| the exponent terms stay below 4 (|tm| + |lg| + |z|)
# 2^-24 = b (|tm| + |lg| + |z|).  The exp2 instruction (within one ulp of the
# correctly rounded value over the probed range; two allowed) and the three
# products' roundings stay below a = 2^-20.
TIE_SLACK = (2.0 ** -20, 2.0 ** -22)


def assert_close_attn_rows(got, ref, amb, what="attention"):
    """Row-wise: max-abs over d <= ATOL + the row's rounding-ambiguity bound
    amb (the oracle's: how far open P decisions can move that row); relative
    L2 <= REL_L2 over everything.  Returns the number of rows whose error
    exceeded ATOL alone (each one explained by an open decision)."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    amb = np.asarray(amb, np.float64)
    assert got.shape == ref.shape and got.shape[:-1] == amb.shape, (got.shape, ref.shape, amb.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    err = np.abs(got - ref).max(-1)
    rel = np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-30)
    bad = err > ATOL + amb
    assert not bad.any(), (f"{what}: {int(bad.sum())} rows beyond 2e-3 + ambiguity, worst err "
                           f"{err[bad].max():.3e} (bound {(ATOL + amb)[bad][np.argmax(err[bad])]:.3e})")
    assert rel <= REL_L2, f"{what}: rel-L2 {rel:.3e}"
    n_open = int((err > ATOL).sum())
    if n_open:
        print(f"[parity] {what}: {n_open} of {err.size} rows beyond 2e-3, each within its ambiguity bound",
              flush=True)
    return n_open


def build_cache(fp4, k, v, ctx, n_sink, n_recent, mid_cap, dual=False):
    """Fill the cache buffers on the GPU from the full bf16 context k, v
    [B,Hkv,L,d] (the middle through fp4_quantize).  With dual, the
    full-precision copy of the middle and its block sums (fp4_kv_block_sums)
    are built too."""
    B, Hkv, Lcap, d = k.shape
    dev = k.device
    kc = torch.zeros((B, Hkv, mid_cap, d // 2), dtype=torch.uint8, device=dev)
    ks = torch.zeros((B, Hkv, mid_cap, d // 16), dtype=torch.uint8, device=dev)
    vc = torch.zeros((B, Hkv, mid_cap // 2, d), dtype=torch.uint8, device=dev)
    vs = torch.zeros((B, Hkv, mid_cap // 16, d), dtype=torch.uint8, device=dev)
    k_sink = k[:, :, :n_sink].contiguous()
    v_sink = v[:, :, :n_sink].contiguous()
    k_rec = torch.zeros((B, Hkv, n_recent, d), dtype=k.dtype, device=dev)
    v_rec = torch.zeros((B, Hkv, n_recent, d), dtype=k.dtype, device=dev)
    k_mid = v_mid = k_sum = None
    if dual:
        k_mid = torch.zeros((B, Hkv, mid_cap, d), dtype=k.dtype, device=dev)
        v_mid = torch.zeros((B, Hkv, mid_cap, d), dtype=k.dtype, device=dev)
        k_sum = torch.full((B, Hkv, (mid_cap + 127) // 128, d), float("nan"), dtype=torch.float64, device=dev)
    mids = []
    for b in range(B):
        L = int(ctx[b])
        M = L - n_sink - n_recent
        assert M >= 0 and M % 16 == 0 and M <= mid_cap
        mids.append(M)
        k_rec[b] = k[b, :, L - n_recent:L]
        v_rec[b] = v[b, :, L - n_recent:L]
        if M:
            km = k[b, :, n_sink:n_sink + M].contiguous().view(Hkv * M, d)
            vm = v[b, :, n_sink:n_sink + M].contiguous().view(Hkv * M, d)
            rk = fp4.fp4_quantize(km, 0, True)
            rv = fp4.fp4_quantize(vm, 1, True)
            kc[b, :, :M] = rk["codes"].view(Hkv, M, d // 2)
            ks[b, :, :M] = rk["scales"].view(Hkv, M, d // 16)
            vc[b, :, :M // 2] = rv["codes"].view(Hkv, M // 2, d)
            vs[b, :, :M // 16] = rv["scales"].view(Hkv, M // 16, d)
            if dual:
                k_mid[b, :, :M] = k[b, :, n_sink:n_sink + M]
                v_mid[b, :, :M] = v[b, :, n_sink:n_sink + M]
    mid_len = torch.tensor(mids, dtype=torch.int32, device=dev)
    cache = fp4.KVCache(k_sink, v_sink, kc, ks, vc, vs, k_rec, v_rec, mid_len, k_mid, v_mid, k_sum)
    if dual:
        fp4.fp4_kv_block_sums(cache)
    return cache
