"""Pins of the oracle's quantize-on-write cache append (the cache middle is
NVFP4 with ScaleSearch, its first and last blocks full precision: ScaleSearch
page, Metodologia / ScaleSearchAttention).

The append is pinned against an independent construction: a cache built in one
go from a longer context (the middle quantized by a single quantizer call over
all its tokens, the window sliced from the context) must equal, byte for byte,
the cache reached by appending the same tokens 16 or 32 at a time.  That holds
only if positions, block alignment (V blocks start at the first middle token)
and the window shift are all right."""
import numpy as np
import pytest

import oracle


def _bf16(a):
    """Round float32 values to bf16 (RNE), kept as float32."""
    u = np.ascontiguousarray(a, np.float32).view(np.uint32)
    r = ((u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000).astype(np.uint32)
    return r.view(np.float32)


def _context(B, H, L, d, seed):
    rng = np.random.default_rng(seed)
    k = _bf16(rng.standard_normal((B, H, L, d)).astype(np.float32))
    v = _bf16(rng.standard_normal((B, H, L, d)).astype(np.float32))
    k[:, :, :, 3] *= 10.0  # an outlier channel, as in the decode workload
    return k, _bf16(v)


def _direct_cache(k, v, n_sink, M, n_recent, cap):
    """Cache of a context whose middle holds M tokens, built in one go."""
    B, H, L, d = k.shape
    kc = np.zeros((B, H, cap, d // 2), np.uint8)
    ks = np.zeros((B, H, cap, d // 16), np.uint8)
    vc = np.zeros((B, H, cap // 2, d), np.uint8)
    vs = np.zeros((B, H, cap // 16, d), np.uint8)
    for b in range(B):
        for h in range(H):
            if M:
                rk = oracle.quantize(k[b, h, n_sink:n_sink + M], 0, True, -2, 6)
                rv = oracle.quantize(v[b, h, n_sink:n_sink + M], 1, True, -2, 6)
                kc[b, h, :M], ks[b, h, :M] = rk["codes"], rk["scales"]
                vc[b, h, :M // 2], vs[b, h, :M // 16] = rv["codes"], rv["scales"]
    kr = k[:, :, n_sink + M:n_sink + M + n_recent].copy()
    vr = v[:, :, n_sink + M:n_sink + M + n_recent].copy()
    return kr, vr, kc, ks, vc, vs, np.full(B, M, np.int32)


@pytest.mark.parametrize("n_recent,step", [(48, 16), (32, 32), (0, 16)])
def test_append_equals_cache_built_in_one_go(n_recent, step):
    B, H, d, n_sink, cap = 2, 2, 64, 16, 96
    M0, M1 = 16, 80
    L = n_sink + M1 + n_recent
    k, v = _context(B, H, L, d, seed=1)
    state = _direct_cache(k, v, n_sink, M0, n_recent, cap)
    pos = n_sink + M0 + n_recent  # next context token to append
    while pos < L:
        kr, vr, kc, ks, vc, vs, ml = state
        kn, vn = k[:, :, pos:pos + step], v[:, :, pos:pos + step]
        *state, over = oracle.kv_append(kr, vr, kc, ks, vc, vs, ml, kn, vn)
        assert not over.any()
        pos += step
    want = _direct_cache(k, v, n_sink, M1, n_recent, cap)
    for got, ref, name in zip(state, want, ["k_recent", "v_recent", "k_codes", "k_scales", "v_codes",
                                           "v_scales", "mid_len"]):
        np.testing.assert_array_equal(got, ref, err_msg=name)


def test_overflow_leaves_the_batch_unchanged():
    B, H, d, cap, n_recent = 2, 1, 64, 32, 16
    k, v = _context(B, H, 64, d, seed=2)
    kr, vr = k[:, :, :n_recent], v[:, :, :n_recent]
    kc = np.full((B, H, cap, d // 2), 7, np.uint8)
    ks = np.full((B, H, cap, d // 16), 9, np.uint8)
    vc = np.full((B, H, cap // 2, d), 5, np.uint8)
    vs = np.full((B, H, cap // 16, d), 3, np.uint8)
    ml = np.array([32, 16], np.int32)  # batch 0 full, batch 1 has room for 16
    kn, vn = k[:, :, 16:32], v[:, :, 16:32]
    out = oracle.kv_append(kr, vr, kc, ks, vc, vs, ml, kn, vn)
    kr2, vr2, kc2, ks2, vc2, vs2, ml2, over = out
    assert list(over) == [1, 0]
    assert list(ml2) == [32, 32]
    np.testing.assert_array_equal(kr2[0], kr[0])
    np.testing.assert_array_equal(kc2[0], kc[0])
    np.testing.assert_array_equal(vs2[0], vs[0])
    # batch 1: the old window went to tokens 16..31, the new tokens are the window
    np.testing.assert_array_equal(kr2[1], kn[1])
    rk = oracle.quantize(kr[1, 0], 0, True, -2, 6)
    np.testing.assert_array_equal(kc2[1, 0, 16:32], rk["codes"])
    np.testing.assert_array_equal(kc2[1, 0, :16], kc[1, 0, :16])  # untouched before mid_len


def test_mid_len_is_normalized_like_the_decode_reads_it():
    B, H, d, cap = 1, 1, 64, 64
    k, v = _context(B, H, 48, d, seed=3)
    kc = np.zeros((B, H, cap, d // 2), np.uint8)
    ks = np.zeros((B, H, cap, d // 16), np.uint8)
    vc = np.zeros((B, H, cap // 2, d), np.uint8)
    vs = np.zeros((B, H, cap // 16, d), np.uint8)
    empty = np.zeros((B, H, 0, d), np.float32)
    for given, used in ((21, 16), (-5, 0), (1000, 64)):
        *_, ml, over = oracle.kv_append(empty, empty, kc, ks, vc, vs, np.array([given], np.int32),
                                        k[:, :, :16], v[:, :, :16])
        if used + 16 > cap:
            assert over[0] == 1 and ml[0] == given
        else:
            assert over[0] == 0 and ml[0] == used + 16


def test_appended_values_dequantize_close_to_the_tokens():
    """The middle region's dequantized values are the tokens up to NVFP4 error
    (a coarse sanity bound: at most half the largest grid step, 1/6 of the
    block maximum for the max-scaling candidate, which ScaleSearch never does
    worse than in squared error)."""
    B, H, d, cap = 1, 1, 128, 32
    k, v = _context(B, H, 32, d, seed=4)
    empty = np.zeros((B, H, 0, d), np.float32)
    kc = np.zeros((B, H, cap, d // 2), np.uint8)
    ks = np.zeros((B, H, cap, d // 16), np.uint8)
    vc = np.zeros((B, H, cap // 2, d), np.uint8)
    vs = np.zeros((B, H, cap // 16, d), np.uint8)
    _, _, kc2, ks2, vc2, vs2, ml, _ = oracle.kv_append(empty, empty, kc, ks, vc, vs, np.array([0], np.int32),
                                                      k[:, :, :32], v[:, :, :32])
    kh = oracle.dequantize(kc2[0, 0], ks2[0, 0], 32, d, 0)
    vh = oracle.dequantize(vc2[0, 0], vs2[0, 0], 32, d, 1)
    ek = np.sqrt(((kh - k[0, 0]) ** 2).sum()) / np.sqrt((k[0, 0] ** 2).sum())
    ev = np.sqrt(((vh - v[0, 0]) ** 2).sum()) / np.sqrt((v[0, 0] ** 2).sum())
    assert ek < 0.15 and ev < 0.15


def test_append_keeps_the_full_precision_copy_and_block_sums():
    """With the dual cache (ThriftAttention page, Significado), appends write
    the tokens unquantized beside the NVFP4 copy and extend the key-block sums;
    after any sequence of appends the sums equal the block sums of the copy
    computed in one go (orc_block_sums), block boundaries every 128 tokens from
    the first middle token."""
    B, H, d, n_sink, n_recent, cap = 2, 2, 64, 16, 32, 320
    M0, M1 = 112, 304  # start mid-block, end in a short last block
    L = n_sink + M1 + n_recent
    k, v = _context(B, H, L, d, seed=5)
    kr, vr, kc, ks, vc, vs, ml = _direct_cache(k, v, n_sink, M0, n_recent, cap)
    nbc = (cap + 127) // 128
    km = np.zeros((B, H, cap, d), np.float32)
    vm = np.zeros((B, H, cap, d), np.float32)
    ksum = np.full((B, H, nbc, d), np.nan)  # blocks never written must not be read
    km[:, :, :M0] = k[:, :, n_sink:n_sink + M0]
    vm[:, :, :M0] = v[:, :, n_sink:n_sink + M0]
    for b in range(B):
        for h in range(H):
            ksum[b, h, :1] = oracle.block_sums(km[b, h, :M0])[:1]  # block 0 holds 112 tokens
    state = (kr, vr, kc, ks, vc, vs, ml)
    dual = (km, vm, ksum)
    pos, step = n_sink + M0 + n_recent, 16
    while pos < L:
        kn, vn = k[:, :, pos:pos + step], v[:, :, pos:pos + step]
        out = oracle.kv_append(*state, kn, vn, *dual)
        assert not out[7].any()
        state, dual = out[:7], out[8:]
        pos += step
        step = 48 if step == 16 else 16
    km, vm, ksum = dual
    np.testing.assert_array_equal(km[:, :, :M1], k[:, :, n_sink:n_sink + M1])
    np.testing.assert_array_equal(vm[:, :, :M1], v[:, :, n_sink:n_sink + M1])
    for b in range(B):
        for h in range(H):
            np.testing.assert_array_equal(ksum[b, h, :3], oracle.block_sums(k[b, h, n_sink:n_sink + M1]))
    want = _direct_cache(k, v, n_sink, M1, n_recent, cap)
    for got, ref in zip(state, want):
        np.testing.assert_array_equal(got, ref)
